"""Pins of the synthetic fidelity report (oracle/fidelity.py).

* Its method variant (int8 Q and K, q4_0 or q8_0 V) is the oracle's own
  decode_attention, to rounding.
* The V errors agree with the closed form of rounding to the format's step:
  a block scale d and codes rounded to nearest leave an error uniform on
  [-d/2, d/2], standard deviation d/sqrt(12).  For N(0, 1) values the q8_0
  step is max|x|/127 and the q4_0 step max|x|/8 over a 32-block, so the
  relative L2 error of the output (which averages errors and values alike)
  is E[d^2 / 12]^(1/2).
* Orderings any correct report shows: zero error for the exact variant,
  KL >= 0, fp16 Q.K closer than int8 Q.K, q8_0 V closer than q4_0 V.
"""
import numpy as np
import pytest

from oracle import fidelity as F
from oracle import kvq_oracle as O

L, D, G = 2048, 128, 4


def _inputs(seed=11):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, D), dtype=np.float32)
    k = rng.standard_normal((L, D), dtype=np.float32)
    v = rng.standard_normal((L, D), dtype=np.float32)
    return q, k, v


@pytest.mark.parametrize("fmt,name", [(O.V_Q4_0, "q4_0"), (O.V_Q8_0, "q8_0")])
def test_method_variant_is_decode_attention(fmt, name):
    q, k, v = _inputs()
    sc = D ** -0.5
    g = F.group_report(q, k, v, sc)
    kw, kd = O.encode_k(k)
    vp, vd = O.encode_v(v, fmt)
    ref = O.decode_attention(q[None, None].reshape(1, 1, G, D), kw[None, None], kd[None, None],
                             vp[None, None], vd[None, None], fmt, [L], sc, False)
    got = g["outs"][("int8", name)]
    np.testing.assert_allclose(got, ref[0, 0], rtol=1e-12, atol=1e-14)


def _expected_rel(v, steps):
    # d per 32-block from the block maximum, as the encoders fix it
    blocks = np.abs(v.reshape(-1, 32)).max(axis=1)
    d = blocks / steps
    return np.sqrt(np.mean(d * d) / 12.0)


def test_v_error_matches_rounding_closed_form():
    q, k, v = _inputs(12)
    r = F.workload_report(q[None], k[:, None], v[:, None], D ** -0.5)
    e8 = _expected_rel(v, 127.0)
    e4 = _expected_rel(v, 8.0)
    # the output averages the value errors like the values themselves; the
    # q4_0 tail (codes clamped at 15) adds a little
    assert 0.9 * e8 < r["rel_l2"][("exact", "q8_0")] < 1.1 * e8
    assert 0.88 * e4 < r["rel_l2"][("exact", "q4_0")] < 1.15 * e4


def test_report_orderings():
    q, k, v = _inputs(13)
    r = F.workload_report(q[None], k[:, None], v[:, None], D ** -0.5)
    assert r["rel_l2"][("exact", "exact")] == 0.0
    assert r["kl_mean"]["f16"] >= 0.0 and r["kl_mean"]["int8"] >= 0.0
    assert r["kl_mean"]["f16"] < r["kl_mean"]["int8"]
    assert r["rel_l2"][("f16", "exact")] < r["rel_l2"][("int8", "exact")]
    for qv in F.QK_VARIANTS:
        assert r["rel_l2"][(qv, "q8_0")] < r["rel_l2"][(qv, "q4_0")]


def test_kl_rows_definition():
    p = np.array([[0.5, 0.5, 0.0], [0.2, 0.3, 0.5]])
    r = np.array([[0.25, 0.75, 0.0], [0.2, 0.3, 0.5]])
    kl = F.kl_rows(p, r)
    assert kl[1] == 0.0
    assert abs(kl[0] - (0.5 * np.log(2.0) + 0.5 * np.log(0.5 / 0.75))) < 1e-15


def test_output_error_agrees_with_report_columns():
    """output_error of the oracle's own method output reproduces the
    report's int8 column (the same denominator, the same exact reference)."""
    q, k, v = _inputs(14)
    sc = D ** -0.5
    r = F.workload_report(q[None], k[:, None], v[:, None], sc)
    kw, kd = O.encode_k(k)
    for fmt, name in ((O.V_Q4_0, "q4_0"), (O.V_Q8_0, "q8_0")):
        vp, vd = O.encode_v(v, fmt)
        out = O.decode_attention(q[None, None], kw[None, None], kd[None, None], vp[None, None],
                                 vd[None, None], fmt, [L], sc, False)[0]
        e = F.output_error(q[None], k[:, None], v[:, None], sc, out)
        assert abs(e - r["rel_l2"][("int8", name)]) <= 1e-12 * max(1.0, e)
    assert F.output_error(q[None], k[:, None], v[:, None], sc,
                          F.group_report(q, k, v, sc)["outs"][("exact", "exact")][None]) == 0.0
