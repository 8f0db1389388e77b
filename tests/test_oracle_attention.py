"""Pins for the oracle's attention: a 50-digit mpmath brute force over the
whole decode step (dequantization re-derived here from the raw bytes), a
closed-form two-token case, and the softmax invariants (weights sum to one,
identical keys give the mean of V, one token gives that token's V, zero
scale gives the mean, a dominant key selects its V, causal rows equal a
truncated context, token order does not matter)."""
import math

import mpmath
import numpy as np
import pytest

from oracle import kvq_oracle as O

mpmath.mp.dps = 50


def _half_mp(bits: int):
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 0:
        return s * mpmath.mpf(f) * mpmath.mpf(2) ** -24
    return s * mpmath.mpf(1024 + f) * mpmath.mpf(2) ** (e - 25)


def _signed8(b: int) -> int:
    return b - 256 if b >= 128 else b


def _k_row_mp(words, dbits):
    """dequantized K row from raw words: byte k of word w is element 4w+k."""
    vals = []
    for w in words:
        for k in range(4):
            vals.append(_signed8((int(w) >> (8 * k)) & 0xFF))
    return [mpmath.mpf(v) * _half_mp(int(dbits[i // 32])) for i, v in enumerate(vals)]


def _v_row_mp(payload, dbits, fmt, D):
    out = [None] * D
    if fmt == O.V_Q4_0:
        for b in range(D // 32):
            d = _half_mp(int(dbits[b]))
            for j in range(16):
                byte = int(payload[16 * b + j])
                out[32 * b + j] = (mpmath.mpf(byte & 15) - 8) * d
                out[32 * b + j + 16] = (mpmath.mpf(byte >> 4) - 8) * d
    else:
        for i in range(D):
            out[i] = mpmath.mpf(_signed8(int(payload[i]))) * _half_mp(int(dbits[i // 32]))
    return out


def _q_row_mp(codes, d):
    return [mpmath.mpf(int(c)) * mpmath.mpf(float(d[i // 32])) for i, c in enumerate(codes)]


def _mp_attention(q_row, k_rows, v_rows, scale):
    s = [scale * mpmath.fsum(a * b for a, b in zip(q_row, kr)) for kr in k_rows]
    m = max(s)
    e = [mpmath.exp(x - m) for x in s]
    z = mpmath.fsum(e)
    D = len(v_rows[0])
    return [mpmath.fsum(e[t] * v_rows[t][c] for t in range(len(e))) / z for c in range(D)]


# Per-block magnitudes (factors of 10-100 between blocks) so that every
# element's dequantized value depends on its own block's scale: an oracle that
# paired an element with another block's scale would move the scores or the
# output far outside the tolerance.  Q's factors are the inverse of K's, which
# keeps every block's share of the score of order one.
_K_BLOCK_GAIN = {32: [2.0], 64: [0.1, 10.0], 128: [0.1, 2.0, 20.0, 0.5]}
_V_BLOCK_GAIN = {32: [1.0], 64: [10.0, 0.1], 128: [1.0, 0.05, 8.0, 0.3]}


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("fmt", [O.V_Q4_0, O.V_Q8_0])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_attention_mp_bruteforce(D, fmt, causal):
    """The whole decode step against a 50-digit evaluation written from the
    raw cache bytes: K words unpacked byte by byte, q4_0 bytes split into
    their two nibbles, every element times the binary16 scale of its own
    32-block (page 1: 32-element blocks with one fp16 scale each), Q codes
    times their fp32 block scale, then the softmax definition.  Four query
    heads share each kv head (grouped-query attention)."""
    rng = np.random.default_rng(10 + fmt + 2 * causal + D)
    S, Tq, Hq, Hkv, Lmax = 2, 2, 8, 2, 8
    seq_len = [8, 5]
    kg = np.repeat(np.asarray(_K_BLOCK_GAIN[D], np.float32), 32)
    vg = np.repeat(np.asarray(_V_BLOCK_GAIN[D], np.float32), 32)
    q = (rng.standard_normal((S, Tq, Hq, D)) / kg).astype(np.float32)
    k = (rng.standard_normal((S, Hkv, Lmax, D)) * kg).astype(np.float32)
    v = (rng.standard_normal((S, Hkv, Lmax, D)) * vg).astype(np.float32)
    kw, kd = O.encode_k(k)
    vp, vd = O.encode_v(v, fmt)
    if D > 32:
        # the blocks' scales really differ by an order of magnitude or more
        ks = O.half_value(kd[0, 0, 0]).astype(np.float64)
        assert ks.max() / ks.min() >= 10
    scale = 1 / math.sqrt(D)
    got = O.decode_attention(q, kw, kd, vp, vd, fmt, seq_len, scale, causal)
    qc, qd = O.quantize_q(q)
    G = Hq // Hkv
    for i in range(S):
        L = seq_len[i]
        for kvh in range(Hkv):
            k_rows = [_k_row_mp(kw[i, kvh, t], kd[i, kvh, t]) for t in range(L)]
            v_rows = [_v_row_mp(vp[i, kvh, t], vd[i, kvh, t], fmt, D) for t in range(L)]
            for j in range(Tq):
                n_vis = L - Tq + j + 1 if causal else L
                for h in range(kvh * G, (kvh + 1) * G):
                    want = _mp_attention(_q_row_mp(qc[i, j, h], qd[i, j, h]), k_rows[:n_vis],
                                         v_rows[:n_vis], mpmath.mpf(scale))
                    want = np.array([float(x) for x in want])
                    np.testing.assert_allclose(got[i, j, h], want, rtol=1e-12, atol=1e-13)


def test_closed_form_two_tokens():
    # q = 127 e0 (d = 1), k0 = 0, k1 = 127 e0 (d = 1): scores 0 and
    # 16129 * scale; with scale = ln 3 / 16129 the weights are 1/4 and 3/4.
    D = 32
    q = np.zeros((1, 1, 1, D), np.float32)
    q[..., 0] = 127
    k = np.zeros((1, 1, 2, D), np.float32)
    k[0, 0, 1, 0] = 127
    v = np.zeros((1, 1, 2, D), np.float32)
    v[0, 0, 0, 0] = 127
    v[0, 0, 1, 1] = -127
    kw, kd = O.encode_k(k)
    vp, vd = O.encode_v(v, O.V_Q8_0)
    out = O.decode_attention(q, kw, kd, vp, vd, O.V_Q8_0, [2], math.log(3) / 16129, False)
    want = np.zeros(D)
    want[0] = 127 / 4
    want[1] = -127 * 3 / 4
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=1e-13, atol=1e-12)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_weights_sum_to_one_and_nonnegative():
    rng = np.random.default_rng(20)
    L = 24
    qh, kh = _rand(rng, 3, 32), _rand(rng, L, 32) * 3
    eye = np.eye(L, 32)                 # V = one-hot rows: output = the weights
    w = O.softmax_attention(qh, kh, eye, 0.7, [L, L, 10])
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(w[2, 10:] == 0)


def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(21)
    kh = np.repeat(_rand(rng, 1, 64), 17, axis=0)
    vh = _rand(rng, 17, 64)
    out = O.softmax_attention(_rand(rng, 2, 64), kh, vh, 1.3, [17, 17])
    np.testing.assert_allclose(out, np.tile(vh.mean(axis=0), (2, 1)), rtol=1e-12, atol=1e-13)


def test_single_token_zero_scale_dominant_key():
    rng = np.random.default_rng(22)
    qh, kh, vh = _rand(rng, 1, 32), _rand(rng, 9, 32), _rand(rng, 9, 32)
    np.testing.assert_allclose(O.softmax_attention(qh, kh, vh, 0.5, [1])[0], vh[0], rtol=1e-14)
    np.testing.assert_allclose(O.softmax_attention(qh, kh, vh, 0.0, [9])[0], vh.mean(axis=0),
                               rtol=1e-12, atol=1e-13)
    kd = kh.copy()
    kd[4] = qh[0] * 100.0
    np.testing.assert_allclose(O.softmax_attention(qh, kd, vh, 1.0, [9])[0], vh[4], rtol=1e-12)


def test_causal_rows_equal_truncated_context_and_permutation():
    rng = np.random.default_rng(23)
    S, Tq, Hq, Hkv, D, L = 1, 4, 4, 1, 64, 40
    q = rng.standard_normal((S, Tq, Hq, D)).astype(np.float32)
    k = rng.standard_normal((S, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((S, Hkv, L, D)).astype(np.float32)
    kw, kd = O.encode_k(k)
    vp, vd = O.encode_v(v, O.V_Q4_0)
    causal = O.decode_attention(q, kw, kd, vp, vd, O.V_Q4_0, [L], 0.125, True)
    for j in range(Tq):
        n = L - Tq + j + 1
        one = O.decode_attention(q[:, j:j + 1], kw, kd, vp, vd, O.V_Q4_0, [n], 0.125, False)
        np.testing.assert_allclose(causal[:, j], one[:, 0], rtol=1e-12, atol=1e-14)
    perm = rng.permutation(L)
    flat = O.decode_attention(q, kw, kd, vp, vd, O.V_Q4_0, [L], 0.125, False)
    flat_p = O.decode_attention(q, kw[:, :, perm], kd[:, :, perm], vp[:, :, perm], vd[:, :, perm],
                                O.V_Q4_0, [L], 0.125, False)
    np.testing.assert_allclose(flat, flat_p, rtol=1e-11, atol=1e-14)


def test_gqa_groups_are_contiguous():
    # Hq = 8 over Hkv = 2: heads 0..3 read kv head 0 and 4..7 read kv head 1
    rng = np.random.default_rng(24)
    q = rng.standard_normal((1, 1, 8, 32)).astype(np.float32)
    k = rng.standard_normal((1, 2, 12, 32)).astype(np.float32)
    v = rng.standard_normal((1, 2, 12, 32)).astype(np.float32)
    kw, kd = O.encode_k(k)
    vp, vd = O.encode_v(v, O.V_Q8_0)
    out = O.decode_attention(q, kw, kd, vp, vd, O.V_Q8_0, [12], 0.3, False)
    for h in range(8):
        kvh = h // 4
        one = O.decode_attention(q[:, :, h:h + 1], kw[:, kvh:kvh + 1], kd[:, kvh:kvh + 1],
                                 vp[:, kvh:kvh + 1], vd[:, kvh:kvh + 1], O.V_Q8_0, [12], 0.3, False)
        np.testing.assert_array_equal(out[:, :, h], one[:, :, 0])


def test_visible_tokens():
    assert list(O.visible_tokens(10, 1, True)) == [10]
    assert list(O.visible_tokens(10, 4, True)) == [7, 8, 9, 10]
    assert list(O.visible_tokens(10, 4, False)) == [10, 10, 10, 10]


def test_f16k_reference_on_representable_inputs():
    """decode_attention_f16k rounds Q and K to binary16; on inputs that
    binary16 holds exactly the rounding is the identity, so the result is the
    (mpmath-pinned) softmax attention of the raw values.  K values are
    multiples of 1/64 in [-4, 4] and Q multiples of 1/256 in [-2, 2]."""
    rng = np.random.default_rng(41)
    S, Tq, Hq, Hkv, D, L = 1, 1, 4, 2, 128, 96
    q = (rng.integers(-512, 513, (S, Tq, Hq, D)) / 256.0).astype(np.float32)
    k = (rng.integers(-256, 257, (S, Hkv, L, D)) / 64.0).astype(np.float32)
    v = rng.standard_normal((S, Hkv, L, D)).astype(np.float32)
    k_bits = O.half_bits(k)
    assert np.array_equal(O.half_value(k_bits), k)
    vp, vd = O.encode_v(v, O.V_Q4_0)
    got = O.decode_attention_f16k(q, k_bits, vp, vd, O.V_Q4_0, [L], D ** -0.5, False)
    for h in range(Hq):
        kvh = h // (Hq // Hkv)
        want = O.softmax_attention(q[0, :, h].astype(np.float64), k[0, kvh].astype(np.float64),
                                   O.dequant_v(vp[0, kvh], vd[0, kvh], O.V_Q4_0), D ** -0.5, [L])
        np.testing.assert_array_equal(got[0, :, h], want)


def test_f16k_reference_rounds_inputs():
    """Away from representable values the reference sees the rounded inputs:
    it equals the exact attention of half_value(half_bits(x))."""
    rng = np.random.default_rng(42)
    q = rng.standard_normal((1, 1, 2, 128)).astype(np.float32)
    k = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    v = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    vp, vd = O.encode_v(v, O.V_Q8_0)
    got = O.decode_attention_f16k(q, O.half_bits(k), vp, vd, O.V_Q8_0, [64], 0.1, False)
    raw = O.decode_attention_f16k(O.half_value(O.half_bits(q)), O.half_bits(k), vp, vd, O.V_Q8_0,
                                  [64], 0.1, False)
    np.testing.assert_array_equal(got, raw)   # rounding twice changes nothing
    assert np.abs(O.half_value(O.half_bits(q)) - q).max() > 0
