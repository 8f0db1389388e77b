"""Pins for the oracle's block quantizers, storage encodings and integer dot
sums.  Expected values come from exact rational arithmetic, from worked
blocks derived by hand from the IEEE-754 definitions, from numpy's own byte
view, and from the 47% figure the first page prints."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import kvq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rne_fraction(q: Fraction) -> int:
    """nearest integer to an exact rational, ties to even."""
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def _fl32(x: float) -> float:
    # a float64 value rounded once to fp32
    return float(np.float32(x))


def _nearest_half(x32: float) -> int:
    """brute-force nearest binary16 (ties to even bits) of an fp32 value."""
    from tests.test_oracle_half import brute_nearest_half_bits
    return int(brute_nearest_half_bits(np.float32(x32)))


def _half_to_fraction(bits: int) -> Fraction:
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 0:
        return s * Fraction(f, 1 << 24)
    return s * Fraction(1024 + f, 1) * Fraction(2) ** (e - 25)


def _exact_codes(xblock, d: Fraction, lo: int, hi: int, offset: int):
    """codes the reading prescribes, computed independently of the oracle:
    the fp32 quotient is formed as the double quotient rounded once to fp32
    (innocuous double rounding for one fp32 division), then rounded to
    nearest-even and clamped.  Also returns, per element, whether the exact
    quotient is far enough from a tie that the exact arg-min must agree."""
    codes, far = [], []
    for x in xblock:
        if d == 0:
            codes.append(offset)
            far.append(True)
            continue
        qf = _fl32(float(x) / float(d))
        codes.append(int(np.clip(np.rint(np.float32(qf)) + offset, lo, hi)))
        exact = Fraction(float(x)) / d
        frac = exact - (exact.numerator // exact.denominator)
        far.append(abs(frac - Fraction(1, 2)) > abs(exact) * Fraction(1, 1 << 20))
    return codes, far


def _argmin_code(x: float, d: Fraction, lo: int, hi: int, offset: int) -> int:
    """arg-min over every code c in [lo, hi] of |x - d (c - offset)|,
    ties to the even (c - offset); brute force in exact arithmetic."""
    best, bestc = None, None
    xf = Fraction(float(x))
    for c in range(lo, hi + 1):
        err = abs(xf - d * (c - offset))
        if best is None or err < best or (err == best and (c - offset) % 2 == 0):
            best, bestc = err, c
    return bestc


def _random_blocks(rng, n, scale_range=(1e-3, 1e3)):
    scales = np.exp(rng.uniform(np.log(scale_range[0]), np.log(scale_range[1]), size=(n, 1)))
    return (rng.standard_normal((n, 32)) * scales).astype(np.float32)


# ---------------------------------------------------------------------------
# K / q8_0 quantizer
# ---------------------------------------------------------------------------

def test_quantize_k_matches_exact_argmin():
    rng = np.random.default_rng(1)
    x = _random_blocks(rng, 300)
    codes, dbits = O.quantize_k(x)
    for b in range(x.shape[0]):
        a = max(abs(float(v)) for v in x[b])
        assert int(dbits[b, 0]) == _nearest_half(_fl32(a / 127.0))
        d = _half_to_fraction(int(dbits[b, 0]))
        want, far = _exact_codes(x[b], d, -127, 127, 0)
        assert list(codes[b]) == want
        for i in range(32):
            if far[i]:
                assert int(codes[b, i]) == _argmin_code(x[b, i], d, -127, 127, 0)


def test_quantize_k_worked_blocks():
    # amax 127 -> fl32(127/127) = 1 -> fp16 0x3C00; codes are x rounded to
    # nearest with ties to even
    x = np.zeros(32, np.float32)
    x[:12] = [127, -127, 63.5, -63.5, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.25, 100.49]
    c, d = O.quantize_k(x)
    assert int(d[0]) == 0x3C00
    assert list(c[:12]) == [127, -127, 64, -64, 0, 2, 2, 0, -2, -2, 3, 100]
    assert not c[12:].any()
    w = O.pack_k(c)
    # little-endian bytes: 7F 81 40 C0 | 00 02 02 00 | FE FE 03 64
    assert [int(v) for v in w[:3]] == [0xC040817F, 0x00020200, 0x6403FEFE]
    assert not w[3:].any()

    # amax 1: fl32(1/127) has bits 0x3C010204; to fp16 that is
    # 2^-7 * (1 + 8/1024) = 129/16384 (bits 0x2008); codes are
    # x * 16384/129 rounded: 1 -> 127.0078 -> 127, 0.5 -> 63.504 -> 64,
    # 0.25 -> 31.752 -> 32
    x = np.zeros(32, np.float32)
    x[:5] = [1.0, -1.0, 0.5, 0.25, 0.0]
    c, d = O.quantize_k(x)
    assert int(d[0]) == 0x2008
    assert list(c[:5]) == [127, -127, 64, 32, 0]


def test_quantize_k_zero_and_tiny_blocks():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = 1e-30          # amax/127 underflows binary16 -> d = 0 -> codes 0
    c, d = O.quantize_k(x)
    assert not c.any()
    assert [int(v) for v in d.ravel()] == [0, 0, 0, 0]


def test_quantize_k_exact_ties_round_to_even():
    # d = 1 (amax 127): x = k + 1/2 is an exact tie
    x = np.zeros(32, np.float32)
    ks = np.arange(-10, 11)
    x[:21] = ks + 0.5
    x[31] = 127.0
    c, _ = O.quantize_k(x)
    want = [k if k % 2 == 0 else k + 1 for k in ks]
    assert list(c[:21]) == want


@settings(max_examples=300, deadline=None)
@given(st.lists(st.floats(min_value=-3e4, max_value=3e4, allow_nan=False, width=32),
                min_size=32, max_size=32))
def test_quantize_k_roundtrip_bound(vals):
    x = np.asarray(vals, np.float32)
    c, dbits = O.quantize_k(x)
    d = float(O.half_value(dbits)[0])
    a = float(np.max(np.abs(x)))
    if a / 127.0 < 2.0 ** -14:
        return      # scale in the binary16 subnormal range: bound not claimed
    err = np.abs(x.astype(np.float64) - c.astype(np.float64) * d)
    assert np.all(err <= d / 2 * (1 + 2.0 ** -20))


# ---------------------------------------------------------------------------
# q4_0 quantizer
# ---------------------------------------------------------------------------

def test_quantize_q4_0_matches_exact_argmin():
    rng = np.random.default_rng(2)
    x = _random_blocks(rng, 300)
    n, dbits = O.quantize_v_q4_0(x)
    for b in range(x.shape[0]):
        j = int(np.argmax(np.abs(x[b])))
        assert all(abs(x[b, i]) < abs(x[b, j]) for i in range(j))
        assert int(dbits[b, 0]) == _nearest_half(_fl32(float(x[b, j]) / -8.0))
        d = _half_to_fraction(int(dbits[b, 0]))
        want, far = _exact_codes(x[b], d, 0, 15, 8)
        assert list(n[b]) == want
        for i in range(32):
            if far[i]:
                assert int(n[b, i]) == _argmin_code(x[b, i], d, 0, 15, 8)


def test_quantize_q4_0_worked_blocks():
    # first element of largest magnitude is x0 = -8 (x5 = +8 ties it later),
    # so d = fp16(-8 / -8) = 1 (0x3C00); n = clamp(rne(x) + 8, 0, 15)
    x = np.zeros(32, np.float32)
    x[:8] = [-8, 7.5, 0.5, 1.5, -0.5, 8.0, 3.49, -7.5]
    x[16:20] = [2.0, -3.0, 6.6, -6.5]
    n, d = O.quantize_v_q4_0(x)
    assert int(d[0]) == 0x3C00
    assert list(n[:8]) == [0, 15, 8, 10, 8, 15, 11, 0]
    assert list(n[16:20]) == [10, 5, 15, 2]
    assert all(v == 8 for v in n[8:16]) and all(v == 8 for v in n[20:])
    p = O.pack_q4_0(n)
    assert [int(v) for v in p] == [0xA0, 0x5F, 0xF8, 0x2A, 0x88, 0x8F, 0x8B, 0x80] + [0x88] * 8
    np.testing.assert_array_equal(O.unpack_q4_0(p), n)
    v = O.dequant_v(p, d, O.V_Q4_0)
    assert list(v[:8]) == [-8, 7, 0, 2, 0, 7, 3, -8]

    # positive extreme: m = 4 -> d = fp16(4 / -8) = -0.5 (0xB800)
    x = np.zeros(32, np.float32)
    x[:3] = [0.0, 4.0, -2.0]
    n, d = O.quantize_v_q4_0(x)
    assert int(d[0]) == 0xB800
    assert list(n[:3]) == [8, 0, 12]
    assert [int(b) for b in O.pack_q4_0(n)[:3]] == [0x88, 0x80, 0x8C]


def test_quantize_q4_0_zero_block():
    n, d = O.quantize_v_q4_0(np.zeros(32, np.float32))
    assert all(v == 8 for v in n)
    assert float(O.half_value(d)[0]) == 0.0


@settings(max_examples=300, deadline=None)
@given(st.lists(st.floats(min_value=-3e4, max_value=3e4, allow_nan=False, width=32),
                min_size=32, max_size=32))
def test_quantize_q4_0_roundtrip_bound(vals):
    x = np.asarray(vals, np.float32)
    n, dbits = O.quantize_v_q4_0(x)
    d = abs(float(O.half_value(dbits)[0]))
    a = float(np.max(np.abs(x)))
    if a / 8.0 < 2.0 ** -14:
        return
    v = O.dequant_v(O.pack_q4_0(n), dbits, O.V_Q4_0)[0:32]
    err = np.abs(x.astype(np.float64) - v)
    tail = n == 15        # clamped top code: error up to |d|
    assert np.all(err[~tail] <= d / 2 * (1 + 2.0 ** -20))
    assert np.all(err[tail] <= d * (1 + 2.0 ** -10))


# ---------------------------------------------------------------------------
# Q quantizer (fp32 scale)
# ---------------------------------------------------------------------------

def test_quantize_q_fp32_scale_worked():
    # amax 1: d = fl32(1/127), bits 0x3C010204 (1/127 = 2^-7 * 1.0000001...b,
    # the bits after the 23rd are 0000 1... so it rounds down).  x0 = 0.99603
    # gives 126.4958 -> 126 with this scale, but 126.5035 -> 127 with the
    # fp16 scale the K quantizer uses.
    x = np.zeros(32, np.float32)
    x[:4] = [0.99603, 1.0, -0.5, 0.25]
    c, d = O.quantize_q(x)
    assert int(np.asarray(d, np.float32).view(np.uint32)[0]) == 0x3C010204
    assert list(c[:4]) == [126, 127, -64, 32]
    ck, _ = O.quantize_k(x)
    assert int(ck[0]) == 127


def test_quantize_q_matches_exact_codes():
    rng = np.random.default_rng(3)
    x = _random_blocks(rng, 200)
    codes, d = O.quantize_q(x)
    for b in range(x.shape[0]):
        a = max(abs(float(v)) for v in x[b])
        assert float(d[b, 0]) == _fl32(a / 127.0)
        want, far = _exact_codes(x[b], Fraction(float(d[b, 0])), -127, 127, 0)
        assert list(codes[b]) == want
        for i in range(32):
            if far[i]:
                assert int(codes[b, i]) == _argmin_code(x[b, i], Fraction(float(d[b, 0])), -127, 127, 0)


# ---------------------------------------------------------------------------
# packing and integer sums
# ---------------------------------------------------------------------------

def test_pack_k_is_little_endian_byte_view():
    rng = np.random.default_rng(4)
    c = rng.integers(-127, 128, size=(5, 128)).astype(np.int8)
    np.testing.assert_array_equal(O.pack_k(c), c.view("<u4"))
    np.testing.assert_array_equal(O.unpack_k(O.pack_k(c)), c)


def test_q8_0_payload_is_raw_int8_bytes():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    p, d = O.encode_v(x, O.V_Q8_0)
    c, d2 = O.quantize_k(x)
    np.testing.assert_array_equal(p.view(np.int8), c)
    np.testing.assert_array_equal(d, d2)


def test_block_isum_bruteforce_and_identity():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 64)).astype(np.float32)
    k = (rng.standard_normal((3, 64)) * 3).astype(np.float32)
    qc, qd = O.quantize_q(q)
    kc, kd = O.quantize_k(k)
    isum = O.block_isum(qc, kc)
    for r in range(3):
        for b in range(2):
            s = 0
            for i in range(32):
                s += int(qc[r, 32 * b + i]) * int(kc[r, 32 * b + i])
            assert int(isum[r, b]) == s
        # sum_b dq_b dk_b isum_b equals the dot of the dequantized vectors
        lhs = sum(Fraction(float(qd[r, b])) * _half_to_fraction(int(kd[r, b])) * int(isum[r, b])
                  for b in range(2))
        rhs = sum(Fraction(int(qc[r, i])) * Fraction(float(qd[r, i // 32]))
                  * Fraction(int(kc[r, i])) * _half_to_fraction(int(kd[r, i // 32]))
                  for i in range(64))
        assert lhs == rhs
    # worst case still fits int32: 32 * 127 * 127
    full = np.full((1, 32), 127, np.int8)
    assert int(O.block_isum(full, -full)[0, 0]) == -516128


def test_k_saving_matches_page_figure():
    g = json.load(open(os.path.join(GOLDEN, "k_saving.json")))
    for D in (64, 128):
        kb, _ = O.kv_bytes_per_token_head(D, O.V_Q4_0)
        saving = 1 - kb / (g["fp16_bytes_per_element"] * D)
        assert saving == 1 - 34 / 64
        assert round(100 * saving) == g["page_figure_percent"]
    assert O.kv_bytes_per_token_head(128, O.V_Q4_0) == (136, 72)
    assert O.kv_bytes_per_token_head(128, O.V_Q8_0) == (136, 136)
    assert O.kv_bytes_per_token_head(64, O.V_Q8_0) == (68, 68)


# ---------------------------------------------------------------------------
# dequantization of whole rows: every element takes its own block's scale
# ---------------------------------------------------------------------------

def _rows_with_block_gains(rng, n, gains):
    """n rows of len(gains) 32-blocks, block b drawn N(0, 1) times gains[b]."""
    g = np.repeat(np.asarray(gains, np.float64), 32)
    return (rng.standard_normal((n, g.size)) * g).astype(np.float32)


@pytest.mark.parametrize("gains", [[0.01, 1.0, 100.0, 0.1], [50.0, 0.02], [1.0, 1e-3, 1e3, 7.0]])
def test_dequant_rows_per_block_roundtrip(gains):
    """Page 1 fixes 32-element blocks with one fp16 scale each (the 47% of its
    title); per element, |x - deq(q(x))| <= d_b / 2 with d_b the scale of the
    element's own block (the q4_0 clamped top code: <= |d_b|).  Blocks whose
    scales differ by 10-10^6 make any mix-up of blocks fail the bound."""
    rng = np.random.default_rng(len(gains) * 7 + int(gains[0] * 100))
    x = _rows_with_block_gains(rng, 64, gains)
    x64 = x.astype(np.float64)
    nb = len(gains)

    def per_elem(d):   # [rows][nb] -> [rows][nb * 32]
        return np.repeat(np.abs(np.asarray(d, np.float64)), 32, axis=-1)

    kw, kd = O.encode_k(x)
    dk = per_elem(O.half_value(kd))
    assert np.all(np.abs(x64 - O.dequant_k(kw, kd)) <= dk / 2 * (1 + 2.0 ** -20))

    vp, vd = O.encode_v(x, O.V_Q8_0)
    assert np.all(np.abs(x64 - O.dequant_v(vp, vd, O.V_Q8_0)) <= per_elem(O.half_value(vd)) / 2 * (1 + 2.0 ** -20))

    n, d4 = O.quantize_v_q4_0(x)
    dv = per_elem(O.half_value(d4))
    err = np.abs(x64 - O.dequant_v(O.pack_q4_0(n), d4, O.V_Q4_0))
    tail = n == 15
    assert np.all(err[~tail] <= dv[~tail] / 2 * (1 + 2.0 ** -20))
    assert np.all(err[tail] <= dv[tail] * (1 + 2.0 ** -10))

    qc, qd = O.quantize_q(x)
    assert np.all(np.abs(x64 - O.dequant_q(qc, qd)) <= per_elem(qd) / 2 * (1 + 2.0 ** -20))
    # and the scales themselves follow the blocks' magnitudes
    ratio = O.half_value(kd).astype(np.float64).mean(axis=0)
    assert np.all(np.diff(np.log10(ratio)) != 0) and ratio.max() / ratio.min() >= 10 ** (nb > 1)
