"""Pins the oracle's fp32 -> binary16 rounding against a brute-force nearest
search over every finite binary16 value (IEEE-754 round to nearest, ties to
the even bit pattern, overflow to infinity past 65520)."""
import numpy as np
import pytest

from oracle import kvq_oracle as O


# all non-negative finite binary16 values, in increasing order of value and bits
_POS_BITS = np.arange(0x0000, 0x7C00, dtype=np.uint16)


def _half_exact(bits):
    """binary16 value computed from the bit fields (no library conversion)."""
    bits = np.asarray(bits, dtype=np.int64)
    sign = np.where(bits & 0x8000, -1.0, 1.0)
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    mag = np.where(e == 0, f * 2.0 ** -24, (1024 + f) * 2.0 ** (e.astype(np.float64) - 25))
    return sign * mag


_POS_VALS = _half_exact(_POS_BITS)
# one step past the largest finite value: 65536 (with even bits 0x7C00 = +inf)
_EXT_VALS = np.append(_POS_VALS, 65536.0)
_EXT_BITS = np.append(_POS_BITS, np.uint16(0x7C00))


def brute_nearest_half_bits(x32):
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    ax = np.abs(x)
    hi = np.searchsorted(_EXT_VALS, ax, side="left")
    hi = np.clip(hi, 1, len(_EXT_VALS) - 1)
    lo = hi - 1
    exact = _EXT_VALS[hi] == ax
    dlo = ax - _EXT_VALS[lo]
    dhi = _EXT_VALS[hi] - ax
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_EXT_BITS[hi] & 1) == 0))
    pick_hi |= exact
    b = np.where(pick_hi, _EXT_BITS[hi], _EXT_BITS[lo]).astype(np.uint16)
    b = np.where(ax >= 65536.0, np.uint16(0x7C00), b)
    neg = np.signbit(x)
    return np.where(neg, b | np.uint16(0x8000), b).astype(np.uint16)


def test_half_value_matches_bit_fields():
    allbits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = (allbits & 0x7C00) != 0x7C00
    got = O.half_value(allbits[finite]).astype(np.float64)
    np.testing.assert_array_equal(got, _half_exact(allbits[finite]))


def test_half_bits_textbook_values():
    # IEEE-754 binary16 encodings fixed by the standard
    cases = {1.0: 0x3C00, -2.0: 0xC000, 0.5: 0x3800, 65504.0: 0x7BFF,
             2.0 ** -14: 0x0400, 2.0 ** -24: 0x0001, 0.0: 0x0000,
             65520.0: 0x7C00, 1.0 + 2.0 ** -11: 0x3C00, 1.0 + 3 * 2.0 ** -11: 0x3C02}
    for x, bits in cases.items():
        assert int(O.half_bits(np.float32(x))) == bits, x
    assert int(O.half_bits(np.float32(-0.0))) == 0x8000


def test_half_bits_random_patterns_bruteforce():
    rng = np.random.default_rng(11)
    raw = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(O.half_bits(x), brute_nearest_half_bits(x))


def test_half_bits_ties_and_neighbours_bruteforce():
    # midpoints between consecutive binary16 values are exact in fp32; probe
    # them and the fp32 values one ulp either side, over the whole range
    mids = ((_EXT_VALS[:-1] + _EXT_VALS[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (_EXT_VALS[:-1] + _EXT_VALS[1:]) / 2)
    probes = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                             np.nextafter(mids, np.float32(0)), _POS_VALS.astype(np.float32)])
    probes = np.concatenate([probes, -probes])
    np.testing.assert_array_equal(O.half_bits(probes), brute_nearest_half_bits(probes))
