"""The kernels' small_div (csrc/kvq_attn.hip): n / d computed as
trunc((n + 0.5) * r) in float32 with r = 1 / d, either correctly rounded (the
host's 1.0f / d) or one ulp off (v_rcp_f32).  Its comment claims exactness for
0 <= n < 2^20 and any d >= 1; the kernels use n < 1024 and d <= 128.  This
checks the float32 arithmetic exhaustively for n < 2^14 and d <= 1024, and on
sampled n up to 2^20."""
import numpy as np


def _small_div(n, r):
    v = (n.astype(np.float32) + np.float32(0.5)) * np.float32(r)
    return np.trunc(v.astype(np.float32)).astype(np.int64)


def _reciprocals(d):
    r0 = np.float32(1.0) / np.float32(d)
    return (np.nextafter(r0, np.float32(0.0)), r0, np.nextafter(r0, np.float32(np.inf)))


def test_small_div_exhaustive_small_operands():
    n = np.arange(0, 1 << 14, dtype=np.int64)
    for d in range(1, 1025):
        for r in _reciprocals(d):
            assert np.array_equal(_small_div(n, r), n // d), d


def test_small_div_sampled_up_to_2_20():
    rng = np.random.default_rng(5)
    n = np.concatenate([rng.integers(0, 1 << 20, 200000), (1 << 20) - 1 - np.arange(4096)]).astype(np.int64)
    for d in list(range(1, 300)) + [511, 512, 513, 1023, 4096, 65535, 1 << 19, (1 << 20) - 1]:
        for r in _reciprocals(d):
            assert np.array_equal(_small_div(n, r), n // d), d
