"""GPU parity over the range of V magnitudes.

Each softmax weight enters the P.V sum as p * d_v rounded to fp16 (d_v the
V block scale).  For small V, p * d_v can fall below the fp16 normal range
and lose precision; the kernels scale the weights by a power of two (16 for
q4_0, 256 for q8_0) that cancels in the normalization.  These cases scale
the V draws of the 8k and 64k workloads by 1e-2 and 1e-3 (and up by 5e3,
within the documented bound of about 32000) and check every query head
against the oracle at the usual tolerance, applied to the outputs divided by
the V factor (the output scales with V; the tolerance is stated for the
workloads' unit-scale draws).  Page 1's body and KLD tables
use both V formats; the scale of V is the model's, not the method's."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_attention_packed_amd import workloads as W  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


def _scaled(name, ctx, fmt, scale):
    cis = [ci for ci in W.make_inputs(name, ctx=ctx) if fmt is None or ci.spec.v_format == fmt]
    ci = cis[0]
    ci.v = (ci.v * np.float32(scale)).astype(np.float32)
    return ci


@pytest.mark.parametrize("fmt", [W.V_Q4_0, W.V_Q8_0])
@pytest.mark.parametrize("scale", [1e-2, 1e-3, 5e3])
def test_v_scale_gqa8k(fmt, scale):
    ci = _scaled("gqa8k", None, fmt, scale)
    print(f"[gpu-test] gqa8k fmt {fmt} V x {scale:g}", flush=True)
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got / scale, H.oracle_attention(ci) / scale, f"gqa8k f{fmt} V x {scale:g}")


@pytest.mark.parametrize("scale", [1e-2, 1e-3])
def test_v_scale_64k_w12(scale):
    """65536 tokens of the long-context recipe with q4_0 V: the 12-wave kernel."""
    ci = _scaled("long128k", 65536, None, scale)
    print(f"[gpu-test] 64k V x {scale:g}", flush=True)
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got / scale, H.oracle_attention(ci) / scale, f"64k q4_0 V x {scale:g}")


@pytest.mark.parametrize("scale", [1e-2, 1e-3])
def test_v_scale_verify_rows(scale):
    """The row layout (4 causal query tokens x 4 heads) with small V."""
    for ci in W.make_inputs("verify128k", ctx=6000):
        ci.v = (ci.v * np.float32(scale)).astype(np.float32)
        print(f"[gpu-test] verify {ci.spec.name} V x {scale:g}", flush=True)
        cache, table, max_segs = H.build_cache(ci)
        got = H.run_attention(cache, ci, table, max_segs)
        H.assert_close(got / scale, H.oracle_attention(ci) / scale,
                       f"verify {ci.spec.name} V x {scale:g}")


@pytest.mark.parametrize("scale", [1e-2, 1e-3])
def test_v_scale_rows_q8_0(scale):
    """The row layout with q8_0 V (the smaller block scale, max|V| / 127) and
    small V: 4 causal query tokens x 4 heads, 2 kv heads, 9000 tokens."""
    rng = np.random.default_rng(4242)
    L, hkv = 9000, 2
    spec = W.CacheSpec("rows_q8", 1, 4, 4 * hkv, hkv, 128, L, W.V_Q8_0, causal=True)
    ci = W.CacheInputs(spec, rng.standard_normal((1, 4, 4 * hkv, 128)).astype(np.float32),
                       (rng.standard_normal((1, L, hkv, 128)) * 1.5).astype(np.float32),
                       (rng.standard_normal((1, L, hkv, 128)) * scale).astype(np.float32),
                       np.array([L], np.int32), None, 1, -(-L // 64) * 64)
    print(f"[gpu-test] rows q8_0 V x {scale:g}", flush=True)
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got / scale, H.oracle_attention(ci) / scale, f"rows q8_0 V x {scale:g}")
