"""GPU parity of the row layout's split-merge launch (`k_split_merge`) at the
split counts that take its different load paths: it loads the first 32
splits' maxima, sums and partial rows in one go and any further splits in
batches of 32, so 64 splits (two full batches) and 47 (one full batch and
15) are checked against the oracle, as are 21 (one partial batch).  Query
rows are 4 causal tokens x 4 heads, so the row layout runs; each case is
one sequence of a few kv heads, the shape of the speculative-verify draft
cache at a length the oracle computes quickly.  The split count is pinned
through the workspace size (one partial slot per split)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_attention_packed_amd as K  # noqa: E402
from decode_attention_packed_amd import workloads as W  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


def _inputs(L, hkv, d, fmt, seed):
    rng = np.random.default_rng(seed)
    g, tq = 4, 4
    spec = W.CacheSpec("split_merge", 1, tq, g * hkv, hkv, d, L, fmt, causal=True)
    q = rng.standard_normal((1, tq, g * hkv, d)).astype(np.float32)
    k = (rng.standard_normal((1, L, hkv, d)) * 1.5).astype(np.float32)
    v = rng.standard_normal((1, L, hkv, d)).astype(np.float32)
    return W.CacheInputs(spec, q, k, v, np.array([L], np.int32), None, 1, -(-L // 64) * 64)


def _slots(cache, spec, L):
    """Partial slots per (sequence, kv head) from the workspace size:
    256-byte counters, then [groups][slots][rows][D] fp32 rows and
    [groups][slots][rows][2] fp32 (m, l), each part rounded to 256 bytes."""
    need = K.attn_decode_packed_workspace_size(cache, 1, spec.n_qtok, spec.n_q_heads, L)
    groups, rows, d = spec.n_kv_heads, spec.n_qtok * (spec.n_q_heads // spec.n_kv_heads), spec.head_dim
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    hits = [s for s in range(1, 65)
            if r256(groups * 256) + r256(groups * s * rows * d * 4) + r256(groups * s * rows * 8) == need]
    assert len(hits) == 1, (need, hits)
    return hits[0]


@pytest.mark.parametrize("L,hkv,d,fmt,splits", [
    (16384, 4, 128, W.V_Q4_0, 64),    # 64 splits of 256 tokens: two full batches of 32
    (12000, 4, 128, W.V_Q8_0, 47),    # 47 splits, the last one short: 32 + 15
    (16384, 4, 64, W.V_Q8_0, 64),     # head_dim 64
    (5376, 4, 128, W.V_Q4_0, 21),     # 21 splits: one partial batch
])
def test_split_merge_launch_batches(L, hkv, d, fmt, splits):
    ci = _inputs(L, hkv, d, fmt, seed=700 + L + d)
    print(f"[gpu-test] split merge L={L} hkv={hkv} D={d} fmt={fmt}", flush=True)
    cache, table, max_segs = H.build_cache(ci)
    assert _slots(cache, ci.spec, L) == splits
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got, H.oracle_attention(ci), f"split merge L={L} D={d}")
