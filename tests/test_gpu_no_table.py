"""GPU parity of calls without a segment table (the contiguous-cache form:
sequence i owns segments i*max_segs ..), where the kernels issue Q, the
first tiles and the appended rows before the sequence's length is known,
bounded by the call's max_seq_len.  Sequences shorter than max_seq_len make
work-groups load past their end (inside the cache) and leave early, and make
the work-group that holds the appended rows stage them twice.  Every case is
checked against the oracle, the appended rows bit for bit.  Page 3 ("BitLLM",
how it differs) keeps the cache in append-only segments; one segment per
sequence is the contiguous case."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_attention_packed_amd as K  # noqa: E402
from decode_attention_packed_amd import workloads as W  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


def _inputs(lens, hkv, g, tq, d, fmt, causal, seed):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    mx = int(lens.max())
    spec = W.CacheSpec("notable", len(lens), tq, g * hkv, hkv, d, mx, fmt, causal=causal)
    q = rng.standard_normal((len(lens), tq, g * hkv, d)).astype(np.float32)
    k = [(rng.standard_normal((int(n), hkv, d)) * 1.5).astype(np.float32) for n in lens]
    v = [rng.standard_normal((int(n), hkv, d)).astype(np.float32) for n in lens]
    return W.CacheInputs(spec, q, k, v, lens, None, len(lens), -(-mx // 64) * 64)


def _attend(cache, ci, append_rows=0):
    """One call without a table; with append_rows > 0, the last rows of every
    sequence are appended in the same launch (their old rows hold other data)."""
    spec = ci.spec
    q = H.dev(ci.q)
    out = torch.empty_like(q)
    mx = int(ci.seq_len.max())
    sl = H.dev(ci.seq_len)
    ws = torch.zeros(max(16, K.attn_decode_packed_workspace_size(cache, spec.n_seq, spec.n_qtok,
                                                                 spec.n_q_heads, mx)),
                     dtype=torch.uint8, device="cuda")
    if append_rows:
        kn = np.stack([H.seq_rows(ci, i, "k")[-append_rows:] for i in range(spec.n_seq)])
        vn = np.stack([H.seq_rows(ci, i, "v")[-append_rows:] for i in range(spec.n_seq)])
        K.attn_decode_packed_append(cache, q, H.dev(kn), H.dev(vn), out, sl, mx, spec.sm_scale,
                                    spec.causal, ws, seg_table=None, max_segs=1)
    else:
        K.attn_decode_packed(cache, q, out, sl, mx, spec.sm_scale, spec.causal, ws, seg_table=None,
                             max_segs=1)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _build(ci, skip_last=0):
    """The cache, one segment per sequence, filled up to each length less
    skip_last rows; the skipped rows are filled with other data."""
    spec = ci.spec
    cache = K.PackedKVCache(spec.n_kv_heads, spec.head_dim, ci.seg_tokens, spec.n_seq, spec.v_format)
    for i in range(spec.n_seq):
        n = int(ci.seq_len[i])
        k = H.seq_rows(ci, i, "k").copy()
        v = H.seq_rows(ci, i, "v").copy()
        if skip_last:
            k[n - skip_last:] = 9.0
            v[n - skip_last:] = -9.0
        t = torch.tensor([[i]], dtype=torch.int32, device="cuda")
        K.kv_append_quant(cache, H.dev(k[None]), H.dev(v[None]),
                          torch.zeros(1, dtype=torch.int32, device="cuda"), seg_table=t)
    return cache


CASES = [
    # lens, hkv, group, qtok, D, V format, causal: 8-wave column kernel
    ([5000, 2000, 8192, 1, 8190], 2, 4, 1, 128, W.V_Q4_0, False),
    ([3000, 8192, 257], 2, 4, 1, 128, W.V_Q8_0, False),
    # row layout (4 causal query tokens x 4 heads) and head_dim 64
    ([4000, 700, 6001], 2, 4, 4, 128, W.V_Q4_0, True),
    ([6000, 300, 2500, 4096], 4, 2, 1, 64, W.V_Q8_0, False),
    ([2049, 5000], 2, 4, 3, 64, W.V_Q4_0, True),
    # 12-wave column kernel: 16 groups -> 16 splits of 4096 tokens
    ([65536, 40000], 8, 4, 1, 128, W.V_Q4_0, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_no_table_ragged_lengths(case):
    lens, hkv, g, tq, d, fmt, causal = CASES[case]
    ci = _inputs(lens, hkv, g, tq, d, fmt, causal, seed=900 + case)
    print(f"[gpu-test] no table, case {case}: lens {lens}", flush=True)
    cache = _build(ci)
    H.assert_close(_attend(cache, ci), H.oracle_attention(ci), f"no table case {case}")


@pytest.mark.parametrize("case", [0, 2, 4, 5])
def test_no_table_fused_append(case):
    """attn_decode_packed_append without a table: the appended rows of every
    sequence land at its own length, which only the work-group holding them
    learns after its first loads went out for max_seq_len."""
    lens, hkv, g, tq, d, fmt, causal = CASES[case]
    ci = _inputs(lens, hkv, g, tq, d, fmt, causal, seed=950 + case)
    n_new = tq if causal else 1
    print(f"[gpu-test] no table fused, case {case}: lens {lens}", flush=True)
    cache = _build(ci, skip_last=n_new)
    got = _attend(cache, ci, append_rows=n_new)
    torch.cuda.synchronize()
    for i in range(ci.spec.n_seq):
        toks = np.arange(int(ci.seq_len[i]) - n_new, int(ci.seq_len[i]))
        for a, b in zip(H.gpu_rows(cache, ci, i, toks), H.oracle_rows(ci, i, toks)):
            assert np.array_equal(a, b), (case, i)
    H.assert_close(got, H.oracle_attention(ci), f"no table fused case {case}")
