"""GPU parity of the kernels the step runs, at the shapes that select them.

* The per-block int32 Q.K sums, captured inside the real attention kernels
  (kvq_debug_attn_isum: the same build, split plan, LDS swizzle and MFMA
  operands as attn_decode_packed), must equal the oracle's block sums bit
  for bit, for the column layout (single-token decode: 8-wave build, and the
  12-wave build that the 128k step runs) and for the row layout (4 query
  tokens x 4 heads).  Page 1 (summary, body): four 8-bit K values per 32-bit
  word go straight into the integer dot, so these sums are exact.
* The 12-wave column kernel (q4_0 V, head_dim 128, chunks of at least 1536
  tokens) against the oracle on all 32 query heads, plain and with the
  fused append, at 65536 tokens, at the 131073-token plan (chunks of 4128
  tokens, a short last split, a partial tile), at lengths that are not
  whole tiles under forced chunk sizes, and at 262144 tokens (8192-token
  chunks, sampled heads).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_attention_packed_amd as K  # noqa: E402
from decode_attention_packed_amd import workloads as W  # noqa: E402
from oracle import kvq_oracle as O  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402
from tests.test_gpu_append_fused import check_appended_rows, run_fused  # noqa: E402


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _table(ci, max_segs):
    if ci.seg_table is not None:
        return H.dev(ci.seg_table)
    return torch.stack([torch.arange(i * max_segs, (i + 1) * max_segs, dtype=torch.int32)
                        for i in range(ci.spec.n_seq)]).cuda()


def _isum_and_out(ci, cache, table):
    spec = ci.spec
    mx = int(ci.seq_len.max())
    q = H.dev(ci.q)
    out = torch.empty_like(q)
    sl = H.dev(ci.seq_len)
    ws = torch.zeros(max(16, K.attn_decode_packed_workspace_size(cache, spec.n_seq, spec.n_qtok,
                                                                 spec.n_q_heads, mx)),
                     dtype=torch.uint8, device="cuda")
    isum = torch.full((spec.n_seq, spec.n_qtok, spec.n_q_heads, mx, spec.head_dim // 32), -(2 ** 31),
                      dtype=torch.int32, device="cuda")
    K.kvq_debug_attn_isum(cache, q, out, sl, mx, spec.sm_scale, spec.causal, ws, isum,
                          seg_table=table)
    ref = torch.empty_like(q)
    K.attn_decode_packed(cache, q, ref, sl, mx, spec.sm_scale, spec.causal, ws, seg_table=table)
    torch.cuda.synchronize()
    return isum.cpu().numpy(), out.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("name,ctx,fmt", [("tiny", None, None), ("gqa8k", None, W.V_Q4_0),
                                          ("gqa8k", None, W.V_Q8_0), ("long128k", 65536, None),
                                          ("ragged", 3000, None), ("verify128k", 3000, None)])
def test_attention_kernel_block_sums_bitexact(name, ctx, fmt):
    """Every block sum every tile of the attention kernel forms, against
    O.block_isum on the oracle's codes of the same fp32 rows: tiny and gqa8k
    (8-wave column kernel, unsplit and in 32 splits), 65536 tokens of the
    long-context recipe (12-wave column kernel), the ragged batch at head_dim
    64 (column layout, 8 query heads x 2 blocks) and both verify caches (row
    layout).  The hook's output must also equal attn_decode_packed's bit for
    bit: the capture changes nothing else."""
    for ci in W.make_inputs(name, ctx=ctx):
        if fmt is not None and ci.spec.v_format != fmt:
            continue
        spec = ci.spec
        _say(f"block sums {spec.name} ctx {spec.ctx}")
        cache, table, max_segs = H.build_cache(ci)
        isum, out, ref = _isum_and_out(ci, cache, _table(ci, max_segs))
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), spec.name
        qc, _ = O.quantize_q(ci.q)
        G = spec.n_q_heads // spec.n_kv_heads
        for i in range(spec.n_seq):
            L = int(ci.seq_len[i])
            kc, _ = O.quantize_k(H.seq_rows(ci, i, "k"))          # [L][Hkv][D]
            for j in range(spec.n_qtok):
                for h in range(spec.n_q_heads):
                    want = O.block_isum(qc[i, j, h][None, :], kc[:, h // G])   # [L][B]
                    got = isum[i, j, h, :L]
                    if not np.array_equal(got, want):
                        bad = np.argwhere(got != want)
                        raise AssertionError((spec.name, i, j, h, bad[:4].tolist(), int(len(bad))))
        del cache


def _all_heads(ci, got, what):
    H.assert_close(got, H.oracle_attention(ci), what)


def test_w12_all_heads_65536():
    """65536 tokens of the long-context recipe: 32 splits of 2048 tokens run
    the 12-wave column kernel; all 32 query heads against the oracle."""
    ci = W.make_inputs("long128k", ctx=65536)[0]
    _say("w12 all heads 65536")
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    _all_heads(ci, got, "w12 65536 all heads")


def test_w12_all_heads_65536_fused_append():
    """The same through attn_decode_packed_append: the last token's rows are
    appended in the launch (the stale rows in the cache hold other data)."""
    ci = W.make_inputs("long128k", ctx=65536)[0]
    _say("w12 fused all heads 65536")
    got, cache = run_fused(ci, 1)
    check_appended_rows(cache, ci, 1)
    _all_heads(ci, got, "w12 fused 65536 all heads")


@pytest.mark.parametrize("L,chunk", [(6001, 1536), (8191, 2048), (6001, 2048), (8191, 1536)])
def test_w12_ragged_tiles_forced_chunks(L, chunk, monkeypatch):
    """gqa8k-shaped caches (32 / 8 heads, q4_0 V) at lengths that are not
    whole 32-token tiles, with the split size forced to 1536 or 2048 tokens
    so the 12-wave kernel runs: a short last split with a partial last tile.
    All heads, plain and fused."""
    monkeypatch.setenv("KVQ_CHUNK_TOKENS", str(chunk))
    ci = W.make_inputs("gqa8k", ctx=L)[0]
    assert ci.spec.v_format == W.V_Q4_0
    _say(f"w12 L={L} chunk={chunk}")
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    _all_heads(ci, got, f"w12 L{L} chunk{chunk}")
    got_f, cache_f = run_fused(ci, 3)
    check_appended_rows(cache_f, ci, 3)
    _all_heads(ci, got_f, f"w12 fused L{L} chunk{chunk}")


def test_w12_131073_tokens_all_heads():
    """One token past 128k: the default plan cuts 131073 tokens into 32
    splits of 4128 tokens (the last one 3105 tokens, ending in a partial
    tile).  Built with the long-context recipe, the new token appended in
    the launch; all 32 query heads against the oracle."""
    base = W.make_inputs("long128k")[0]
    L = base.spec.ctx + 1
    spec = W.CacheSpec("long131073", 1, 1, base.spec.n_q_heads, base.spec.n_kv_heads,
                       base.spec.head_dim, L, base.spec.v_format)
    k = np.concatenate([base.k, base.extra["append_k"]], axis=1)
    v = np.concatenate([base.v, base.extra["append_v"]], axis=1)
    ci = W.CacheInputs(spec, base.q, k, v, np.array([L], np.int32), None, 1, -(-L // 64) * 64)
    del base
    _say("w12 131073 tokens")
    got, cache = run_fused(ci, 1)
    check_appended_rows(cache, ci, 1)
    _all_heads(ci, got, "w12 131073 fused all heads")


@pytest.mark.parametrize("name,ctx", [("tiny", None), ("gqa8k", 4096), ("verify128k", 3000)])
def test_timeline_hook(name, ctx):
    """kvq_debug_attn_timeline runs the same kernels as attn_decode_packed
    (bit-identical output) and stores, for every work-group that has tokens,
    stamps in phase order: entry <= Q ready <= ring ends, and a merge or
    direct-output stamp for exactly one work-group per (sequence, kv head)."""
    ci = W.make_inputs(name, ctx=ctx)[0]
    spec = ci.spec
    cache, table, max_segs = H.build_cache(ci)
    table = _table(ci, max_segs)
    q, sl, mx = H.dev(ci.q), H.dev(ci.seq_len), int(ci.seq_len.max())
    ws = torch.zeros(max(16, K.attn_decode_packed_workspace_size(cache, spec.n_seq, spec.n_qtok,
                                                                 spec.n_q_heads, mx)),
                     dtype=torch.uint8, device="cuda")
    st = torch.zeros((spec.n_seq, spec.n_kv_heads, 64, 8), dtype=torch.int64, device="cuda")
    out, ref = torch.empty_like(q), torch.empty_like(q)
    K.kvq_debug_attn_timeline(cache, q, out, sl, mx, spec.sm_scale, spec.causal, ws, st, seg_table=table)
    K.attn_decode_packed(cache, q, ref, sl, mx, spec.sm_scale, spec.causal, ws, seg_table=table)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
    T = st.cpu().numpy().view(np.uint64).astype(np.int64)
    live = T[..., 0] > 0
    assert live.any()
    for k in (1, 3, 4):
        assert np.all(T[..., k][live] >= T[..., 0][live])
    assert np.all(T[..., 4][live] >= T[..., 3][live]) and np.all(T[..., 3][live] >= T[..., 1][live])
    merged = live & ((T[..., 7] & 3) != 0)
    assert np.array_equal(merged.sum(axis=2), np.ones(merged.shape[:2], int)) or spec.n_qtok * (
        spec.n_q_heads // spec.n_kv_heads) * (spec.head_dim // 32) > 16   # row layout: merge launch


def test_w12_262144_tokens_sampled_heads():
    """Twice the 128k context: the planner cuts 262144 tokens into 32 splits
    of 8192 (256 tiles per work-group, 21-22 per wave), the longest chunks
    the column kernel runs at this head count; the long-context recipe,
    seven of the 32 query heads (spread over five kv heads) against the
    oracle."""
    ci = W.make_inputs("long128k", ctx=262144)[0]
    _say("w12 262144 tokens")
    cache, table, max_segs = H.build_cache(ci)
    heads = [0, 5, 9, 14, 19, 27, 31]
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got, H.oracle_attention(ci, q_heads=heads), "w12 262144 sampled heads")
