"""GPU parity: the HIP path (through the C ABI) against the oracle.

Quantize/pack output, Q codes and per-block integer sums are compared bit
for bit; attention outputs must be within max |err| 2e-3 and relative L2
1e-3 of the oracle on the same seeded inputs."""
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


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


# ---------------------------------------------------------------------------
# append: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "gqa8k", "ragged"])
def test_append_bitexact_full(name):
    for ci in W.make_inputs(name):
        _say(f"append {ci.spec.name}")
        cache, table, max_segs = H.build_cache(ci)
        torch.cuda.synchronize()
        for i in range(ci.spec.n_seq):
            toks = np.arange(int(ci.seq_len[i]))
            got = H.gpu_rows(cache, ci, i, toks)
            want = H.oracle_rows(ci, i, toks)
            for g, w, nm in zip(got, want, ("k_qs", "k_d", "v_qs", "v_d")):
                assert g.shape == w.shape, nm
                assert np.array_equal(g, w), (ci.spec.name, i, nm, int((g != w).sum()))


def test_append_token_by_token_equals_bulk():
    ci = W.make_inputs("tiny", ctx=200)[0]
    bulk, _, _ = H.build_cache(ci)
    spec = ci.spec
    step = K.PackedKVCache(spec.n_kv_heads, spec.head_dim, bulk.seg_tokens, 1, spec.v_format)
    for t in range(200):
        kk = H.dev(ci.k[:, t:t + 1])
        vv = H.dev(ci.v[:, t:t + 1])
        K.kv_append_quant(step, kk, vv, torch.tensor([t], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    toks = np.arange(200)
    for a, b in zip(H.gpu_rows(bulk, ci, 0, toks), H.gpu_rows(step, ci, 0, toks)):
        assert np.array_equal(a, b)


def test_append_edge_blocks_bitexact():
    # zero blocks, exact ties, tiny values, large values, sign mixtures
    rng = np.random.default_rng(7)
    D, Hkv, n = 128, 2, 64
    k = rng.standard_normal((1, n, Hkv, D)).astype(np.float32)
    k[0, 0] = 0.0
    k[0, 1, :, :32] = np.float32(-0.0)
    k[0, 2] = (np.arange(D) % 32 - 15.5).astype(np.float32)
    k[0, 3] *= np.float32(1e-6)
    k[0, 4] *= np.float32(3e3)
    k[0, 5, :, 0] = 127.0
    k[0, 5, :, 1:32] = np.arange(31, dtype=np.float32) + 0.5
    k[0, 6, :, :32] = 5.0                    # every element ties for the largest magnitude
    k[0, 7, :, 32:64] = -5.0
    k[0, 7, :, 40] = 5.0
    for fmt in (O.V_Q4_0, O.V_Q8_0):
        spec = W.CacheSpec("edge", 1, 1, Hkv, Hkv, D, n, fmt)
        ci = W.CacheInputs(spec, np.zeros((1, 1, Hkv, D), np.float32), k, k.copy(),
                           np.array([n], np.int32), None, 1, 64)
        cache, _, _ = H.build_cache(ci)
        torch.cuda.synchronize()
        toks = np.arange(n)
        got = H.gpu_rows(cache, ci, 0, toks)
        want = H.oracle_rows(ci, 0, toks)
        for g, w, nm in zip(got, want, ("k_qs", "k_d", "v_qs", "v_d")):
            assert np.array_equal(g, w), (fmt, nm, np.argwhere(g != w)[:5])


def test_append_full_size_sampled_rows():
    # long-context cache at full size: bulk append, then check 4096 sampled rows
    ci = W.make_inputs("long128k")[0]
    _say("append long128k full size")
    cache, _, _ = H.build_cache(ci)
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(0).choice(ci.spec.ctx, 4096, replace=False))
    toks[-1] = ci.spec.ctx - 1
    got = H.gpu_rows(cache, ci, 0, toks)
    want = H.oracle_rows(ci, 0, toks)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


# ---------------------------------------------------------------------------
# Q quantization and per-block integer sums: bit-exact
# ---------------------------------------------------------------------------

def test_quant_q_bitexact():
    rng = np.random.default_rng(8)
    for D in (64, 128):
        q = rng.standard_normal((300, D)).astype(np.float32)
        q[0] = 0
        q[1] *= np.float32(1e-5)
        q[2] = (np.arange(D) % 32 - 15.5).astype(np.float32)
        q[3, :32] = 127.0 * (np.arange(32) % 2 * 2 - 1)
        q[4] *= np.float32(5e3)
        codes = torch.empty((300, D), dtype=torch.int8, device="cuda")
        scales = torch.empty((300, D // 32), dtype=torch.float32, device="cuda")
        K.kvq_debug_quant_q(H.dev(q), codes, scales)
        torch.cuda.synchronize()
        wc, wd = O.quantize_q(q)
        assert np.array_equal(codes.cpu().numpy(), wc)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), wd.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "gqa8k", "ragged"])
def test_qk_isum_bitexact(name):
    ci = W.make_inputs(name, ctx=None if name != "ragged" else 3000)[0]
    cache, table, max_segs = H.build_cache(ci)
    spec = ci.spec
    mx = int(ci.seq_len.max())
    isum = torch.zeros((spec.n_seq, spec.n_qtok, spec.n_q_heads, mx, spec.head_dim // 32),
                       dtype=torch.int32, device="cuda")
    if table is None:
        table = torch.arange(spec.n_seq, dtype=torch.int32, device="cuda")[:, None]
    K.kvq_debug_qk_isum(cache, H.dev(ci.q), H.dev(ci.seq_len), mx, isum, seg_table=table)
    torch.cuda.synchronize()
    got = isum.cpu().numpy()
    qc, _ = O.quantize_q(ci.q)
    G = spec.n_q_heads // spec.n_kv_heads
    for i in range(spec.n_seq):
        L = int(ci.seq_len[i])
        kc, _ = O.quantize_k(H.seq_rows(ci, i, "k"))          # [L][Hkv][D]
        for h in range(spec.n_q_heads):
            want = O.block_isum(qc[i, 0, h][None, :], kc[:, h // G])   # [L][B]
            assert np.array_equal(got[i, 0, h, :L], want), (name, i, h)


# ---------------------------------------------------------------------------
# attention parity
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "gqa8k", "ragged"])
def test_attention_parity(name):
    for ci in W.make_inputs(name):
        _say(f"attention {ci.spec.name}")
        cache, table, max_segs = H.build_cache(ci)
        got = H.run_attention(cache, ci, table, max_segs)
        ref = H.oracle_attention(ci)
        H.assert_close(got, ref, ci.spec.name)


@pytest.mark.parametrize("n_seq,hkv,fmt", [(40, 8, W.V_Q8_0), (23, 15, W.V_Q4_0), (70, 4, W.V_Q4_0)])
def test_attention_wide_batch_length_order(n_seq, hkv, fmt):
    """Wide unsplit batches: up to 64 sequences, work-groups take groups in
    order of decreasing length (first half) and increasing length (second
    half), each work-group ranking the sequences itself; ties keep sequence
    order.  Lengths with repeats, an odd group count (23 x 15 = 345) and a
    batch past 64 sequences (plain order) must all match the oracle."""
    rng = np.random.default_rng(n_seq * 100 + hkv)
    D, G = 128, 2
    lens = rng.integers(1, 700, size=n_seq).astype(np.int32)
    lens[::5] = lens[0]            # ties
    lens[1] = 1
    seg = (int(lens.max()) + 63) // 64 * 64
    spec = W.CacheSpec("wide", n_seq, 1, G * hkv, hkv, D, int(lens.max()), fmt)
    ci = W.CacheInputs(spec, rng.standard_normal((n_seq, 1, G * hkv, D)).astype(np.float32),
                       [rng.standard_normal((int(n), hkv, D)).astype(np.float32) for n in lens],
                       [rng.standard_normal((int(n), hkv, D)).astype(np.float32) for n in lens],
                       lens, None, n_seq, seg)
    _say(f"wide batch {n_seq} seqs x {hkv} kv heads")
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got, H.oracle_attention(ci), f"wide batch {n_seq}x{hkv}")


@pytest.mark.parametrize("chunk", [1024, 4096])
def test_attention_ragged_forced_splits(chunk, monkeypatch):
    """The ragged batch with the split size forced small, so its long
    sequences cross many splits and segments (its default plan keeps at most
    two splits per sequence, the batch being wide enough to fill the GPU)."""
    monkeypatch.setenv("KVQ_CHUNK_TOKENS", str(chunk))
    ci = W.make_inputs("ragged")[0]
    _say(f"attention ragged, {chunk}-token splits")
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got, H.oracle_attention(ci), f"ragged chunk {chunk}")


def test_attention_parity_long128k_step():
    """The long-context step at full size: append one token at the last
    position, then attend over all 131072 tokens; the oracle checks the
    query heads of kv heads 0 and 5 (one head computed one by one is the
    same computation for every head)."""
    ci = W.make_inputs("long128k")[0]
    _say("attention long128k full size")
    cache, table, max_segs = H.build_cache(ci)
    L = ci.spec.ctx
    ak, av = ci.extra["append_k"], ci.extra["append_v"]
    K.kv_append_quant(cache, H.dev(ak), H.dev(av), torch.tensor([L - 1], dtype=torch.int32, device="cuda"))
    got = H.run_attention(cache, ci, table, max_segs)
    ci.k = ci.k.copy()
    ci.v = ci.v.copy()
    ci.k[:, L - 1] = ak[:, 0]
    ci.v[:, L - 1] = av[:, 0]
    ref = H.oracle_attention(ci, q_heads=list(range(0, 4)) + list(range(20, 24)))
    H.assert_close(got, ref, "long128k")


@pytest.mark.parametrize("D,G,fmt,L", [(128, 1, 0, 1), (128, 2, 1, 63), (128, 8, 0, 777),
                                       (64, 1, 1, 4097), (64, 4, 0, 130), (128, 4, 1, 2049),
                                       (64, 8, 1, 65), (128, 4, 0, 3)])
def test_attention_shapes_and_ragged_tails(D, G, fmt, L):
    rng = np.random.default_rng(D * 1000 + G * 10 + fmt + L)
    Hkv = 2
    spec = W.CacheSpec("edge", 1, 1, G * Hkv, Hkv, D, L, fmt)
    cap = -(-L // 64) * 64 + 64
    ci = W.CacheInputs(spec, rng.standard_normal((1, 1, G * Hkv, D)).astype(np.float32),
                       (rng.standard_normal((1, L, Hkv, D)) * 2).astype(np.float32),
                       rng.standard_normal((1, L, Hkv, D)).astype(np.float32),
                       np.array([L], np.int32), None, 1, cap)
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got, H.oracle_attention(ci), f"D{D} G{G} f{fmt} L{L}")


@pytest.mark.parametrize("D,Tq,G,causal,L,fmt", [(128, 4, 4, True, 2000, 0), (128, 2, 8, True, 333, 1),
                                                (128, 16, 1, True, 130, 0), (128, 3, 4, False, 4100, 1),
                                                (128, 4, 2, True, 4, 0), (128, 5, 3, True, 700, 1),
                                                (64, 4, 4, True, 1500, 1), (64, 16, 1, True, 300, 0),
                                                (64, 3, 4, False, 2100, 0), (64, 9, 1, True, 9, 1),
                                                (128, 1, 16, False, 3000, 0), (64, 1, 16, True, 777, 1)])
def test_attention_multi_query(D, Tq, G, causal, L, fmt):
    """The row layout (more than 16 query-row x block columns): head_dim 128
    and 64, both V formats, causal and not, contexts down to the query count."""
    rng = np.random.default_rng(D * 7 + Tq * 100 + G * 10 + L)
    Hkv = 2
    spec = W.CacheSpec("mq", 1, Tq, G * Hkv, Hkv, D, L, fmt, causal=causal)
    cap = -(-L // 64) * 64
    ci = W.CacheInputs(spec, rng.standard_normal((1, Tq, G * Hkv, D)).astype(np.float32),
                       (rng.standard_normal((1, L, Hkv, D)) * 1.5).astype(np.float32),
                       rng.standard_normal((1, L, Hkv, D)).astype(np.float32),
                       np.array([L], np.int32), None, 1, cap)
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got, H.oracle_attention(ci), f"D{D} Tq{Tq} G{G} causal{causal} L{L}")


@pytest.mark.parametrize("D,Tq,G,L,fmt", [(128, 2, 2, 517, 0), (128, 4, 1, 1000, 1),
                                           (128, 3, 1, 64, 0), (64, 4, 2, 4200, 0),
                                           (64, 2, 4, 300, 1), (128, 2, 1, 2, 0)])
def test_attention_multi_query_column_layout(D, Tq, G, L, fmt):
    """Causal multi-token groups small enough for the column layout
    (rows x blocks <= 16), including a context equal to the query count."""
    rng = np.random.default_rng(D + Tq * 100 + G * 10 + L)
    Hkv = 2
    spec = W.CacheSpec("mqc", 1, Tq, G * Hkv, Hkv, D, L, fmt, causal=True)
    cap = -(-L // 64) * 64
    ci = W.CacheInputs(spec, rng.standard_normal((1, Tq, G * Hkv, D)).astype(np.float32),
                       (rng.standard_normal((1, L, Hkv, D)) * 1.5).astype(np.float32),
                       rng.standard_normal((1, L, Hkv, D)).astype(np.float32),
                       np.array([L], np.int32), None, 1, cap)
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)
    H.assert_close(got, H.oracle_attention(ci), f"cols D{D} Tq{Tq} G{G} L{L}")


def test_attention_verify_small():
    # the speculative-verify recipe (main 32/8 and draft 16/4, 4 causal query
    # tokens) at a short context, every output checked
    for ci in W.make_inputs("verify128k", ctx=3000):
        _say(f"verify small {ci.spec.name}")
        cache, table, max_segs = H.build_cache(ci)
        got = H.run_attention(cache, ci, table, max_segs)
        H.assert_close(got, H.oracle_attention(ci), "verify-small " + ci.spec.name)


def test_attention_verify128k_full_size():
    """Both caches of the verify step at 131072 tokens; the oracle checks
    the query heads of two kv heads per cache."""
    for ci, kvs in zip(W.make_inputs("verify128k"), ([0, 7], [1, 3])):
        _say(f"verify full {ci.spec.name}")
        cache, table, max_segs = H.build_cache(ci)
        got = H.run_attention(cache, ci, table, max_segs)
        G = ci.spec.n_q_heads // ci.spec.n_kv_heads
        heads = [h for kv in kvs for h in range(kv * G, (kv + 1) * G)]
        H.assert_close(got, H.oracle_attention(ci, q_heads=heads), "verify-full " + ci.spec.name)
        del cache


@pytest.mark.parametrize("name,ctx", [("tiny", None), ("gqa8k", None), ("long128k", 65536),
                                      ("verify128k", 6000), ("ragged", None)])
def test_attention_deterministic(name, ctx):
    """For a fixed split plan, repeated calls on the same inputs give
    bit-identical outputs: every wave accumulates a fixed set of tiles in a
    fixed order, and the split merge combines partials in split order.
    Covers the 8-wave and 12-wave column kernels (tiny, gqa8k in both V
    formats, a 64k-token cache), the row layout with its merge launch (the
    verify caches) and the length-ordered ragged batch."""
    for ci in W.make_inputs(name, ctx=ctx):
        _say(f"determinism {ci.spec.name} ctx {ci.spec.ctx}")
        cache, table, max_segs = H.build_cache(ci)
        runs = [H.run_attention(cache, ci, table, max_segs) for _ in range(3)]
        for r in runs[1:]:
            assert np.array_equal(runs[0].view(np.uint32), r.view(np.uint32)), ci.spec.name
        del cache


def test_workspace_reuse_across_shapes():
    # counters left at zero: the same workspace serves calls of different shapes
    ci = W.make_inputs("gqa8k", ctx=4096)[0]
    cache, table, max_segs = H.build_cache(ci)
    need = K.attn_decode_packed_workspace_size(cache, 1, 1, 32, 4096)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    q = H.dev(ci.q)
    out = torch.empty_like(q)
    ref_full = H.oracle_attention(ci)
    for L in (4096, 1000, 4096, 77):
        sl = torch.tensor([L], dtype=torch.int32, device="cuda")
        K.attn_decode_packed(cache, q, out, sl, L, ci.spec.sm_scale, False, ws)
        torch.cuda.synchronize()
        if L == 4096:
            H.assert_close(out.cpu().numpy(), ref_full, f"reuse L={L}")
    counters = ws[:256 * 8].cpu().numpy().view(np.uint32)   # one per 256 bytes, the rest unused
    assert not counters.any()


def test_workspace_reuse_changing_inputs_odd_groups():
    """Three kv heads (a group count that is not a multiple of 8) split many
    ways, three calls with different queries on one workspace: every call
    must match the oracle.  The group's splits are spread over the XCDs, so
    its split merge reads partials written through other XCDs' L2s after an
    agent-scope acquire; lines an earlier call left in any L2 must not leak
    into a later call's output."""
    rng = np.random.default_rng(31)
    L, Hkv, G, D = 16384, 3, 4, 128
    spec = W.CacheSpec("odd3", 1, 1, Hkv * G, Hkv, D, L, W.V_Q4_0)
    k = rng.standard_normal((1, L, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((1, L, Hkv, D)).astype(np.float32)
    ci = W.CacheInputs(spec, rng.standard_normal((1, 1, Hkv * G, D)).astype(np.float32), k, v,
                       np.array([L], np.int32), None, 1, L)
    _say("workspace reuse, 3 kv heads, changing queries")
    cache, table, max_segs = H.build_cache(ci)
    need = K.attn_decode_packed_workspace_size(cache, 1, 1, Hkv * G, L)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    for call in range(3):
        ci.q = (rng.standard_normal(ci.q.shape) * (1.0 + call)).astype(np.float32)
        q = H.dev(ci.q)
        out = torch.empty_like(q)
        K.attn_decode_packed(cache, q, out, sl, L, spec.sm_scale, False, ws)
        torch.cuda.synchronize()
        H.assert_close(out.cpu().numpy(), H.oracle_attention(ci), f"odd groups call {call}")
    assert not ws[:256 * Hkv].cpu().numpy().any()


def test_attention_errors_leave_output_untouched():
    ci = W.make_inputs("tiny", ctx=128)[0]
    cache, table, max_segs = H.build_cache(ci)
    q = H.dev(ci.q)
    out = torch.full_like(q, 7.0)
    sl = H.dev(ci.seq_len)
    need = K.attn_decode_packed_workspace_size(cache, 1, 1, 4, 128)
    small = torch.zeros(max(need - 16, 16), dtype=torch.uint8, device="cuda")
    with pytest.raises(K.KvqError) as e:
        K.attn_decode_packed(cache, q, out, sl, 128, 0.1, False, small)
    assert e.value.status == K.KVQ_ERR_WORKSPACE
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(K.KvqError) as e:
        K.attn_decode_packed(cache, q, out, sl, 100000, 0.1, False, ws)
    assert e.value.status == K.KVQ_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
