"""GPU parity of the fused step attn_decode_packed_append: the rows it
appends must equal the oracle's encoding bit for bit (as kv_append_quant's
do), and its output must match the oracle's attention over the whole
context, new rows included, within max |err| 2e-3 and relative L2 1e-3."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_attention_packed_amd as K  # noqa: E402
from decode_attention_packed_amd import workloads as W  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _split_inputs(ci, n_new):
    """The cache inputs without each sequence's last n_new rows (the rows
    the fused call appends), and those rows as [S][n_new][Hkv][D]."""
    old = W.CacheInputs(ci.spec, ci.q, None, None, ci.seq_len.copy(), ci.seg_table, ci.n_segs,
                        ci.seg_tokens)
    ks, vs, kn, vn = [], [], [], []
    for i in range(ci.spec.n_seq):
        k = H.seq_rows(ci, i, "k")
        v = H.seq_rows(ci, i, "v")
        ks.append(k[:-n_new])
        vs.append(v[:-n_new])
        kn.append(k[-n_new:])
        vn.append(v[-n_new:])
    old.k, old.v = ks, vs
    old.seq_len = ci.seq_len - n_new
    return old, np.stack(kn), np.stack(vn)


def run_fused(ci, n_new, poison=True):
    """Build the cache from all but the last n_new rows (those rows hold
    other data when `poison`), then run one fused call; returns the output
    and the cache."""
    spec = ci.spec
    old, kn, vn = _split_inputs(ci, n_new)
    cache = K.PackedKVCache(spec.n_kv_heads, spec.head_dim, ci.seg_tokens, ci.n_segs, spec.v_format)
    max_segs = ci.seg_table.shape[1] if ci.seg_table is not None else ci.n_segs // spec.n_seq
    if ci.seg_table is not None:
        table = H.dev(ci.seg_table)
    else:
        table = torch.stack([torch.arange(i * max_segs, (i + 1) * max_segs, dtype=torch.int32)
                             for i in range(spec.n_seq)]).cuda()
    for i in range(spec.n_seq):
        if int(old.seq_len[i]) > 0:
            K.kv_append_quant(cache, H.dev(old.k[i][None]), H.dev(old.v[i][None]),
                              torch.zeros(1, dtype=torch.int32, device="cuda"),
                              seg_table=table[i:i + 1])
    if poison:
        # stale rows where the new ones go: the fused call must not use them
        junk = (np.random.default_rng(99).standard_normal(kn.shape) * 5).astype(np.float32)
        K.kv_append_quant(cache, H.dev(junk), H.dev(-junk), H.dev(old.seq_len), seg_table=table)
    q = H.dev(ci.q)
    out = torch.empty_like(q)
    mx = int(ci.seq_len.max())
    ws = torch.zeros(K.attn_decode_packed_workspace_size(cache, spec.n_seq, spec.n_qtok,
                                                          spec.n_q_heads, mx),
                     dtype=torch.uint8, device="cuda")
    K.attn_decode_packed_append(cache, q, H.dev(kn), H.dev(vn), out, H.dev(ci.seq_len), mx,
                                spec.sm_scale, spec.causal, ws, seg_table=table)
    torch.cuda.synchronize()
    return out.cpu().numpy(), cache


def check_appended_rows(cache, ci, n_new):
    for i in range(ci.spec.n_seq):
        L = int(ci.seq_len[i])
        toks = np.arange(L - n_new, L)
        for g, w, nm in zip(H.gpu_rows(cache, ci, i, toks), H.oracle_rows(ci, i, toks),
                            ("k_qs", "k_d", "v_qs", "v_d")):
            assert np.array_equal(g, w), (ci.spec.name, i, nm, int((g != w).sum()))


@pytest.mark.parametrize("D,G,fmt,L,n_new", [(128, 4, 0, 512, 1), (128, 2, 1, 700, 3),
                                             (64, 1, 1, 4097, 1), (64, 8, 0, 130, 16),
                                             (128, 4, 0, 33, 1), (128, 1, 0, 1, 1),
                                             (128, 4, 1, 258, 4), (64, 2, 0, 4099, 5)])
def test_fused_append_shapes(D, G, fmt, L, n_new):
    """Short and ragged contexts, both V formats, new rows that straddle a
    32-token tile or a 256-token split boundary, and a context made only of
    the new row."""
    rng = np.random.default_rng(D * 7 + G * 3 + fmt + L + n_new)
    Hkv = 2
    spec = W.CacheSpec("fused", 1, 1, G * Hkv, Hkv, D, L, fmt)
    cap = -(-L // 64) * 64 + 64
    ci = W.CacheInputs(spec, rng.standard_normal((1, 1, G * Hkv, D)).astype(np.float32),
                       (rng.standard_normal((1, L, Hkv, D)) * 2).astype(np.float32),
                       rng.standard_normal((1, L, Hkv, D)).astype(np.float32),
                       np.array([L], np.int32), None, 1, cap)
    got, cache = run_fused(ci, n_new)
    check_appended_rows(cache, ci, n_new)
    H.assert_close(got, H.oracle_attention(ci), f"fused D{D} G{G} f{fmt} L{L} new{n_new}")


@pytest.mark.parametrize("name", ["tiny", "gqa8k"])
def test_fused_append_workloads(name):
    for ci in W.make_inputs(name):
        _say(f"fused {ci.spec.name}")
        got, cache = run_fused(ci, 1)
        check_appended_rows(cache, ci, 1)
        H.assert_close(got, H.oracle_attention(ci), "fused " + ci.spec.name)


def test_fused_append_ragged_segments():
    """16 sequences of mixed lengths in scattered 4096-token segments, one
    new row each (some land on the first row of a segment)."""
    ci = W.make_inputs("ragged")[0]
    _say("fused ragged")
    got, cache = run_fused(ci, 1)
    check_appended_rows(cache, ci, 1)
    H.assert_close(got, H.oracle_attention(ci), "fused ragged")


def test_fused_verify_step_appends_draft_tokens():
    """The verify step: the 4 draft tokens are appended and attended under
    the causal mask, for both caches of the workload."""
    for ci in W.make_inputs("verify128k", ctx=3000):
        _say(f"fused verify {ci.spec.name}")
        got, cache = run_fused(ci, ci.spec.n_qtok)
        check_appended_rows(cache, ci, ci.spec.n_qtok)
        H.assert_close(got, H.oracle_attention(ci), "fused verify " + ci.spec.name)


def test_fused_long128k_step():
    """The long-context step at full size: the new token at position 131071
    is appended and attended in one launch; the oracle checks the query
    heads of kv heads 0 and 5."""
    ci = W.make_inputs("long128k")[0]
    L = ci.spec.ctx
    ci.k = ci.k.copy()
    ci.v = ci.v.copy()
    ci.k[:, L - 1] = ci.extra["append_k"][:, 0]
    ci.v[:, L - 1] = ci.extra["append_v"][:, 0]
    _say("fused long128k full size")
    got, cache = run_fused(ci, 1)
    check_appended_rows(cache, ci, 1)
    H.assert_close(got, H.oracle_attention(ci, q_heads=list(range(0, 4)) + list(range(20, 24))),
                   "fused long128k")


def test_fused_equals_append_then_attend():
    """Same cache contents and (to fp32 accumulation order) the same output
    as kv_append_quant followed by attn_decode_packed."""
    ci = W.make_inputs("gqa8k", ctx=5000)[0]
    got, cache_f = run_fused(ci, 2, poison=False)
    old, kn, vn = _split_inputs(ci, 2)
    cache_s = K.PackedKVCache(ci.spec.n_kv_heads, ci.spec.head_dim, ci.seg_tokens, 1, ci.spec.v_format)
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kv_append_quant(cache_s, H.dev(old.k[0][None]), H.dev(old.v[0][None]), z)
    K.kv_append_quant(cache_s, H.dev(kn), H.dev(vn), H.dev(old.seq_len))
    ref = H.run_attention(cache_s, ci, None, 1)
    torch.cuda.synchronize()
    toks = np.arange(int(ci.seq_len[0]))   # rows past the context are never written
    for a, b in zip(H.gpu_rows(cache_f, ci, 0, toks), H.gpu_rows(cache_s, ci, 0, toks)):
        assert np.array_equal(a, b)
    assert np.abs(got - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())
