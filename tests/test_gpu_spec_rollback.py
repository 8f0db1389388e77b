"""Speculative decoding around the verify step, on one packed cache.

Each verify call appends the draft tokens' K/V rows and attends with the
draft's query tokens under the causal mask, in one launch
(attn_decode_packed_append).  Accepting k of the n drafted tokens is a
rewind of seq_len to the accepted length: no cache data moves, the rejected
rows stay behind the length, and the next call's appended rows overwrite
them.  Every cycle is checked against the oracle on the accepted history
(output within max |err| 2e-3 and relative L2 1e-3; every cache row below
the new length bit for bit), with sequences that accept different counts,
plain one-token decode steps in between, and segments that the drafted rows
straddle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_attention_packed_amd as K  # noqa: E402
from decode_attention_packed_amd import workloads as W  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402

# (tokens drafted this cycle, tokens accepted per sequence)
CYCLES = [(4, [2, 0]), (4, [4, 1]), (1, [1, 1]), (4, [0, 3]), (3, [3, 2]), (1, [1, 1])]


def _table(S, n_segs_per_seq, scattered, rng):
    ids = np.arange(S * n_segs_per_seq, dtype=np.int32)
    if scattered:
        rng.shuffle(ids)
    return ids.reshape(S, n_segs_per_seq)


@pytest.mark.parametrize("seg_tokens,scattered", [(2048, False), (512, True)])
def test_verify_accept_rollback_cycles(seg_tokens, scattered):
    rng = np.random.default_rng(seg_tokens + scattered)
    S, Hq, Hkv, D, fmt = 2, 32, 8, 128, W.V_Q4_0
    # the drafted rows of the second sequence straddle a 512-token segment
    # boundary in the first cycles
    L = np.array([1000, 1534], dtype=np.int64)
    n_segs_per_seq = 4096 // seg_tokens
    table_np = _table(S, n_segs_per_seq, scattered, rng)
    table = H.dev(table_np)
    cache = K.PackedKVCache(Hkv, D, seg_tokens, S * n_segs_per_seq, fmt)
    hist_k = [rng.standard_normal((int(L[i]), Hkv, D), dtype=np.float32) * 1.5 for i in range(S)]
    hist_v = [rng.standard_normal((int(L[i]), Hkv, D), dtype=np.float32) for i in range(S)]
    for i in range(S):
        K.kv_append_quant(cache, H.dev(hist_k[i][None]), H.dev(hist_v[i][None]),
                          torch.zeros(1, dtype=torch.int32, device="cuda"), seg_table=table[i:i + 1])
    max_len = 4096
    ws = torch.zeros(K.attn_decode_packed_workspace_size(cache, S, 4, Hq, max_len),
                     dtype=torch.uint8, device="cuda")
    for cycle, (n, accept) in enumerate(CYCLES):
        kn = rng.standard_normal((S, n, Hkv, D), dtype=np.float32) * 1.5
        vn = rng.standard_normal((S, n, Hkv, D), dtype=np.float32)
        q = rng.standard_normal((S, n, Hq, D), dtype=np.float32)
        seq_len = (L + n).astype(np.int32)
        spec = W.CacheSpec(f"spec{cycle}", S, n, Hq, Hkv, D, int(seq_len.max()), fmt, causal=True)
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        print(f"[gpu-test] spec cycle {cycle}: seg_tokens={seg_tokens} lengths {L.tolist()} "
              f"+ {n} drafted, accept {accept}", flush=True)
        K.attn_decode_packed_append(cache, H.dev(q), H.dev(kn), H.dev(vn), out, H.dev(seq_len),
                                    int(seq_len.max()), spec.sm_scale, True, ws, seg_table=table)
        torch.cuda.synchronize()
        full_k = [np.concatenate([hist_k[i], kn[i]]) for i in range(S)]
        full_v = [np.concatenate([hist_v[i], vn[i]]) for i in range(S)]
        ci = W.CacheInputs(spec, q, full_k, full_v, seq_len, table_np, S * n_segs_per_seq,
                           seg_tokens)
        H.assert_close(out.cpu().numpy(), H.oracle_attention(ci), f"spec cycle {cycle}")
        for i in range(S):
            toks = np.arange(int(seq_len[i]))
            for g, w, nm in zip(H.gpu_rows(cache, ci, i, toks), H.oracle_rows(ci, i, toks),
                                ("k_qs", "k_d", "v_qs", "v_d")):
                assert np.array_equal(g, w), (cycle, i, nm, int((g != w).sum()))
        # accept a prefix of the drafted tokens: the length moves, no data does
        for i in range(S):
            a = accept[i]
            hist_k[i] = np.concatenate([hist_k[i], kn[i, :a]])
            hist_v[i] = np.concatenate([hist_v[i], vn[i, :a]])
            L[i] += a
    counters = ws[:256 * S * Hkv].cpu().numpy().view(np.uint32)   # one per 256 bytes, the rest unused
    assert not counters.any()
