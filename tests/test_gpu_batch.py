"""GPU parity of attn_decode_packed_batch: several attention calls in one
launch (the verify step's main and draft caches; column-layout caches of
different shapes), each call within max |err| 2e-3 and relative L2 1e-3 of
the oracle, and the workspace counters left at zero."""
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


def run_batch(cis):
    built = []
    calls = []
    for ci in cis:
        cache, table, max_segs = H.build_cache(ci)
        spec = ci.spec
        if table is None:
            table = torch.stack([torch.arange(i * max_segs, (i + 1) * max_segs, dtype=torch.int32)
                                 for i in range(spec.n_seq)]).cuda()
        q = H.dev(ci.q)
        out = torch.full_like(q, float("nan"))
        calls.append(dict(cache=cache, q=q, out=out, seq_len=H.dev(ci.seq_len),
                          max_seq_len=int(ci.seq_len.max()), sm_scale=spec.sm_scale,
                          causal=spec.causal, seg_table=table))
        built.append(cache)
    ws = torch.zeros(K.attn_decode_packed_batch_workspace_size(calls), dtype=torch.uint8, device="cuda")
    K.attn_decode_packed_batch(calls, ws)
    torch.cuda.synchronize()
    return [c["out"].cpu().numpy() for c in calls], ws


def test_batch_verify_small():
    cis = W.make_inputs("verify128k", ctx=3000)
    _say("batch verify ctx 3000")
    outs, ws = run_batch(cis)
    for ci, got in zip(cis, outs):
        H.assert_close(got, H.oracle_attention(ci), "batch verify " + ci.spec.name)


def test_batch_verify128k_full_size():
    """Both caches of the verify step at 131072 tokens in one launch; the
    oracle checks kv heads 0 and 3 of each."""
    cis = W.make_inputs("verify128k")
    _say("batch verify128k full size")
    outs, ws = run_batch(cis)
    for ci, got in zip(cis, outs):
        G = ci.spec.n_q_heads // ci.spec.n_kv_heads
        heads = [h for h in range(ci.spec.n_q_heads) if h // G in (0, 3)]
        H.assert_close(got, H.oracle_attention(ci, heads), "batch verify128k " + ci.spec.name)


def test_batch_column_layout_mixed_shapes():
    """Column-layout calls of different shapes and lengths in one launch:
    tiny (1 kv head), gqa8k (8 kv heads) and a 2-sequence ragged-length cache."""
    rng = np.random.default_rng(77)
    spec = W.CacheSpec("two_seq", 2, 1, 8, 2, 128, 5000, W.V_Q4_0)
    lens = np.array([5000, 1234], np.int32)
    ci3 = W.CacheInputs(spec, rng.standard_normal((2, 1, 8, 128)).astype(np.float32),
                        [rng.standard_normal((int(n), 2, 128)).astype(np.float32) for n in lens],
                        [rng.standard_normal((int(n), 2, 128)).astype(np.float32) for n in lens],
                        lens, None, 2, 5056)
    cis = [W.make_inputs("tiny")[0], W.make_inputs("gqa8k")[0], ci3]
    _say("batch column layout")
    outs, ws = run_batch(cis)
    for ci, got in zip(cis, outs):
        H.assert_close(got, H.oracle_attention(ci), "batch cols " + ci.spec.name)
    # each call's counters (the first bytes of its workspace part) end at zero
    assert not ws.cpu().numpy()[:16].any()


def test_batch_wide_unsplit_call_with_split_call():
    """A wide unsplit call (24 sequences x 16 kv heads, lengths with ties:
    its work-groups take groups by length) and a split call (8 kv heads, 32
    splits merged in their last work-group) in one launch; each must match
    the oracle and leave its counters at zero."""
    rng = np.random.default_rng(5151)
    S, hkv, G, D = 24, 16, 2, 128
    lens = rng.integers(1, 900, size=S).astype(np.int32)
    lens[::4] = lens[1]
    seg = (int(lens.max()) + 63) // 64 * 64
    spec = W.CacheSpec("wide", S, 1, G * hkv, hkv, D, int(lens.max()), W.V_Q4_0)
    wide = W.CacheInputs(spec, rng.standard_normal((S, 1, G * hkv, D)).astype(np.float32),
                         [rng.standard_normal((int(n), hkv, D)).astype(np.float32) for n in lens],
                         [rng.standard_normal((int(n), hkv, D)).astype(np.float32) for n in lens],
                         lens, None, S, seg)
    cis = [wide, W.make_inputs("gqa8k", ctx=4096)[0]]
    _say("batch wide unsplit + split")
    outs, ws = run_batch(cis)
    for ci, got in zip(cis, outs):
        H.assert_close(got, H.oracle_attention(ci), "batch " + ci.spec.name)
    assert not ws.cpu().numpy()[:4 * S * hkv].any()
