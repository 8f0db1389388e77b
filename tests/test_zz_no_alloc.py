"""GPU check of attn_decode_packed_noalloc, the entry point for callers that
cannot allocate: its workspace is the library's static device array.  Its
output must equal attn_decode_packed's (caller workspace) bit for bit, and
both must match the oracle, over a sequence of calls of different sizes and
layouts on the one shared array: each later call smaller than the first,
then the first again (the array keeps every call's bytes, so counters and
partials left by one call must not leak into the next)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_attention_packed_amd as K  # noqa: E402
from decode_attention_packed_amd import workloads as W  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


def _case(ci):
    spec = ci.spec
    cache, table, max_segs = H.build_cache(ci)
    if table is None:
        table = torch.stack([torch.arange(i * max_segs, (i + 1) * max_segs, dtype=torch.int32)
                             for i in range(spec.n_seq)]).cuda()
    return dict(ci=ci, cache=cache, table=table, q=H.dev(ci.q), sl=H.dev(ci.seq_len),
                mx=int(ci.seq_len.max()), ref=H.oracle_attention(ci))


def _run(c, noalloc):
    spec = c["ci"].spec
    out = torch.full_like(c["q"], float("nan"))
    if noalloc:
        K.attn_decode_packed_noalloc(c["cache"], c["q"], out, c["sl"], c["mx"], spec.sm_scale,
                                     spec.causal, seg_table=c["table"])
    else:
        ws = torch.zeros(max(16, K.attn_decode_packed_workspace_size(
            c["cache"], spec.n_seq, spec.n_qtok, spec.n_q_heads, c["mx"])), dtype=torch.uint8,
            device="cuda")
        K.attn_decode_packed(c["cache"], c["q"], out, c["sl"], c["mx"], spec.sm_scale, spec.causal,
                             ws, seg_table=c["table"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_workspace_entry_point():
    rows_big = _case(W.make_inputs("verify128k", ctx=65536)[0])   # 12-wave row kernels + merge launch
    big = _case(W.make_inputs("long128k", ctx=65536)[0])        # 12-wave build, 32 splits
    small = _case(W.make_inputs("gqa8k", ctx=4096)[0])          # 8-wave build, 16 splits
    rows = _case(W.make_inputs("verify128k", ctx=3000)[1])      # row layout + merge launch
    for name, c in (("verify main 65536", rows_big), ("65536 tokens", big), ("gqa8k 4096", small),
                    ("verify draft 3000", rows), ("verify main 65536 again", rows_big)):
        print(f"[gpu-test] noalloc {name}", flush=True)
        got = _run(c, noalloc=True)
        want = _run(c, noalloc=False)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name
        H.assert_close(got, c["ref"], "noalloc " + name)


def test_noalloc_rejects_oversize_calls():
    ci = W.make_inputs("tiny", ctx=64)[0]
    cache, table, max_segs = H.build_cache(ci)
    q = torch.zeros((128, 4, 4, 128), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    sl = torch.full((128,), 64, dtype=torch.int32, device="cuda")
    tab = torch.zeros((128, 1), dtype=torch.int32, device="cuda")
    # 128 sequences x 1 kv head x 16 rows: 1 MiB of partials fits
    K.attn_decode_packed_noalloc(cache, q, out, sl, 64, 0.1, True, seg_table=tab)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    big_q = torch.zeros((1100, 4, 4, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(K.KvqError) as e:
        K.attn_decode_packed_noalloc(cache, big_q, torch.empty_like(big_q),
                                     torch.full((1100,), 64, dtype=torch.int32, device="cuda"), 64,
                                     0.1, True, seg_table=torch.zeros((1100, 1), dtype=torch.int32,
                                                                      device="cuda"))
    assert e.value.status == K.KVQ_ERR_WORKSPACE


def test_noalloc_captured_in_a_graph():
    """The entry point for callers that cannot allocate, captured once in a
    graph (its counter fill is a kernel, not a memset) and replayed with new
    Q each time, eager calls of the workspace entry point in between: every
    replay equals the eager call on the same Q bit for bit."""
    ci = W.make_inputs("gqa8k", ctx=4096)[0]
    c = _case(ci)
    spec = ci.spec
    q = c["q"].clone()
    out = torch.empty_like(q)
    args = (c["cache"], q, out, c["sl"], c["mx"], spec.sm_scale, spec.causal)
    # the first call on a device looks up the scratch array's address: outside the capture
    K.attn_decode_packed_noalloc(*args, seg_table=c["table"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side), torch.cuda.graph(graph, stream=side):
        K.attn_decode_packed_noalloc(*args, seg_table=c["table"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(4242)
    for rep in range(4):
        print(f"[gpu-test] noalloc graph replay {rep}", flush=True)
        qn = (rng.standard_normal(tuple(q.shape)) * (1.0 + rep)).astype(np.float32)
        q.copy_(torch.from_numpy(qn).cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = _run(dict(c, q=q), noalloc=False)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), rep
