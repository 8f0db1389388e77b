"""GPU parity of the row layout in the 12-wave build: q4_0 V at head_dim 128
with more than 16 query-row x block columns (e.g. 4 causal query tokens x 4
heads, the speculative-verify shape) runs the 12-wave kernels once its
chunks reach 1536 tokens (12 waves x 4 tiles), in a single call and in a
batched launch.  Every case is checked against the oracle on all query
heads; the per-block int32 sums of the 12-wave row kernel are compared bit
for bit.  Chunk sizes are forced through KVQ_CHUNK_TOKENS, so the lengths
below end in short last splits and partial tiles; ragged sequences in
shuffled append-only segments (page 3, "BitLLM", how it differs) and calls
without a segment table take the same kernels."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_attention_packed_amd import workloads as W  # noqa: E402
from oracle import kvq_oracle as O  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402
from tests.test_gpu_append_fused import check_appended_rows, run_fused  # noqa: E402
from tests.test_gpu_batch import run_batch  # noqa: E402
from tests.test_gpu_headline import _isum_and_out, _table  # noqa: E402


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _inputs(L, tq, g, hkv, seed):
    rng = np.random.default_rng(seed)
    spec = W.CacheSpec("w12rows", 1, tq, g * hkv, hkv, 128, L, W.V_Q4_0, causal=True)
    q = rng.standard_normal((1, tq, g * hkv, 128)).astype(np.float32)
    k = (rng.standard_normal((1, L, hkv, 128)) * 1.5).astype(np.float32)
    v = rng.standard_normal((1, L, hkv, 128)).astype(np.float32)
    return W.CacheInputs(spec, q, k, v, np.array([L], np.int32), None, 1, -(-L // 64) * 64)


# (L, chunk, query tokens, heads per kv head): 16 rows; 12 rows (4 padding
# rows in the MFMA columns); 16 query tokens of one head each; one query
# token of 16 grouped heads; a last split of one token, which only the last
# query token sees (the other rows' partials of that split are empty)
CASES = [(6001, 1536, 4, 4), (8191, 2048, 4, 4), (5000, 1536, 3, 4), (7001, 1536, 16, 1),
         (9000, 2048, 1, 16), (6145, 1536, 4, 4)]


@pytest.mark.parametrize("L,chunk,tq,g", CASES)
def test_w12_rows_forced_chunks(L, chunk, tq, g, monkeypatch):
    monkeypatch.setenv("KVQ_CHUNK_TOKENS", str(chunk))
    ci = _inputs(L, tq, g, 2, seed=L + 31 * tq + g)
    _say(f"w12 rows L={L} chunk={chunk} tq={tq} g={g}")
    cache, table, max_segs = H.build_cache(ci)
    want = H.oracle_attention(ci)
    H.assert_close(H.run_attention(cache, ci, table, max_segs), want, f"w12 rows L{L} c{chunk}")
    del cache
    # the fused append of the query tokens' own rows (causal verify step)
    got, cache = run_fused(ci, tq)
    check_appended_rows(cache, ci, tq)
    H.assert_close(got, want, f"w12 rows fused L{L} c{chunk}")


def test_w12_rows_block_sums_bitexact(monkeypatch):
    """The block sums the 12-wave row kernel forms (test hook, same kernel
    build and plan) against O.block_isum, bit for bit, and the hook's output
    bit-identical to the plain call's."""
    monkeypatch.setenv("KVQ_CHUNK_TOKENS", "1536")
    ci = _inputs(4700, 4, 4, 2, seed=4700)
    spec = ci.spec
    _say("w12 rows block sums")
    cache, table, max_segs = H.build_cache(ci)
    isum, out, ref = _isum_and_out(ci, cache, _table(ci, max_segs))
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    qc, _ = O.quantize_q(ci.q)
    kc, _ = O.quantize_k(H.seq_rows(ci, 0, "k"))
    G = spec.n_q_heads // spec.n_kv_heads
    for j in range(spec.n_qtok):
        for h in range(spec.n_q_heads):
            want = O.block_isum(qc[0, j, h][None, :], kc[:, h // G])
            assert np.array_equal(isum[0, j, h, :spec.ctx], want), (j, h)


def test_w12_rows_batched_verify():
    """Both caches of the verify recipe at 40000 tokens in one launch: the
    joint plan's 1920-token chunks run the 12-wave batch kernels; all heads
    of both calls against the oracle."""
    cis = W.make_inputs("verify128k", ctx=40000)
    _say("w12 rows batched verify 40000")
    outs, _ = run_batch(cis)
    for ci, got in zip(cis, outs):
        H.assert_close(got, H.oracle_attention(ci), "w12 batched verify " + ci.spec.name)


def _ragged_segmented(lens, seg, tq, g, hkv, seed):
    """Sequences of the given lengths in `seg`-token segments, dealt from a
    shuffled pool (the segment table of the ragged recipe)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    spec = W.CacheSpec("w12rows_seg", len(lens), tq, g * hkv, hkv, 128, int(lens.max()), W.V_Q4_0,
                       causal=True)
    q = rng.standard_normal((len(lens), tq, g * hkv, 128)).astype(np.float32)
    k = [(rng.standard_normal((int(n), hkv, 128)) * 1.5).astype(np.float32) for n in lens]
    v = [rng.standard_normal((int(n), hkv, 128)).astype(np.float32) for n in lens]
    nseg = (lens + seg - 1) // seg
    pool = rng.permutation(int(nseg.sum())).astype(np.int32)
    table = np.full((len(lens), int(nseg.max())), -1, np.int32)
    pos = 0
    for i, n in enumerate(nseg):
        table[i, :n] = pool[pos:pos + n]
        pos += n
    return W.CacheInputs(spec, q, k, v, lens, table, int(nseg.sum()), seg)


def test_w12_rows_ragged_segments(monkeypatch):
    """Three sequences of 9000, 2500 and 6001 tokens in shuffled 1024-token
    segments, 1536-token chunks: splits cross segment boundaries, the short
    sequence's work-groups leave early, and the fused append lands in each
    sequence's last segment."""
    monkeypatch.setenv("KVQ_CHUNK_TOKENS", "1536")
    ci = _ragged_segmented([9000, 2500, 6001], 1024, 4, 4, 2, seed=515)
    _say("w12 rows ragged segments")
    cache, table, max_segs = H.build_cache(ci)
    want = H.oracle_attention(ci)
    H.assert_close(H.run_attention(cache, ci, table, max_segs), want, "w12 rows ragged segments")
    del cache
    got, cache = run_fused(ci, 4)
    check_appended_rows(cache, ci, 4)
    H.assert_close(got, want, "w12 rows ragged segments fused")


def test_w12_rows_no_table(monkeypatch):
    """The contiguous form without a segment table (sequence i owns segments
    i*max_segs ..): tiles go out before the length is known, bounded by
    max_seq_len, so the shorter sequence's work-groups load past its end."""
    monkeypatch.setenv("KVQ_CHUNK_TOKENS", "1536")
    from tests.test_gpu_no_table import _attend, _build, _inputs as nt_inputs
    ci = nt_inputs([7000, 3100], 2, 4, 4, 128, W.V_Q4_0, True, seed=616)
    _say("w12 rows without a table")
    cache = _build(ci)
    H.assert_close(_attend(cache, ci), H.oracle_attention(ci), "w12 rows no table")
    cache = _build(ci, skip_last=4)
    got = _attend(cache, ci, append_rows=4)
    H.assert_close(got, H.oracle_attention(ci), "w12 rows no table fused")


def test_w12_rows_batched_mixed_calls():
    """Three row-layout calls of different kv-head counts and lengths in one
    batched launch (40000 tokens at 32/8 heads, 30000 at 16/4, 20000 at
    8/2; 4 causal query tokens each): the joint plan's 1920-token chunks run
    the 12-wave batch kernels with 21, 16 and 11 splits, and the merge
    launch combines each call's own split count.  All heads of every call
    against the oracle."""
    cis = [_inputs(40000, 4, 4, 8, seed=41), _inputs(30000, 4, 4, 4, seed=42),
           _inputs(20000, 4, 4, 2, seed=43)]
    _say("w12 rows batched, three calls")
    outs, _ = run_batch(cis)
    for i, (ci, got) in enumerate(zip(cis, outs)):
        H.assert_close(got, H.oracle_attention(ci), f"w12 batched call {i}")
