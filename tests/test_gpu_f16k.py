"""GPU parity of the fp16-K A/B reference (kv_append_f16k, attn_decode_f16k)
against the oracle's decode_attention_f16k: K rows bit for bit as binary16
(round to nearest even), V rows bit for bit as kv_append_quant's, attention
within max |err| 2e-3 and relative L2 1e-3."""
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


def build_f16k(ci):
    """One contiguous segment per sequence, filled by kv_append_f16k."""
    spec = ci.spec
    cache = K.F16KCache(spec.n_kv_heads, spec.head_dim, ci.seg_tokens, ci.n_segs, spec.v_format)
    per = ci.n_segs // spec.n_seq
    table = torch.arange(ci.n_segs, dtype=torch.int32).view(spec.n_seq, per).cuda()
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(spec.n_seq):
        K.kv_append_f16k(cache, H.dev(H.seq_rows(ci, i, "k")[None]), H.dev(H.seq_rows(ci, i, "v")[None]),
                         zero, seg_table=table[i:i + 1])
    torch.cuda.synchronize()
    return cache, table


def check_rows(cache, ci):
    """K rows as binary16 bits, V planes as the oracle's encoding (one
    segment per sequence)."""
    per = ci.n_segs // ci.spec.n_seq
    for i in range(ci.spec.n_seq):
        L = int(ci.seq_len[i])
        k = H.seq_rows(ci, i, "k")[:L]
        got_k = cache.k[i * per, :, :L].cpu().numpy().view(np.uint16)     # [Hkv][L][D]
        assert np.array_equal(got_k, O.half_bits(k.transpose(1, 0, 2))), ("k", i)
        v = H.seq_rows(ci, i, "v")[:L].transpose(1, 0, 2)
        vp, vd = O.encode_v(v, ci.spec.v_format)
        ntile = ci.seg_tokens // 32
        for plane, want in ((cache.v_qs, vp), (cache.v_d, vd)):
            s_, h_, _, w_ = plane.shape
            t5 = plane.view(s_, h_, ntile, w_, 32)[i * per]          # [Hkv][tile][w][32]
            g = t5.permute(0, 1, 3, 2).reshape(h_, ntile * 32, w_)[:, :L].cpu().numpy()
            assert np.array_equal(g.view(want.dtype), want), ("v plane", i)


def oracle_f16k(ci, q_heads=None):
    spec = ci.spec
    G = spec.n_q_heads // spec.n_kv_heads
    heads = list(range(spec.n_q_heads)) if q_heads is None else list(q_heads)
    out = np.full(ci.q.shape, np.nan)
    for i in range(spec.n_seq):
        L = int(ci.seq_len[i])
        k = H.seq_rows(ci, i, "k")[:L].transpose(1, 0, 2)
        v = H.seq_rows(ci, i, "v")[:L].transpose(1, 0, 2)
        kvs = sorted({h // G for h in heads})
        vp, vd = O.encode_v(v[kvs], spec.v_format)
        kb = O.half_bits(k[kvs])
        for j, kvh in enumerate(kvs):
            qsub = ci.q[i:i + 1][:, :, kvh * G:(kvh + 1) * G]
            o = O.decode_attention_f16k(qsub, kb[None, j:j + 1], vp[None, j:j + 1], vd[None, j:j + 1],
                                        spec.v_format, ci.seq_len[i:i + 1], spec.sm_scale,
                                        spec.causal)
            for h in heads:
                if h // G == kvh:
                    out[i, :, h] = o[0, :, h - kvh * G]
    return out


def run_f16k(cache, ci, table):
    spec = ci.spec
    q = H.dev(ci.q)
    out = torch.empty_like(q)
    mx = int(ci.seq_len.max())
    ws = torch.zeros(max(16, K.attn_decode_f16k_workspace_size(cache, spec.n_seq, spec.n_qtok,
                                                               spec.n_q_heads, mx)),
                     dtype=torch.uint8, device="cuda")
    K.attn_decode_f16k(cache, q, out, H.dev(ci.seq_len), mx, spec.sm_scale, spec.causal, ws,
                       seg_table=table)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "gqa8k"])
def test_f16k_workloads(name):
    for ci in W.make_inputs(name):
        _say(f"f16k {ci.spec.name}")
        cache, table = build_f16k(ci)
        check_rows(cache, ci)
        H.assert_close(run_f16k(cache, ci, table), oracle_f16k(ci), "f16k " + ci.spec.name)


@pytest.mark.parametrize("G,Tq,causal,L,fmt", [(2, 2, True, 700, 0), (4, 1, False, 33, 1),
                                               (1, 4, True, 4099, 0), (1, 1, False, 1, 0)])
def test_f16k_shapes(G, Tq, causal, L, fmt):
    rng = np.random.default_rng(G * 100 + Tq * 10 + L + fmt)
    Hkv, D = 2, 128
    spec = W.CacheSpec("f16k", 1, Tq, G * Hkv, Hkv, D, L, fmt, causal=causal)
    cap = -(-L // 64) * 64 + 64
    ci = W.CacheInputs(spec, rng.standard_normal((1, Tq, G * Hkv, D)).astype(np.float32),
                       (rng.standard_normal((1, L, Hkv, D)) * 2).astype(np.float32),
                       rng.standard_normal((1, L, Hkv, D)).astype(np.float32),
                       np.array([L], np.int32), None, 1, cap)
    _say(f"f16k G{G} Tq{Tq} causal{causal} L{L} f{fmt}")
    cache, table = build_f16k(ci)
    check_rows(cache, ci)
    H.assert_close(run_f16k(cache, ci, table), oracle_f16k(ci), f"f16k G{G} Tq{Tq} L{L}")


def test_f16k_long128k():
    """The long-context cache at full size with fp16 K; the oracle checks the
    query heads of kv heads 0 and 5."""
    ci = W.make_inputs("long128k")[0]
    _say("f16k long128k")
    cache, table = build_f16k(ci)
    heads = [h for h in range(ci.spec.n_q_heads) if h // 4 in (0, 5)]
    H.assert_close(run_f16k(cache, ci, table), oracle_f16k(ci, heads), "f16k long128k")
