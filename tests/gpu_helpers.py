"""Helpers for the GPU parity tests: build packed caches on the GPU through
the C ABI, build the oracle's own encoding of the same fp32 inputs, and
read GPU cache planes back into per-sequence token order."""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_packed_amd as K
from decode_attention_packed_amd.workloads import CacheInputs
from oracle import kvq_oracle as O

ATOL = 2e-3      # max |gpu - oracle| over the output of one call
RTOL_L2 = 1e-3   # ||gpu - oracle||_2 / ||oracle||_2 over the output of one call


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def seq_rows(ci: CacheInputs, i: int, which: str):
    arr = ci.k if which == "k" else ci.v
    if isinstance(arr, list):
        return arr[i]
    return arr[i, :int(ci.seq_len[i])]


def build_cache(ci: CacheInputs, capacity: int | None = None):
    """Allocate a cache for ci and fill it with kv_append_quant (bulk)."""
    spec = ci.spec
    seg_tokens = ci.seg_tokens if capacity is None else capacity
    cache = K.PackedKVCache(spec.n_kv_heads, spec.head_dim, seg_tokens, ci.n_segs, spec.v_format)
    table = None if ci.seg_table is None else dev(ci.seg_table)
    max_segs = ci.seg_table.shape[1] if ci.seg_table is not None else ci.n_segs // spec.n_seq
    for i in range(spec.n_seq):
        kk = dev(seq_rows(ci, i, "k")[None])
        vv = dev(seq_rows(ci, i, "v")[None])
        start = torch.zeros(1, dtype=torch.int32, device="cuda")
        if table is not None:
            K.kv_append_quant(cache, kk, vv, start, seg_table=table[i:i + 1])
        else:
            # sequence i owns segments i*max_segs ...: append through a one-row table
            t = torch.arange(i * max_segs, (i + 1) * max_segs, dtype=torch.int32, device="cuda")[None]
            K.kv_append_quant(cache, kk, vv, start, seg_table=t)
        del kk, vv
    return cache, table, max_segs


def gpu_rows(cache, ci: CacheInputs, i: int, tokens: np.ndarray):
    """Cache rows of sequence i at the given token positions, per kv head:
    (k_qs [Hkv][n][D/4] u32, k_d u16, v_qs u8, v_d u16) as numpy."""
    seg_tokens = cache.seg_tokens
    max_segs = ci.seg_table.shape[1] if ci.seg_table is not None else ci.n_segs // ci.spec.n_seq
    segj = tokens // seg_tokens
    seg = ci.seg_table[i, segj] if ci.seg_table is not None else i * max_segs + segj
    row = torch.from_numpy((tokens - segj * seg_tokens).astype(np.int64)).cuda()
    segt = torch.from_numpy(seg.astype(np.int64)).cuda()
    ntile = seg_tokens // 32
    tile = torch.from_numpy((tokens - segj * seg_tokens).astype(np.int64) // 32).cuda()
    slot = torch.from_numpy((tokens - segj * seg_tokens).astype(np.int64) % 32).cuda()
    out = []
    x = cache.k_qs[segt, :, row]                   # K codes: token-major rows, [n][Hkv][...]
    out.append(x.permute(1, 0, 2).contiguous().cpu().numpy())
    for plane in (cache.k_d, cache.v_qs, cache.v_d):   # 32-token tiles, [row byte][token]
        s_, h_, _, w_ = plane.shape
        t5 = plane.view(s_, h_, ntile, w_, 32)
        x = t5[segt, :, tile, :, slot]             # [n][Hkv][w]
        out.append(x.permute(1, 0, 2).contiguous().cpu().numpy())
    kq, kd, vq, vd = out
    return kq.view(np.uint32), kd.view(np.uint16), vq.view(np.uint8), vd.view(np.uint16)


def oracle_rows(ci: CacheInputs, i: int, tokens: np.ndarray):
    """Oracle encoding of the same rows: (k_qs [Hkv][n][D/4], k_d, v_qs, v_d)."""
    k = seq_rows(ci, i, "k")[tokens].transpose(1, 0, 2)
    v = seq_rows(ci, i, "v")[tokens].transpose(1, 0, 2)
    kw, kd = O.encode_k(k)
    vp, vd = O.encode_v(v, ci.spec.v_format)
    return kw, kd, vp, vd


def oracle_cache_arrays(ci: CacheInputs, i: int, kv_heads=None):
    """Oracle-encoded cache of sequence i as [1][Hkv'][L][...] arrays."""
    k = seq_rows(ci, i, "k")
    v = seq_rows(ci, i, "v")
    if kv_heads is not None:
        k = k[:, kv_heads]
        v = v[:, kv_heads]
    kw, kd = O.encode_k(k.transpose(1, 0, 2))
    vp, vd = O.encode_v(v.transpose(1, 0, 2), ci.spec.v_format)
    return kw[None], kd[None], vp[None], vd[None]


def run_attention(cache, ci: CacheInputs, table, max_segs, q=None, seq_len=None, max_seq_len=None,
                  causal=None):
    spec = ci.spec
    q = dev(ci.q) if q is None else q
    sl = dev(ci.seq_len) if seq_len is None else seq_len
    mx = int(ci.seq_len.max()) if max_seq_len is None else max_seq_len
    causal = spec.causal if causal is None else causal
    out = torch.empty_like(q)
    n_seq, n_qtok, n_q_heads, _ = q.shape
    ws_bytes = K.attn_decode_packed_workspace_size(cache, n_seq, n_qtok, n_q_heads, mx)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    if table is None:
        table = torch.stack([torch.arange(i * max_segs, (i + 1) * max_segs, dtype=torch.int32)
                             for i in range(n_seq)]).cuda()
    K.attn_decode_packed(cache, q, out, sl, mx, spec.sm_scale, causal, ws, seg_table=table)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_attention(ci: CacheInputs, q_heads=None):
    """Oracle output [S][Tq][Hq][D] (NaN outside q_heads) from fp32 inputs."""
    spec = ci.spec
    G = spec.n_q_heads // spec.n_kv_heads
    out = np.full(ci.q.shape, np.nan)
    heads = list(range(spec.n_q_heads)) if q_heads is None else list(q_heads)
    kvs = sorted({h // G for h in heads})
    for i in range(spec.n_seq):
        kw, kd, vp, vd = oracle_cache_arrays(ci, i, kvs)
        # remap the selected kv heads to 0..len(kvs)-1 and their query heads
        for j, kvh in enumerate(kvs):
            hs = [h for h in heads if h // G == kvh]
            qsub = ci.q[i:i + 1][:, :, kvh * G:(kvh + 1) * G]
            o = O.decode_attention(qsub, kw[:, j:j + 1], kd[:, j:j + 1], vp[:, j:j + 1],
                                   vd[:, j:j + 1], spec.v_format, ci.seq_len[i:i + 1],
                                   spec.sm_scale, spec.causal)
            for h in hs:
                out[i, :, h] = o[0, :, h - kvh * G]
    return out


def assert_close(gpu, ref, what=""):
    mask = ~np.isnan(ref)
    g = gpu[mask].astype(np.float64)
    r = ref[mask]
    err = np.abs(g - r)
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    print(f"[parity] {what}: max_abs={err.max():.3e} rel_l2={rel:.3e} n={r.size}", flush=True)
    assert np.all(np.isfinite(g)), what
    assert err.max() <= ATOL, (what, err.max())
    assert rel <= RTOL_L2, (what, rel)
    return err.max(), rel
