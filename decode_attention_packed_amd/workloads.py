"""Seeded synthetic workloads (inputs only; none of the method's arithmetic).

Five decode workloads, each drawn from numpy's PCG64 with a fixed seed;
the seed is split with SeedSequence.spawn so Q, K, V and auxiliary draws are
independent streams.  All values are fp32 N(0, 1) unless stated.

  tiny        1 sequence, 1 query token, 4 query / 1 kv heads, head_dim 128,
              512 tokens, V q4_0, scale 1/sqrt(128)
  gqa8k       1 sequence, 1 query token, 32/8 heads, head_dim 128, 8192 tokens,
              V q4_0 and q8_0; 1% of token positions (82, shared by all kv
              heads) have their K rows multiplied by 8 before quantization
  long128k    1 sequence, 1 query token, 32/8 heads, head_dim 128, 131072
              tokens, V q4_0; K channel (kv head, dim) scaled by a std drawn
              U(0.5, 2); each step appends one token at position 131071
  verify128k  two caches per step: main 32/8 heads and draft 16/4 heads,
              head_dim 128, 131072 tokens, 4 query tokens each under a causal
              mask over the last 4 positions, V q4_0
  ragged      16 sequences, 1 query token, 32/32 heads, head_dim 64, V q8_0;
              lengths round(exp(U(ln 256, ln 32768))) clamped to [256, 32768];
              KV in append-only segments of 4096 tokens whose ids come from a
              shuffled pool, so a sequence's segments are scattered

Arrays come out in the append order the C ABI takes: K and V are
[n_seq][n_tokens][n_kv_heads][head_dim] float32, Q is
[n_seq][n_qtok][n_q_heads][head_dim] float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

V_Q4_0, V_Q8_0 = 0, 1


@dataclass
class CacheSpec:
    name: str
    n_seq: int
    n_qtok: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx: int                 # tokens per sequence (max for ragged)
    v_format: int
    causal: bool = False
    seg_tokens: int = 0      # 0: one contiguous segment per sequence

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass
class Workload:
    name: str
    seed: int
    caches: list = field(default_factory=list)
    append_per_step: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", 1, [CacheSpec("tiny", 1, 1, 4, 1, 128, 512, V_Q4_0)]),
    "gqa8k": Workload("gqa8k", 2, [CacheSpec("gqa8k_q4_0", 1, 1, 32, 8, 128, 8192, V_Q4_0),
                                   CacheSpec("gqa8k_q8_0", 1, 1, 32, 8, 128, 8192, V_Q8_0)]),
    "long128k": Workload("long128k", 3, [CacheSpec("long128k", 1, 1, 32, 8, 128, 131072, V_Q4_0)],
                         append_per_step=1),
    "verify128k": Workload("verify128k", 4,
                           [CacheSpec("main", 1, 4, 32, 8, 128, 131072, V_Q4_0, causal=True),
                            CacheSpec("draft", 1, 4, 16, 4, 128, 131072, V_Q4_0, causal=True)]),
    "ragged": Workload("ragged", 5, [CacheSpec("ragged", 16, 1, 32, 32, 64, 32768, V_Q8_0,
                                               seg_tokens=4096)]),
}


@dataclass
class CacheInputs:
    spec: CacheSpec
    q: np.ndarray            # [S][Tq][Hq][D]
    k: np.ndarray            # [S][L][Hkv][D]; ragged: a list of [L_i][Hkv][D]
    v: np.ndarray
    seq_len: np.ndarray      # int32 [S]
    seg_table: np.ndarray | None = None   # int32 [S][max_segs]
    n_segs: int = 0
    seg_tokens: int = 0
    extra: dict = field(default_factory=dict)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def ragged_lengths(rng, n, lo=256, hi=32768):
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)


def make_inputs(name: str, ctx: int | None = None) -> list:
    """Inputs for every cache of workload `name`.  `ctx` overrides the
    context length (same recipe at a smaller size, for quick tests)."""
    wl = WORKLOADS[name]
    streams = np.random.SeedSequence(wl.seed).spawn(4 * len(wl.caches))
    out = []
    for ci, spec in enumerate(wl.caches):
        # the two gqa8k caches differ only in the V format: same draws
        si = 0 if name == "gqa8k" else ci
        rq, rk, rv, ra = (np.random.Generator(np.random.PCG64(s)) for s in streams[4 * si:4 * si + 4])
        L = spec.ctx if ctx is None else ctx
        S, Hkv, D = spec.n_seq, spec.n_kv_heads, spec.head_dim
        q = _normal(rq, (S, spec.n_qtok, spec.n_q_heads, D))
        if name == "ragged":
            lens = ragged_lengths(ra, S, hi=L) if ctx is None else ragged_lengths(ra, S, lo=min(256, L), hi=L)
            lmax = int(lens.max())
            k = [_normal(rk, (int(n), Hkv, D)) for n in lens]
            v = [_normal(rv, (int(n), Hkv, D)) for n in lens]
            seg = spec.seg_tokens
            nseg_each = (lens + seg - 1) // seg
            n_segs = int(nseg_each.sum())
            pool = ra.permutation(n_segs).astype(np.int32)
            max_segs = int((lmax + seg - 1) // seg)
            table = np.full((S, max_segs), -1, np.int32)
            pos = 0
            for i in range(S):
                table[i, :nseg_each[i]] = pool[pos:pos + nseg_each[i]]
                pos += nseg_each[i]
            out.append(CacheInputs(spec, q, k, v, lens, table, n_segs, seg))
            continue
        k = _normal(rk, (S, L, Hkv, D))
        v = _normal(rv, (S, L, Hkv, D))
        extra = {}
        if name == "gqa8k":
            n_out = int(round(0.01 * L))
            rows = ra.choice(L, size=n_out, replace=False)
            k[:, rows] *= np.float32(8.0)
            extra["outlier_rows"] = np.sort(rows)
        if name == "long128k":
            std = ra.uniform(0.5, 2.0, size=(Hkv, D)).astype(np.float32)
            k *= std[None, None]
            extra["channel_std"] = std
            extra["append_k"] = _normal(rk, (S, 1, Hkv, D)) * std[None, None]
            extra["append_v"] = _normal(rv, (S, 1, Hkv, D))
        seq_len = np.full(S, L, np.int32)
        seg_tokens = -(-L // 64) * 64     # one segment per sequence, rows padded to 64
        out.append(CacheInputs(spec, q, k, v, seq_len, None, S, seg_tokens, extra))
    return out
