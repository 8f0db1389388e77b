"""Synthetic fidelity report: what the packed formats cost in accuracy.

TEST AND REPORTING INFRASTRUCTURE ONLY, like the rest of oracle/: nothing in
the product path imports it.

Page 1 ("Flash Attention for llama.cpp on RDNA3 ... Part 1", its KLD tables)
measures the end-to-end effect of int8 K with q4_0 or q8_0 V as the KL
divergence of a model's token distributions over a text corpus.  Without a
model or a corpus, this report measures the kernel-level errors those come
from, on inputs with the shapes and value structure of the decode workloads
(workloads.py), everything in float64 from the fp32 inputs:

* Q.K variants: exact (fp32 inputs), "f16" (Q and K rounded to binary16, the
  unpacked-K baseline page 1 compares against) and "int8" (the method: Q and
  K through the block quantizers of kvq_oracle).
* V variants: exact, q8_0, q4_0 (kvq_oracle's encoders, then dequantized).
* Attention weights: KL(p_exact || p_variant) per query row, in nats, and
  the largest |p_exact - p_variant|.
* Output: relative L2 error of each (Q.K, V) combination against the exact
  output, over all query rows of a workload.
"""
from __future__ import annotations

import argparse

import numpy as np

from oracle import kvq_oracle as O

QK_VARIANTS = ("exact", "f16", "int8")
V_VARIANTS = ("exact", "q8_0", "q4_0")


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=1, keepdims=True)


def qk_operands(q: np.ndarray, k: np.ndarray, variant: str):
    """(q_hat [R, D], k_hat [L, D]) float64 for one Q.K variant; q, k fp32."""
    if variant == "exact":
        return q.astype(np.float64), k.astype(np.float64)
    if variant == "f16":
        return (O.half_value(O.half_bits(q)).astype(np.float64),
                O.half_value(O.half_bits(k)).astype(np.float64))
    if variant == "int8":
        qc, qd = O.quantize_q(q)
        kw, kd = O.encode_k(k)
        return O.dequant_q(qc, qd), O.dequant_k(kw, kd)
    raise ValueError(variant)


def v_operand(v: np.ndarray, variant: str) -> np.ndarray:
    if variant == "exact":
        return v.astype(np.float64)
    fmt = O.V_Q8_0 if variant == "q8_0" else O.V_Q4_0
    payload, d = O.encode_v(v, fmt)
    return O.dequant_v(payload, d, fmt)


def group_report(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float) -> dict:
    """All variants for one kv head: q [R, D] (its query rows), k and v
    [L, D], every row seeing all L tokens.  Returns per-variant weights and
    outputs plus the exact ones."""
    weights = {}
    for qv in QK_VARIANTS:
        qh, kh = qk_operands(q, k, qv)
        weights[qv] = _softmax_rows((qh @ kh.T) * float(sm_scale))
    vs = {vv: v_operand(v, vv) for vv in V_VARIANTS}
    outs = {(qv, vv): weights[qv] @ vs[vv] for qv in QK_VARIANTS for vv in V_VARIANTS}
    return {"weights": weights, "outs": outs}


def kl_rows(p: np.ndarray, r: np.ndarray) -> np.ndarray:
    """KL(p || r) per row in nats; terms with p = 0 contribute 0."""
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, p * (np.log(p) - np.log(r)), 0.0)
    return t.sum(axis=1)


def workload_report(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
                    kv_heads=None) -> dict:
    """q [Tq][Hq][D], k and v [L][Hkv][D] of one sequence (fp32).  Aggregates
    over the chosen kv heads (all by default)."""
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    heads = range(Hkv) if kv_heads is None else kv_heads
    kl = {qv: [] for qv in QK_VARIANTS[1:]}
    dp = {qv: 0.0 for qv in QK_VARIANTS[1:]}
    num = {key: 0.0 for key in ((a, b) for a in QK_VARIANTS for b in V_VARIANTS)}
    den = 0.0
    for h in heads:
        qr = q[:, h * G:(h + 1) * G, :].reshape(Tq * G, D)
        g = group_report(qr, k[:, h, :], v[:, h, :], sm_scale)
        pe = g["weights"]["exact"]
        for qv in QK_VARIANTS[1:]:
            kl[qv].append(kl_rows(pe, g["weights"][qv]))
            dp[qv] = max(dp[qv], float(np.abs(pe - g["weights"][qv]).max()))
        oe = g["outs"][("exact", "exact")]
        den += float(np.sum(oe * oe))
        for key, o in g["outs"].items():
            num[key] += float(np.sum((o - oe) ** 2))
    rel = {key: np.sqrt(val / den) for key, val in num.items()}
    kls = {qv: np.concatenate(v_) for qv, v_ in kl.items()}
    return {"kl_mean": {qv: float(x.mean()) for qv, x in kls.items()},
            "kl_max": {qv: float(x.max()) for qv, x in kls.items()},
            "max_dp": dp, "rel_l2": rel}


def output_error(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float, out: np.ndarray,
                 kv_heads=None) -> float:
    """Relative L2 error of a given attention output `out` [Tq][Hq][D] (for
    example a GPU kernel's) against the exact attention of the unquantized
    fp32 inputs q [Tq][Hq][D], k and v [L][Hkv][D], over the query heads of
    the chosen kv heads (all by default), every row seeing all L tokens: the
    same denominator as workload_report's output columns."""
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    heads = range(Hkv) if kv_heads is None else kv_heads
    num = den = 0.0
    for h in heads:
        qr = q[:, h * G:(h + 1) * G, :].reshape(Tq * G, D).astype(np.float64)
        w = _softmax_rows((qr @ k[:, h, :].astype(np.float64).T) * float(sm_scale))
        oe = w @ v[:, h, :].astype(np.float64)
        o = np.asarray(out[:, h * G:(h + 1) * G, :], dtype=np.float64).reshape(Tq * G, D)
        num += float(np.sum((o - oe) ** 2))
        den += float(np.sum(oe * oe))
    return float(np.sqrt(num / den))


def _workloads_module():
    """The seeded input generators, loaded from their file so that the
    library package (and its HIP binding) is not imported."""
    import importlib.util
    import os
    import sys
    name = "kvq_workloads_inputs"
    if name in sys.modules:
        return sys.modules[name]
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "decode_attention_packed_amd", "workloads.py")
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


def _inputs(name: str, ctx: int | None):
    W = _workloads_module()
    out = []
    for ci in W.make_inputs(name, ctx=ctx)[:1]:   # the caches of gqa8k share their inputs
        L = int(ci.seq_len[0])
        k = ci.k[0][:L] if not isinstance(ci.k, list) else ci.k[0]
        v = ci.v[0][:L] if not isinstance(ci.v, list) else ci.v[0]
        out.append((ci.spec.name, ci.q[0], k, v, ci.spec.sm_scale))
    return out


def markdown(results) -> str:
    lines = ["| inputs | Q.K | KL(p_exact ‖ p) mean / max, nats | max \\|Δp\\| | out rel-L2, V exact | V q8_0 | V q4_0 |",
             "|---|---|---|---|---|---|---|"]
    for name, r in results:
        for qv in QK_VARIANTS:
            kl = "—" if qv == "exact" else f"{r['kl_mean'][qv]:.2e} / {r['kl_max'][qv]:.2e}"
            dp = "—" if qv == "exact" else f"{r['max_dp'][qv]:.2e}"
            cells = [f"{r['rel_l2'][(qv, vv)]:.2e}" for vv in V_VARIANTS]
            lines.append(f"| {name} | {qv} | {kl} | {dp} | " + " | ".join(cells) + " |")
    return "\n".join(lines) + "\n"


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workloads", nargs="+", default=["gqa8k", "long128k"])
    ap.add_argument("--ctx", type=int, default=None, help="override the context length")
    ap.add_argument("--kv-heads", type=int, default=None, help="first N kv heads only")
    a = ap.parse_args()
    results = []
    for w in a.workloads:
        for name, q, k, v, sc in _inputs(w, a.ctx):
            heads = None if a.kv_heads is None else range(a.kv_heads)
            results.append((f"{w} ({k.shape[0]} tokens)", workload_report(q, k, v, sc, heads)))
            print(f"[fidelity] {name} done", flush=True)
    print(markdown(results))


if __name__ == "__main__":
    main()
