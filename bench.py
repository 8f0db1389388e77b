"""Decode-attention benchmark on one MI355X.

A step is one pass of the whole hot path on the 128k-context workload
(1 sequence, 32 query / 8 kv heads, head_dim 128, 131072 tokens, int8 K
packed 4 per word with fp16 scales, q4_0 V): one new token is quantized and
packed at position 131071 and attention runs over all 131072 tokens, in one
launch of attn_decode_packed_append (the same work as kv_append_quant
followed by attn_decode_packed, which is timed too, as "two_launch").
Inputs are seeded synthetic data resident in HBM before timing.
Steps rotate over R cache replicas (default 3, 654 MB) so the 256 MB
Infinity Cache cannot hold the working set between reuses.

Prints one JSON line: value = algorithmic KV bytes per step / time per step
(GB/s), with ms and us per step, the roofline of the attention kernel and
the oracle timed on the host.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "decode_attention_packed_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_long128k.txt")
CALIB_BYTES = 256 << 20   # known sizes read / written by the calibration kernels
ATTN_KERNEL = "kvq::w12::k_attn_cols<128, 0>"   # the 12-wave build that runs the step


def kernel_source_hash() -> str:
    """sha256 over the kernel sources: a traffic summary is only valid for
    the sources it was measured on."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def read_traffic() -> int | None:
    """Calibrated HBM bytes per attention launch from the committed counter
    summary, or None when it is missing or stale."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return int(float(kv["attn_traffic_bytes"]))
    except (OSError, KeyError, ValueError):
        return None


def _counter_rows(d: str, counter: str) -> dict:
    """Per-kernel lists of one counter's per-dispatch values from a
    rocprofv3 --pmc output directory."""
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") == counter:
                    out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def summarize_pmc(fetch_dir: str, write_dir: str, fetch_cmd: str, write_cmd: str) -> str:
    """Turn the FETCH_SIZE and WRITE_SIZE runs (of `bench.py --calibrate`)
    into the traffic summary: each counter is scaled by what it reads for a
    kernel of known size (the library's stream-read kernel over CALIB_BYTES
    for fetches, a device copy of CALIB_BYTES for writes)."""
    fetch = _counter_rows(fetch_dir, "FETCH_SIZE")
    write = _counter_rows(write_dir, "WRITE_SIZE")

    def pick(d, key):
        return [v for k, vs in d.items() if key in k for v in vs]

    def med(vals, what):
        if not vals:
            raise SystemExit(f"no dispatches of {what} in the counter output")
        return float(np.median(vals)), len(vals)

    # in a --calibrate run every stream read covers CALIB_BYTES; the same
    # counter must then agree across them
    rd = pick(fetch, "k_debug_stream_read")
    if rd and max(rd) > 1.05 * min(rd):
        raise SystemExit("stream-read dispatches of different sizes: use a --calibrate run")
    rd_kib, n_rd = med(rd, "k_debug_stream_read")
    # the calibration copies are the large ones; the small copies are input uploads
    cp = pick(write, "copyBuffer")
    cp = [v for v in cp if v >= 0.5 * max(cp)] if cp else cp
    cp_kib, n_cp = med(cp, "the calibration copy")
    at_f, n_af = med(pick(fetch, ATTN_KERNEL), ATTN_KERNEL)
    at_w, n_aw = med(pick(write, ATTN_KERNEL), ATTN_KERNEL)
    ffac = CALIB_BYTES / (rd_kib * 1024)
    wfac = CALIB_BYTES / (cp_kib * 1024)
    fb = at_f * 1024 * ffac
    wb = at_w * 1024 * wfac
    from decode_attention_packed_amd import workloads as W
    alg = algorithmic_bytes(W.WORKLOADS["long128k"].caches[0], 131072, 1)["step"]
    lines = [
        "# HBM traffic of one launch of the step kernel (append one token + attention) on the",
        "# long128k workload, from rocprofv3",
        "# counters (KiB per dispatch, medians), each scaled by the same counter read",
        f"# for a kernel of known size ({CALIB_BYTES} bytes read / written).",
        f"# fetch run: {fetch_cmd}",
        f"# write run: {write_cmd}",
        f"kernel_source_sha256 = {kernel_source_hash()}",
        f"calib_read_fetch_kib = {rd_kib:.1f}   # k_debug_stream_read, {n_rd} dispatches",
        f"calib_copy_write_kib = {cp_kib:.1f}   # device copy, {n_cp} dispatches",
        f"fetch_factor = {ffac:.4f}",
        f"write_factor = {wfac:.4f}",
        f"attn_fetch_kib = {at_f:.1f}   # {ATTN_KERNEL}, {n_af} dispatches",
        f"attn_write_kib = {at_w:.1f}   # {n_aw} dispatches",
        f"attn_fetch_bytes = {fb:.0f}",
        f"attn_write_bytes = {wb:.0f}",
        f"attn_traffic_bytes = {fb + wb:.0f}",
        f"algorithmic_bytes = {alg}",
        f"traffic_over_algorithmic = {(fb + wb) / alg:.4f}",
    ]
    return "\n".join(lines) + "\n"


def summarize_trace(trace_dir: str, cmd: str, steps: int, warmup: int) -> str:
    """Per-kernel statistics of a `rocprofv3 --kernel-trace --stats` run of
    this benchmark, with the attention kernel's durations split by bench
    phase (cold rotating replicas, per-step events, warm single replica)."""
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    lines = ["# Kernel durations of the long128k decode step (bench.py) from rocprofv3.",
             f"# command: {cmd}",
             "# kernel | calls | average us | min us | max us"]
    with open(stats[0]) as fh:
        for row in csv.DictReader(fh):
            lines.append(f"{row['Name'][:90]} | {row['Calls']} | {float(row['AverageNs']) / 1e3:.2f} | "
                         f"{float(row['MinNs']) / 1e3:.2f} | {float(row['MaxNs']) / 1e3:.2f}")
    with open(trace[0]) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
    att = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
           for r in rows if ATTN_KERNEL in r["Kernel_Name"]]
    # bench order: warmup, timed steps, the two-launch form (warmup, steps),
    # per-step events, warm warmup, warm steps
    phases = [("cold warmup", warmup), ("cold timed steps", steps), ("two-launch warmup", warmup),
              ("two-launch steps", steps), ("cold per-step events", steps), ("warm warmup", warmup),
              ("warm single replica", steps)]
    lines.append(f"# {ATTN_KERNEL} by bench phase: phase | dispatches | average us | median us")
    i = 0
    for name, n in phases:
        seg = np.array(att[i:i + n])
        i += n
        if seg.size:
            lines.append(f"{name} | {seg.size} | {seg.mean():.2f} | {np.median(seg):.2f}")
    return "\n".join(lines) + "\n"


def algorithmic_bytes(spec, n_tokens: int, append_rows: int) -> dict:
    """K payload + K scales + V payload + V scales of every attended
    (token, kv head), plus the packed bytes written by the append."""
    D = spec.head_dim
    nb = D // 32
    kb = D + 2 * nb
    vb = (D // 2 if spec.v_format == 0 else D) + 2 * nb
    attn = n_tokens * spec.n_kv_heads * (kb + vb)
    app = append_rows * spec.n_kv_heads * (kb + vb)
    return {"attn": attn, "append": app, "step": attn + app, "per_token_head": kb + vb}


def _build_cache(K, torch, ci):
    """One packed cache holding every sequence of `ci`, filled by bulk
    kv_append_quant through each sequence's segment list.  Returns the cache
    and the segment table the attention calls take: the workload's own for
    segmented caches, None for contiguous ones (one segment per sequence,
    the table-free form of the ABI)."""
    spec = ci.spec
    cache = K.PackedKVCache(spec.n_kv_heads, spec.head_dim, ci.seg_tokens, ci.n_segs, spec.v_format)
    if ci.seg_table is not None:
        table = torch.from_numpy(ci.seg_table).cuda()
    else:
        per = ci.n_segs // spec.n_seq
        table = torch.arange(ci.n_segs, dtype=torch.int32).view(spec.n_seq, per).cuda()
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(spec.n_seq):
        n = int(ci.seq_len[i])
        k = ci.k[i] if isinstance(ci.k, list) else ci.k[i, :n]
        v = ci.v[i] if isinstance(ci.v, list) else ci.v[i, :n]
        K.kv_append_quant(cache, torch.from_numpy(np.ascontiguousarray(k[None])).cuda(),
                          torch.from_numpy(np.ascontiguousarray(v[None])).cuda(), zero,
                          seg_table=table[i:i + 1])
    return cache, (table if ci.seg_table is not None else None)


def other_configs(K, W, torch, stream, steps: int, warmup: int) -> list:
    """The other workloads, each step the attention calls its recipe
    defines (no append): tiny, gqa8k in both V formats, the verify step
    (main and draft caches, two calls on one stream) and the ragged batch.
    Enough cache replicas rotate that one pass touches more than the 256 MB
    Infinity Cache, except for tiny (106 KB), which is latency-bound."""
    rows = []
    plans = [("tiny", ["tiny"], 1), ("gqa8k_q4_0", ["gqa8k_q4_0"], 24), ("gqa8k_q8_0", ["gqa8k_q8_0"], 18),
             ("verify128k", ["main", "draft"], 2), ("ragged", ["ragged"], 2)]
    inputs = {}
    for wl in ("tiny", "gqa8k", "verify128k", "ragged"):
        for ci in W.make_inputs(wl):
            inputs[ci.spec.name] = ci
    for label, names, reps in plans:
        calls = []
        nbytes = 0
        for nm in names:
            ci = inputs[nm]
            spec = ci.spec
            built = [_build_cache(K, torch, ci) for _ in range(reps)]
            q = torch.from_numpy(ci.q).cuda()
            out = torch.empty_like(q)
            sl = torch.from_numpy(ci.seq_len).cuda()
            mx = int(ci.seq_len.max())
            ws = torch.zeros(max(16, K.attn_decode_packed_workspace_size(
                built[0][0], spec.n_seq, spec.n_qtok, spec.n_q_heads, mx)), dtype=torch.uint8,
                device="cuda")
            calls.append((built, q, out, sl, mx, spec, ws))
            per = algorithmic_bytes(spec, 1, 0)["per_token_head"]
            nbytes += int(ci.seq_len.astype(np.int64).sum()) * spec.n_kv_heads * per
        torch.cuda.synchronize()

        def run(i):
            for built, q, out, sl, mx, spec, ws in calls:
                cache, table = built[i % len(built)]
                K.attn_decode_packed(cache, q, out, sl, mx, spec.sm_scale, spec.causal, ws,
                                     seg_table=table, stream=stream)
        for i in range(warmup):
            run(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        rows.append({"workload": label, "us_per_step": round(ms * 1e3, 2), "kv_bytes_per_step": nbytes,
                     "gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                     "launches_per_step": len(names), "replicas": reps})
        print(f"[bench] {label}: {ms * 1e3:.2f} us/step, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
        if len(calls) > 1:
            # the same calls as one attn_decode_packed_batch launch
            def batch_args(i):
                return [dict(cache=built[i % len(built)][0], q=q, out=out, seq_len=sl, max_seq_len=mx,
                             sm_scale=spec.sm_scale, causal=spec.causal, seg_table=built[i % len(built)][1])
                        for built, q, out, sl, mx, spec, _ in calls]
            bws = torch.zeros(K.attn_decode_packed_batch_workspace_size(batch_args(0)), dtype=torch.uint8,
                              device="cuda")
            args_r = [batch_args(i) for i in range(reps)]
            for i in range(warmup):
                K.attn_decode_packed_batch(args_r[i % reps], bws, stream=stream)
            e0.record(stream)
            for i in range(steps):
                K.attn_decode_packed_batch(args_r[i % reps], bws, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            gbs = nbytes / (ms * 1e-3) / 1e9
            rows.append({"workload": label + " (one batched launch)", "us_per_step": round(ms * 1e3, 2),
                         "kv_bytes_per_step": nbytes, "gbs": round(gbs, 1),
                         "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "launches_per_step": 1,
                         "replicas": reps})
            print(f"[bench] {label} batched: {ms * 1e3:.2f} us/step, {gbs:.0f} GB/s", file=sys.stderr,
                  flush=True)
        del calls
        torch.cuda.empty_cache()
    return rows


def ab_f16k(K, torch, stream, ci, caches, steps: int, warmup: int) -> dict:
    """Page 1's comparison on this hardware: attention alone over the same
    long128k inputs with the packed int8 K (the method) and with K kept as
    fp16 rows (attn_decode_f16k), both with q4_0 V and rotating replicas.  If
    the time follows the bytes, the time ratio equals the byte ratio."""
    spec = ci.spec
    L = spec.ctx
    f16 = []
    for _ in range(len(caches)):
        c = K.F16KCache(spec.n_kv_heads, spec.head_dim, ci.seg_tokens, 1, spec.v_format)
        K.kv_append_f16k(c, torch.from_numpy(ci.k).cuda(), torch.from_numpy(ci.v).cuda(),
                         torch.zeros(1, dtype=torch.int32, device="cuda"))
        f16.append(c)
    torch.cuda.synchronize()
    q = torch.from_numpy(ci.q).cuda()
    out = torch.empty_like(q)
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(K.attn_decode_packed_workspace_size(caches[0], 1, 1, spec.n_q_heads, L),
                         K.attn_decode_f16k_workspace_size(f16[0], 1, 1, spec.n_q_heads, L)),
                     dtype=torch.uint8, device="cuda")
    runs = {"packed_int8_k": (caches, K.attn_decode_packed), "fp16_k": (f16, K.attn_decode_f16k)}
    res = {}
    for name, (cs, fn) in runs.items():
        for i in range(warmup):
            fn(cs[i % len(cs)], q, out, sl, L, spec.sm_scale, False, ws, stream=stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(cs[i % len(cs)], q, out, sl, L, spec.sm_scale, False, ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        per = (2 * spec.head_dim if name == "fp16_k" else algorithmic_bytes(spec, 1, 0)["per_token_head"]
               - (spec.head_dim // 2 + 2 * (spec.head_dim // 32)))
        kvb = L * spec.n_kv_heads * (per + spec.head_dim // 2 + 2 * (spec.head_dim // 32))
        res[name] = {"us": round(us, 2), "kv_bytes": kvb, "gbs": round(kvb / us / 1e3, 1),
                     "pct_hbm_peak": round(100 * kvb / us / 1e3 / HBM_PEAK_GBS, 1)}
    res["byte_ratio"] = round(res["fp16_k"]["kv_bytes"] / res["packed_int8_k"]["kv_bytes"], 3)
    res["time_ratio"] = round(res["fp16_k"]["us"] / res["packed_int8_k"]["us"], 3)
    res["note"] = ("attention only; fp16 K: 6 waves x 2 ring slots (its 8 KB K tiles), "
                   "Q rounded to fp16, f16 MFMA for Q.K")
    print(f"[bench] A/B fp16 K: {res['fp16_k']['us']} us vs packed {res['packed_int8_k']['us']} us "
          f"(time x{res['time_ratio']}, bytes x{res['byte_ratio']})", file=sys.stderr, flush=True)
    del f16
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_step(O, ci, kw, kd, vp, vd, kv_heads):
    """One step of the oracle restricted to some kv heads: quantize the new
    token's rows into the packed cache, then attention over all tokens for
    the query heads of those kv heads (the oracle's own per-kv-head loop)."""
    spec = ci.spec
    L = spec.ctx
    G = spec.n_q_heads // spec.n_kv_heads
    for kvh in kv_heads:
        nk, nkd = O.encode_k(ci.extra["append_k"][0, 0, kvh])
        nv, nvd = O.encode_v(ci.extra["append_v"][0, 0, kvh], spec.v_format)
        kw[kvh, L - 1], kd[kvh, L - 1], vp[kvh, L - 1], vd[kvh, L - 1] = nk, nkd, nv, nvd
        O.decode_attention(ci.q[:, :, kvh * G:(kvh + 1) * G], kw[None, kvh:kvh + 1],
                           kd[None, kvh:kvh + 1], vp[None, kvh:kvh + 1], vd[None, kvh:kvh + 1],
                           spec.v_format, ci.seq_len, spec.sm_scale, False)


def cpu_baseline(ci, target_s: float = 12.0) -> dict:
    """The oracle on the host: the same step (quantize the new token into
    the packed cache, then attention over all tokens from the packed cache),
    repeated for about `target_s` seconds on all the cores this process may
    use (one thread per kv head, the BLAS threads sharing the rest), then for
    about a third of that on one core; reported in the metric's unit."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import kvq_oracle as O
    spec = ci.spec
    L = spec.ctx
    step_bytes = algorithmic_bytes(spec, L, 1)["step"]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    # the packed cache is an input of the step, built outside the timing
    kw, kd = O.encode_k(ci.k[0].transpose(1, 0, 2))
    vp, vd = O.encode_v(ci.v[0].transpose(1, 0, 2), spec.v_format)
    heads = list(range(spec.n_kv_heads))

    def timed(n_workers, blas, budget):
        reps, t_total = 0, 0.0
        with threadpool_limits(limits=blas), ThreadPoolExecutor(n_workers) as ex:
            parts = [heads[w::n_workers] for w in range(n_workers)]
            while t_total < budget:
                t0 = time.perf_counter()
                list(ex.map(lambda hs: _oracle_step(O, ci, kw, kd, vp, vd, hs), parts))
                t_total += time.perf_counter() - t0
                reps += 1
        return reps, t_total

    workers = max(1, min(cores, spec.n_kv_heads))
    reps, t_all = timed(workers, max(1, cores // workers), target_s)
    reps1, t_one = timed(1, 1, target_s / 3)
    s_all, s_one = t_all / reps, t_one / reps1
    return {"value": round(step_bytes / s_all / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "us_per_step": round(s_all * 1e6, 1),
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(),
            "sample": f"{reps} whole long128k steps (append 1 token + attention over 131072 tokens, "
                      f"all 8 kv heads) in {t_all:.1f} s, numpy float64, {workers} threads over kv "
                      f"heads x {max(1, cores // workers)} BLAS threads on the {cores} cores this "
                      f"process may use",
            "one_core": {"value": round(step_bytes / s_one / 1e9, 3), "unit": "GB/s", "cores": 1,
                         "us_per_step": round(s_one * 1e6, 1),
                         "sample": f"{reps1} whole steps in {t_one:.1f} s, one thread, BLAS "
                                   f"limited to 1 thread"}}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the timing of the other workloads (tiny, gqa8k, verify128k, ragged)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run the known-size read and copy kernels (for counter runs)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "CMD"),
                    help="write the kernel-trace summary of a rocprofv3 run of this benchmark and exit")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "FETCH_CMD", "WRITE_CMD"),
                    help="write the traffic summary from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        text = summarize_trace(*args.summarize_trace, args.steps, args.warmup)
        with open(os.path.join(ROOT, "profiles", "attn_kernel_trace_long128k.txt"), "w") as fh:
            fh.write(text)
        print(text, end="")
        return 0
    if args.summarize_pmc:
        text = summarize_pmc(*args.summarize_pmc)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as fh:
            fh.write(text)
        print(text, end="")
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path is not "
                                   "sharded across GPUs", "n_gpus": args.gpus}))
        return 2

    import torch

    import decode_attention_packed_amd as K
    from decode_attention_packed_amd import workloads as W

    torch.cuda.set_device(0)
    ci = W.make_inputs("long128k")[0]
    spec = ci.spec
    L = spec.ctx
    print(f"[bench] inputs ready: {spec.name} L={L}", file=sys.stderr, flush=True)

    caches = []
    for _ in range(args.replicas):
        c = K.PackedKVCache(spec.n_kv_heads, spec.head_dim, ci.seg_tokens, 1, spec.v_format)
        kk = torch.from_numpy(ci.k).cuda()
        vv = torch.from_numpy(ci.v).cuda()
        K.kv_append_quant(c, kk, vv, torch.zeros(1, dtype=torch.int32, device="cuda"))
        del kk, vv
        caches.append(c)
    torch.cuda.synchronize()
    q = torch.from_numpy(ci.q).cuda()
    out = torch.empty_like(q)
    ak = torch.from_numpy(ci.extra["append_k"]).cuda()
    av = torch.from_numpy(ci.extra["append_v"]).cuda()
    pos = torch.tensor([L - 1], dtype=torch.int32, device="cuda")
    seq_len = torch.tensor([L], dtype=torch.int32, device="cuda")
    ws_bytes = K.attn_decode_packed_workspace_size(caches[0], 1, 1, spec.n_q_heads, L)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")   # counters start at zero
    stream = torch.cuda.current_stream()
    print(f"[bench] caches built: {args.replicas} x {caches[0].nbytes / 1e6:.1f} MB", file=sys.stderr,
          flush=True)

    def step(i, ev=None):
        c = caches[i % len(caches)]
        if ev is not None:
            ev[0].record(stream)
        K.attn_decode_packed_append(c, q, ak, av, out, seq_len, L, spec.sm_scale, False, ws,
                                    stream=stream)
        if ev is not None:
            ev[1].record(stream)

    def step_two_launch(i):
        c = caches[i % len(caches)]
        K.kv_append_quant(c, ak, av, pos, stream=stream)
        K.attn_decode_packed(c, q, out, seq_len, L, spec.sm_scale, False, ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps

    # the same step as two launches (kv_append_quant, then attn_decode_packed)
    for i in range(args.warmup):
        step_two_launch(i)
    u0 = torch.cuda.Event(enable_timing=True)
    u1 = torch.cuda.Event(enable_timing=True)
    u0.record(stream)
    for i in range(args.steps):
        step_two_launch(i)
    u1.record(stream)
    torch.cuda.synchronize()
    two_launch_ms = u0.elapsed_time(u1) / args.steps

    # the step's kernel alone, per step, with events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    attn_ms = np.array([a.elapsed_time(b) for a, b in evs])

    # one replica reused every step (with nontemporal K/V loads little of it
    # stays in the 256 MB Infinity Cache)
    for i in range(args.warmup):
        step(0)
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for i in range(args.steps):
        step(0)
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps

    # HBM read ceiling: the library's plain 16-byte streaming read over 1 GiB
    # (skipped in counter runs, whose only reads of that kernel are the
    # known-size calibration ones)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    read_gbs = None
    if not args.calibrate:
        buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            K.kvq_debug_stream_read(buf, sink, stream=stream)
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for _ in range(10):
            K.kvq_debug_stream_read(buf, sink, stream=stream)
        r1.record(stream)
        torch.cuda.synchronize()
        read_gbs = round(buf.numel() / (r0.elapsed_time(r1) / 10 * 1e-3) / 1e9, 1)
        del buf
    else:
        a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            K.kvq_debug_stream_read(a, sink, stream=stream)
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    nbytes = algorithmic_bytes(spec, L, 1)
    gbs = nbytes["step"] / (ms_step * 1e-3) / 1e9
    # The step is one launch, so the kernel's average launch duration is the
    # timed region (events on the launch stream around all K launches) over K.
    # Per-step event pairs (kernel_us) add their own packets between launches
    # and read ~2 us longer; they are kept for the spread.
    achieved = nbytes["step"] / (ms_step * 1e-3) / 1e9
    result = {
        "metric": "decode attention µs/step + KV GB/s (% of HBM peak) at 128k ctx, 1 GPU",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 K x int8 Q block dot (int32), fp32 rescale and softmax, q4_0 V codes as "
                 "exact fp16 with the P.V operand p*d_v rounded once to fp16, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "long128k: 1 seq, 1 query token, 32 q / 8 kv heads, head_dim 128, "
                               "131072 ctx, K int8+fp16 scale packed 4/u32, V q4_0, 1 append/step",
                   "replicas": args.replicas, "kv_bytes_per_step": nbytes["step"],
                   "launches_per_step": 1},
        "two_launch": {"us_per_step": round(two_launch_ms * 1e3, 2),
                       "gbs": round(nbytes["step"] / (two_launch_ms * 1e-3) / 1e9, 1),
                       "note": "kv_append_quant then attn_decode_packed, same work"},
        "kernel_us": {"note": "per-step event pairs around each launch (they add their own gaps)",
                      "mean": round(float(attn_ms.mean()) * 1e3, 2),
                    "p10": round(float(np.percentile(attn_ms, 10)) * 1e3, 2),
                    "p50": round(float(np.percentile(attn_ms, 50)) * 1e3, 2),
                    "p90": round(float(np.percentile(attn_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic()},
        "read_ceiling_gbs": read_gbs,
        "warm_single_replica": {"us_per_step": round(warm_ms * 1e3, 2),
                                "gbs": round(nbytes["step"] / (warm_ms * 1e-3) / 1e9, 1),
                                "note": "one cache replica reused every step; the K/V loads are "
                                        "nontemporal, so little of it stays in the Infinity Cache"},
    }
    print(f"[bench] timed: {ms_step * 1e3:.2f} us/step, attention {attn_ms.mean() * 1e3:.2f} us",
          file=sys.stderr, flush=True)
    if not args.no_other_configs:
        result["ab_f16k"] = ab_f16k(K, torch, stream, ci, caches, max(100, args.steps // 4),
                                    max(20, args.warmup // 4))
        del caches
        torch.cuda.empty_cache()
        result["other_configs"] = other_configs(K, W, torch, stream, max(50, args.steps // 5),
                                                max(10, args.warmup // 4))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ci, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
