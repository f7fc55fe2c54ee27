#!/usr/bin/env python3
"""Benchmark: causal bf16 attention fwd + bwd on one MI355X.

One step = the whole path over one batch of resident synthetic inputs:
attn_fwd -> attn_bwd_preprocess -> attn_bwd_dkdv -> attn_bwd_dq (the last two
are exactly the two launches attn_bwd makes). The step is timed as replays of
its captured HIP graph (no host-side launch cost; --eager times Python-issued
launches instead); per-kernel times come from an eager pass with HIP events.
Default workload: the 1B-class Llama attention, B=4, S=2048, Hq=32, Hkv=8,
d=64, dO ~ N(0, 0.1).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload llama1b]

Prints ONE JSON line on stdout (diagnostics go to stderr). Throughput counts
algorithmic flops only: 4*d per valid causal (query, key) pair per query head
forward, 2.5x that backward (five products including the QK^T recompute).

Other modes (measurement tooling, used under rocprofv3):
    --copy-calibration       run a plain device copy of known size (counter scale)
    --pmc-summary DIR ...    turn rocprofv3 --pmc outputs into profiles/*_pmc.txt
    --trace-summary DIR      turn a rocprofv3 --kernel-trace --stats run into profiles/*_trace.txt
    --sq-summary DIR ...     turn rocprofv3 --pmc runs of SQ counters into profiles/*_sq.txt
    --decode                 decode attention against a key/value cache instead
                             (workload decode_llama1b; HBM GB/s, one step = one
                             attn_decode call)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal bf16 attention fwd+bwd TFLOP/s and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA peak (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
KERNEL_SOURCES = ["causal_attention_fwd_amd/csrc/attn_kernels.hip", "causal_attention_fwd_amd/csrc/attn_common.h"]
KERNEL_NAMES = {"fwd": "fwd_kernel", "pre": "preprocess_kernel", "dkdv": "bwd_dkdv_kernel", "dq": "bwd_dq_kernel",
                "dsplit": "decode_split_kernel", "dmerge": "decode_merge_kernel"}
DECODE_METRIC = "decode attention over a bf16 key/value cache, HBM GB/s (algorithmic bytes) and % of 8 TB/s"
MALL_BYTES = 256 << 20         # MI355X last-level (Infinity) cache


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- traffic

def read_traffic(kernel: str, workload: str):
    """HBM bytes per dispatch from a committed rocprofv3 --pmc summary, or None
    when there is none or it was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL_NAMES[kernel]}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_sha():
        return None
    try:
        return float(fields["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def _pmc_rows(d):
    import csv
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _avg_counter(rows, match, counter):
    vals = {}
    for r in rows:
        if match in r.get("Kernel_Name", "") and r.get("Counter_Name") == counter:
            key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(vals))
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return (sum(vals.values()) / len(vals), len(vals)) if vals else (None, 0)


def pmc_summary(args):
    """profiles/<kernel>_<workload>_pmc.txt from four rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE of the bench and of the copy calibration."""
    fetch = _pmc_rows(args.pmc_summary[0])
    write = _pmc_rows(args.pmc_summary[1])
    cfetch = _pmc_rows(args.pmc_summary[2])
    cwrite = _pmc_rows(args.pmc_summary[3])
    copy_bytes = float(args.copy_bytes)
    # the copy kernel reads and writes copy_bytes each; counters are in KiB
    cf, _ = _avg_counter(cfetch, args.copy_kernel, "FETCH_SIZE")
    cw, _ = _avg_counter(cwrite, args.copy_kernel, "WRITE_SIZE")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for key, kname in KERNEL_NAMES.items():
        fk, n1 = _avg_counter(fetch, kname, "FETCH_SIZE")
        wk, n2 = _avg_counter(write, kname, "WRITE_SIZE")
        if fk is None or wk is None:
            continue
        traffic = fk * 1024.0 * f_scale + wk * 1024.0 * w_scale
        path = os.path.join(ROOT, "profiles", f"{kname}_{args.workload}_pmc.txt")
        with open(path, "w") as out:
            out.write(f"# HBM traffic of {kname} on workload {args.workload} (rocprofv3 --pmc)\n")
            out.write(f"# commands: {args.pmc_command}\n")
            out.write(f"kernel_source_sha256_16: {kernel_source_sha()}\n")
            out.write(f"dispatches_fetch: {n1}\ndispatches_write: {n2}\n")
            out.write(f"fetch_kib_per_dispatch: {fk:.1f}\nwrite_kib_per_dispatch: {wk:.1f}\n")
            out.write(f"copy_bytes: {copy_bytes:.0f}\n")
            out.write(f"copy_fetch_kib: {cf:.1f}\ncopy_write_kib: {cw:.1f}\n")
            out.write(f"scale_fetch: {f_scale:.4f}\nscale_write: {w_scale:.4f}\n")
            out.write(f"traffic_bytes_per_dispatch: {traffic:.0f}\n")
        log(f"wrote {path}: {traffic / 1e6:.1f} MB per dispatch")


def sq_summary(args):
    """profiles/<kernel>_<workload>_sq.txt from rocprofv3 --pmc runs of SQ
    counters (any split over runs), averaged per dispatch, with the derived
    utilisation figures: MFMA busy and VALU active per SIMD (the SQ counters
    sum over SIMDs and count quad-cycles where noted), GRBM_GUI_ACTIVE summed
    over the 8 XCDs."""
    rows = []
    for d in args.sq_summary:
        rows += _pmc_rows(d)
    counters = sorted({r["Counter_Name"] for r in rows})
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for kname in KERNEL_NAMES.values():
        vals = {}
        for c in counters:
            v, n = _avg_counter(rows, kname, c)
            if v is not None:
                vals[c] = (v, n)
        if not vals:
            continue
        path = os.path.join(ROOT, "profiles", f"{kname}_{args.workload}_sq.txt")
        with open(path, "w") as out:
            out.write(f"# SQ counters of {kname} on workload {args.workload} (per dispatch, mean over dispatches)\n")
            out.write(f"# commands: {args.pmc_command}\n")
            out.write(f"kernel_source_sha256_16: {kernel_source_sha()}\n")
            for c, (v, n) in vals.items():
                out.write(f"{c}: {v:.6g}  ({n} dispatches)\n")
            simds, xcds = 1024, 8
            if "GRBM_GUI_ACTIVE" in vals:
                cyc = vals["GRBM_GUI_ACTIVE"][0] / xcds
                out.write(f"elapsed_cycles_per_xcd: {cyc:.0f}\n")
                if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
                    out.write(f"mfma_busy_fraction: {vals['SQ_VALU_MFMA_BUSY_CYCLES'][0] / (cyc * simds):.3f}\n")
                if "SQ_ACTIVE_INST_VALU" in vals:  # quad-cycles
                    out.write(f"valu_active_fraction: {4 * vals['SQ_ACTIVE_INST_VALU'][0] / (cyc * simds):.3f}\n")
                if "SQ_LDS_IDX_ACTIVE" in vals:
                    out.write(f"lds_active_fraction_per_cu: {vals['SQ_LDS_IDX_ACTIVE'][0] / (cyc * 256):.3f}\n")
            if "SQ_INSTS_MFMA" in vals:
                out.write(f"mfma_flop_executed: {vals['SQ_INSTS_MFMA'][0] * 32768:.4g}  (32x32x16 bf16 = 32768 flop each)\n")
        log(f"wrote {path}")


def trace_summary(args):
    """profiles/<kernel>_<workload>_trace.txt from a rocprofv3 --kernel-trace --stats run."""
    import csv
    from attn_workloads import DECODE_WORKLOADS, WORKLOADS, algorithmic_flops, workload_inputs
    if args.workload in DECODE_WORKLOADS:
        return decode_trace_summary(args)
    w = WORKLOADS[args.workload]
    seqlens = workload_inputs(w).seqlens if w.padded else None
    fl = algorithmic_flops(w, seqlens)
    share = {"fwd_kernel": fl["fwd"], "bwd_dkdv_kernel": fl["bwd_dkdv"], "bwd_dq_kernel": fl["bwd_dq"]}
    B, S, Hq, d = w.B, w.S, w.Hq, w.d
    pre_bytes = 2.0 * B * S * Hq * d * 2 + B * Hq * S * 4.0
    files = glob.glob(os.path.join(args.trace_summary, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_stats.csv under {args.trace_summary}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for row in csv.DictReader(open(files[0])):
        kname = next((k for k in KERNEL_NAMES.values() if k in row["Name"]), None)
        if kname is None:
            continue
        avg_us = float(row["AverageNs"]) / 1e3
        path = os.path.join(ROOT, "profiles", f"{kname}_{w.name}_trace.txt")
        with open(path, "w") as out:
            out.write(f"# rocprofv3 kernel-trace summary: {kname} on workload {w.name} {w.describe()}\n")
            out.write(f"# command: {args.pmc_command}\n")
            out.write(f"kernel: {row['Name']}\n")
            out.write(f"kernel_source_sha256_16: {kernel_source_sha()}\n")
            out.write(f"calls: {row['Calls']}\n")
            out.write(f"average_us: {avg_us:.2f}\nmin_us: {float(row['MinNs']) / 1e3:.2f}\n"
                      f"max_us: {float(row['MaxNs']) / 1e3:.2f}\n")
            if kname in share:
                out.write(f"algorithmic_gflop_per_launch: {share[kname] / 1e9:.3f}\n")
                out.write(f"achieved_tflops_at_average: {share[kname] / (avg_us * 1e-6) / 1e12:.1f}\n")
            else:
                out.write(f"algorithmic_bytes_per_launch: {pre_bytes:.0f}\n")
                out.write(f"achieved_gbs_at_average: {pre_bytes / (avg_us * 1e-6) / 1e9:.1f}\n")
        log(f"wrote {path}: {avg_us:.1f} us")


def decode_trace_summary(args):
    import csv
    from attn_workloads import DECODE_WORKLOADS, decode_bytes, decode_workload_inputs
    w = DECODE_WORKLOADS[args.workload]
    nb = decode_bytes(w.B, w.Sq, w.Smax, w.Hq, w.Hkv, w.d, decode_workload_inputs(w).cache_lens)
    alg = {"decode_split_kernel": nb["cache"] + w.B * w.Sq * w.Hq * w.d * 2,
           "decode_merge_kernel": w.B * w.Sq * w.Hq * (w.d * 2 + 4)}
    files = glob.glob(os.path.join(args.trace_summary, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_stats.csv under {args.trace_summary}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for row in csv.DictReader(open(files[0])):
        kname = next((k for k in alg if k in row["Name"]), None)
        if kname is None:
            continue
        avg_us = float(row["AverageNs"]) / 1e3
        path = os.path.join(ROOT, "profiles", f"{kname}_{w.name}_trace.txt")
        with open(path, "w") as out:
            out.write(f"# rocprofv3 kernel-trace summary: {kname} on workload {w.name} {w.describe()}\n")
            out.write(f"# command: {args.pmc_command}\n")
            out.write(f"kernel: {row['Name']}\n")
            out.write(f"kernel_source_sha256_16: {kernel_source_sha()}\n")
            out.write(f"calls: {row['Calls']}\n")
            out.write(f"average_us: {avg_us:.2f}\nmin_us: {float(row['MinNs']) / 1e3:.2f}\n"
                      f"max_us: {float(row['MaxNs']) / 1e3:.2f}\n")
            out.write(f"algorithmic_bytes_per_launch: {alg[kname]:.0f}\n")
            out.write(f"achieved_gbs_at_average: {alg[kname] / (avg_us * 1e-6) / 1e9:.1f}\n")
        log(f"wrote {path}: {avg_us:.1f} us")


# ----------------------------------------------------------------------------- copy calibration

def copy_calibration(args):
    import torch
    n = int(args.copy_bytes)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}))


# ----------------------------------------------------------------------------- the benchmark

def cpu_baseline(w, inp, budget_s: float, causal: bool = True, rope_base: float = 0.0):
    """The oracle (fp32 mode, untuned) on whole (sequence, kv head) units of the
    same workload until about `budget_s` seconds of CPU work have been spent."""
    import numpy as np
    import oracle
    from attn_workloads import valid_pairs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    q, k, v, do = (x.float().numpy() for x in (inp.q, inp.k, inp.v, inp.do))
    sl = inp.seqlens.numpy() if inp.seqlens is not None else None
    G = w.Hq // w.Hkv
    units = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    done, flops, t0 = 0, 0.0, time.perf_counter()
    # whole passes over the units are repeated while the budget lasts (a small
    # workload finishes one pass well inside it)
    for i in range(1 << 20):
        b, g = units[i % len(units)]
        hs = slice(g * G, (g + 1) * G)
        args = (q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1], do[b:b + 1, :, hs],
                inp.scale, None if sl is None else sl[b:b + 1])
        if rope_base:
            oracle.rope.backward(*args, base=rope_base, dtype=np.float32, causal=causal)
        else:
            oracle.backward(*args, dtype=np.float32, causal=causal)
        done += 1
        pairs = valid_pairs(w.S, 1, None if sl is None else sl[b:b + 1], causal)
        flops += 3.5 * 4.0 * w.d * G * pairs
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    # the forward alone, timed separately on one pass over the same units
    ffl, t1 = 0.0, time.perf_counter()
    for b, g in units:
        hs = slice(g * G, (g + 1) * G)
        args = (q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1], inp.scale,
                None if sl is None else sl[b:b + 1])
        if rope_base:
            oracle.rope.forward(*args, base=rope_base, dtype=np.float32, causal=causal)
        else:
            oracle.forward(*args, dtype=np.float32, causal=causal)
        ffl += 4.0 * w.d * G * valid_pairs(w.S, 1, None if sl is None else sl[b:b + 1], causal)
        if time.perf_counter() - t1 >= budget_s / 4:
            break
    dtf = time.perf_counter() - t1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "fwd_value": ffl / dtf / 1e12,
            "sample": f"{done} (sequence, kv head) unit evaluations ({done / len(units):.2f} passes over the "
                      f"{len(units)} units) of {w.name}, fwd+bwd, numpy fp32, {dt:.1f} s; fwd_value: the "
                      f"forward alone on the same units, {dtf:.1f} s"}


def time_graph_replays(torch, makers, args):
    """Capture one HIP graph per maker, replay them in turn (warm-up, then the
    timed steps between synchronisations) and return ms per step; None when a
    capture fails (the caller then keeps the eager timing)."""
    try:
        graphs = [make() for make in makers]
    except Exception as e:  # capture errors only; a faulting replay is not caught
        log(f"graph capture failed ({type(e).__name__}: {e}); timing the eager launches instead")
        torch.cuda.synchronize()
        return None
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / args.steps


def run(args):
    import torch
    import causal_attention_fwd_amd as attn
    from attn_workloads import WORKLOADS, algorithmic_flops, workload_inputs

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    attn.load_library()  # fails loudly when the HIP library is not built
    w = WORKLOADS[args.workload]
    inp = workload_inputs(w)
    dev = torch.device("cuda")
    q, k, v, do = (x.to(dev).contiguous() for x in (inp.q, inp.k, inp.v, inp.do))
    sl = inp.seqlens.to(dev) if inp.seqlens is not None else None
    B, S, Hq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, S, device=dev)
    delta = torch.empty(B, Hq, S, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    scale = inp.scale
    causal = not args.non_causal
    fl = algorithmic_flops(w, inp.seqlens, causal)
    cz = int(causal)
    rb = args.rope_base if args.rope else 0.0
    qa, ka = q, k
    if args.rope:
        # the rotated copies the forward and backward read (kept like saved activations)
        qa, ka = torch.empty_like(q), torch.empty_like(k)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if args.rope:
            attn.attn_rope(q, k, qa, ka, rb)
        if ev is not None:
            ev[5].record()
        attn.attn_fwd(qa, ka, v, o, lse, scale, sl, cz)
        if ev is not None:
            ev[1].record()
        if args.fused_bwd:
            # preprocess folded into dQ, which runs first; events 2 and 3 bracket dQ + D
            if ev is not None:
                ev[2].record()
            attn.attn_bwd_fused(qa, ka, v, o, do, lse, delta, dq, dk, dv, scale, sl, None, cz, rb)
            if ev is not None:
                ev[3].record()
                ev[4].record()
        else:
            attn.attn_bwd_preprocess(o, do, delta, sl)
            if ev is not None:
                ev[2].record()
            attn.attn_bwd_dkdv(qa, ka, v, do, lse, delta, dk, dv, scale, sl, cz, rb)
            if ev is not None:
                ev[3].record()
            attn.attn_bwd_dq(qa, ka, v, do, lse, delta, dq, scale, sl, cz, rb)
            if ev is not None:
                ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["fwd", "pre", "dkdv", "dq"]
    per = {n: 0.0 for n in names}
    rope_ms = 0.0
    for ev in events:
        per["fwd"] += ev[5].elapsed_time(ev[1])
        for j, n in enumerate(names[1:], start=1):
            per[n] += ev[j].elapsed_time(ev[j + 1])
        rope_ms += ev[0].elapsed_time(ev[5])
    per = {n: per[n] / args.steps for n in names}           # ms per launch
    rope_ms /= args.steps
    # per-step event times (first to last launch of the step): median, min, p90
    step_ev = sorted(ev[0].elapsed_time(ev[4]) for ev in events)
    step_stats = {"median": round(step_ev[len(step_ev) // 2], 4), "min": round(step_ev[0], 4),
                  "p90": round(step_ev[min(len(step_ev) - 1, (9 * len(step_ev)) // 10)], 4)}
    ms_step = wall * 1e3 / args.steps
    launch = "eager"
    if not args.eager:
        # the same launches captured in one HIP graph and replayed (the
        # default: no host-side launch cost in the timed step); the per-kernel
        # times above stay those of the eager launches
        def capture():
            return attn.capture_step(q, k, v, do, o, lse, delta, dq, dk, dv, scale, sl, causal, None,
                                     fused=args.fused_bwd, rope_base=rb, q_rot=qa if args.rope else None,
                                     k_rot=ka if args.rope else None)
        g_step = time_graph_replays(torch, [capture], args)
        if g_step is None:
            launch = "eager (graph capture failed)"
        else:
            log(f"eager step {ms_step:.4f} ms, graph step {g_step:.4f} ms")
            ms_step = g_step
            launch = "hip graph"
    tflops = fl["total"] / (ms_step * 1e-3) / 1e12

    # roofline of the dominant kernel
    dom = max(per, key=per.get)
    if args.fused_bwd:
        # one call launches dQ (+D) and dK/dV back to back: priced together
        # against the backward's algorithmic flops
        achieved = fl["bwd"] / (per["dkdv"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "kernel": "bwd_dq_kernel+bwd_dkdv_kernel (attn_bwd_fused)",
                "ms_per_launch": per["dkdv"], "traffic": None}
    elif dom == "pre":
        alg_bytes = 2.0 * B * S * Hq * d * 2 + B * Hq * S * 4.0
        achieved = alg_bytes / (per[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        share = {"fwd": fl["fwd"], "dkdv": fl["bwd_dkdv"], "dq": fl["bwd_dq"]}[dom]
        achieved = share / (per[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    if not args.fused_bwd:
        roof["kernel"] = KERNEL_NAMES[dom]
        roof["ms_per_launch"] = per[dom]
        roof["traffic"] = read_traffic(dom, w.name) if (causal and not args.rope) else None

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": dict(w.describe(), causal=causal, launch=launch, fused_bwd=bool(args.fused_bwd),
                       valid_pairs_per_head=fl["pairs_per_head"],
                       algorithmic_gflop_per_step=round(fl["total"] / 1e9, 3),
                       rope_base=rb if args.rope else None),
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "step_event_ms": step_stats,
        "kernel_ms": dict({KERNEL_NAMES[n]: round(per[n], 4) for n in names} if not args.fused_bwd else
                          {"fwd_kernel": round(per["fwd"], 4),
                           "attn_bwd_fused (bwd_dq_kernel + bwd_dkdv_kernel)": round(per["dkdv"], 4)},
                          **({"rope_kernel": round(rope_ms, 4)} if args.rope else {})),
        "kernel_tflops": ({KERNEL_NAMES[n]: round(s / (per[n] * 1e-3) / 1e12, 1)
                           for n, s in (("fwd", fl["fwd"]), ("dkdv", fl["bwd_dkdv"]), ("dq", fl["bwd_dq"]))}
                          if not args.fused_bwd else
                          {"fwd_kernel": round(fl["fwd"] / (per["fwd"] * 1e-3) / 1e12, 1),
                           "attn_bwd_fused": round(fl["bwd"] / (per["dkdv"] * 1e-3) / 1e12, 1)}),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget, causal, rb)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def decode_cpu_baseline(w, inp, budget_s: float):
    """The oracle (fp32 mode, untuned) on whole sequences of the decode workload
    until about `budget_s` seconds of CPU work have been spent; priced in the
    same algorithmic bytes as the GPU figure."""
    import numpy as np
    import oracle
    from attn_workloads import decode_bytes
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    q = inp.q.float().numpy()
    k, v = inp.k_cache.float().numpy(), inp.v_cache.float().numpy()
    lens = inp.cache_lens.numpy() if inp.cache_lens is not None else None
    done, nbytes, t0 = 0, 0.0, time.perf_counter()
    for b in range(w.B):
        lb = None if lens is None else lens[b:b + 1]
        oracle.decode(q[b:b + 1], k[b:b + 1], v[b:b + 1], inp.scale, lb, dtype=np.float32)
        done += 1
        nbytes += decode_bytes(1, w.Sq, w.Smax, w.Hq, w.Hkv, w.d, None if lb is None else inp.cache_lens[b:b + 1])["total"]
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {w.B} sequences of {w.name}, numpy fp32, {dt:.1f} s"}


def run_decode(args):
    """One step = one attn_decode call (split-KV partials, then their merge)
    over the resident cache. Several copies of the inputs are rotated so that
    a call never finds its cache in the last-level cache from the call before
    (serving walks a different layer's cache each call)."""
    import torch
    import causal_attention_fwd_amd as attn
    from attn_workloads import DECODE_WORKLOADS, decode_bytes, decode_workload_inputs

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    attn.load_library()
    w = DECODE_WORKLOADS[args.workload]
    inp = decode_workload_inputs(w)
    dev = torch.device("cuda")
    alloc = 2 * inp.k_cache.numel() * 2
    copies = max(2, math.ceil(3 * MALL_BYTES / alloc) + 1)
    lens = inp.cache_lens.to(dev) if inp.cache_lens is not None else None
    sets = []
    for _ in range(copies):
        q, k, v = (x.to(dev).contiguous() for x in (inp.q, inp.k_cache, inp.v_cache))
        if args.decode_layout == "head":
            # caches stored head-major [B, Hkv, Smax, d], passed as strided views
            k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
            v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        sets.append((q, k, v, torch.empty_like(q), torch.empty(w.B, w.Hq, w.Sq, device=dev)))
    ws = torch.empty(max(16, attn.attn_decode_workspace_bytes(w.B, w.Sq, w.Smax, w.Hq, w.Hkv, w.d)),
                     dtype=torch.uint8, device=dev)
    nb = decode_bytes(w.B, w.Sq, w.Smax, w.Hq, w.Hkv, w.d, inp.cache_lens)

    def step(i, ev=None):
        q, k, v, o, lse = sets[i % copies]
        if ev is not None:
            ev[0].record()
        attn.attn_decode(q, k, v, o, lse, inp.scale, lens, ws)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_call = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    ms_step = wall * 1e3 / args.steps
    launch = "eager"
    if not args.eager:
        # one graph per rotated input set (a graph is bound to its tensors)
        makers = [lambda t=t: attn.capture_decode(t[0], t[1], t[2], t[3], t[4], inp.scale, lens, ws)
                  for t in sets]
        g_ms = time_graph_replays(torch, makers, args)
        if g_ms is None:
            launch = "eager (graph capture failed)"
        else:
            log(f"eager call {ms_step:.4f} ms, graph replay {g_ms:.4f} ms")
            ms_step = g_ms
            launch = "hip graph"
    gbs = nb["total"] / (ms_step * 1e-3) / 1e9
    achieved = nb["total"] / (ms_call * 1e-3) / 1e9
    t_split, t_merge = read_traffic("dsplit", w.name), read_traffic("dmerge", w.name)
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": (t_split + t_merge) if (t_split is not None and t_merge is not None) else None,
            "kernel": "decode_split_kernel+decode_merge_kernel", "ms_per_launch": ms_call}
    result = {
        "metric": DECODE_METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": dict(w.describe(), launch=launch, input_copies_rotated=copies,
                       cache_layout="[B,Hkv,Smax,d]" if args.decode_layout == "head" else "[B,Smax,Hkv,d]",
                       algorithmic_bytes_per_step=nb["total"]),
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = decode_cpu_baseline(w, inp, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="llama1b (default), or decode_llama1b with --decode")
    ap.add_argument("--decode", action="store_true", help="decode attention against a key/value cache")
    ap.add_argument("--decode-layout", choices=("position", "head"), default="position",
                    help="cache storage for --decode: position-major [B,Smax,Hkv,d] or head-major [B,Hkv,Smax,d]")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work in cpu_baseline")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as eager launches from Python instead of replays of its captured HIP graph")
    ap.add_argument("--graph", action="store_true",
                    help="(the default) time replays of the step captured in one HIP graph")
    ap.add_argument("--non-causal", action="store_true",
                    help="bidirectional attention (causal = 0): every key of the valid prefix, all pairs priced")
    ap.add_argument("--fused-bwd", action="store_true",
                    help="attn_bwd_fused: the preprocess folded into the dQ pass (3 launches per step)")
    ap.add_argument("--rope", action="store_true",
                    help="rotary position embedding: attn_rope pre-pass, backward with the fused adjoint")
    ap.add_argument("--rope-base", type=float, default=10000.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--copy-bytes", type=float, default=1 << 30)
    ap.add_argument("--copy-kernel", default="copy")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--sq-summary", nargs="+", metavar="DIR")
    ap.add_argument("--pmc-command", default="", help="command line recorded in the written summaries")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (each GPU would run its own "
              "(sequence, kv-head) units independently); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.workload is None:
        args.workload = "decode_llama1b" if args.decode else "llama1b"
    if args.pmc_summary:
        pmc_summary(args)
    elif args.trace_summary:
        trace_summary(args)
    elif args.sq_summary:
        sq_summary(args)
    elif args.copy_calibration:
        copy_calibration(args)
    elif args.decode:
        run_decode(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
