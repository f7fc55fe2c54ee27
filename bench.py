#!/usr/bin/env python3
"""Benchmark: causal bf16 attention fwd + bwd on one MI355X.

One step = the whole path over one batch of resident synthetic inputs:
attn_fwd -> attn_bwd_dq_delta (the dQ pass, which also computes the
preprocess's D = rowsum(dO * O)) -> attn_bwd_dkdv (which reads that D); the
last two are exactly the launches attn_bwd_fused makes.
--separate-preprocess runs attn_fwd -> attn_bwd_preprocess -> attn_bwd_dkdv ->
attn_bwd_dq instead (the last two being attn_bwd). The step is timed as replays of
its captured HIP graph (no host-side launch cost; --eager times Python-issued
launches instead); per-kernel times come from an eager pass with HIP events.
Before anything is measured the step runs untimed for --clock-warmup-ms
(default 250 ms; again as graph replays after the capture, which leaves the
GPU idle; both reported as "clock_warmup"), then the --warmup steps: an idle
GPU runs its first tens of milliseconds of MFMA work at a lower clock.
Default workload: the 1B-class Llama attention, B=4, S=2048, Hq=32, Hkv=8,
d=64, dO ~ N(0, 0.1).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload llama1b]

Prints ONE JSON line on stdout (diagnostics go to stderr). Throughput counts
algorithmic flops only: 4*d per valid causal (query, key) pair per query head
forward, 2.5x that backward (five products including the QK^T recompute).

Other modes:
    --decode                 decode attention against a key/value cache instead
                             (workload decode_llama1b; HBM GB/s, one step = one
                             attn_decode call)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal bf16 attention fwd+bwd TFLOP/s and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA peak (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
KERNEL_SOURCES = ["causal_attention_fwd_amd/csrc/attn_kernels.hip", "causal_attention_fwd_amd/csrc/attn_common.h",
                  "causal_attention_fwd_amd/csrc/attn_launch.h", "causal_attention_fwd_amd/csrc/attn_plan.cpp"]
KERNEL_NAMES = {"fwd": "fwd_kernel", "pre": "preprocess_kernel", "dkdv": "bwd_dkdv_kernel", "dq": "bwd_dq_kernel",
                "dsplit": "decode_split_kernel", "dmerge": "decode_merge_kernel"}
DECODE_METRIC = "decode attention over a bf16 key/value cache, HBM GB/s (algorithmic bytes) and % of 8 TB/s"
MALL_BYTES = 256 << 20         # MI355X last-level (Infinity) cache


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed: what
    the compiler sees of it (string literals in these sources hold no comment
    markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha() -> str:
    """Hash of the kernel and launch-planning sources, comments and layout
    excluded: profiler summaries taken on other code are not used."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
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


# ----------------------------------------------------------------------------- the benchmark

def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


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
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "fwd_value": ffl / dtf / 1e12,
            "sample": f"{done} (sequence, kv head) unit evaluations ({done / len(units):.2f} passes over the "
                      f"{len(units)} units) of {w.name}, fwd+bwd, numpy fp32, {dt:.1f} s; fwd_value: the "
                      f"forward alone on the same units, {dtf:.1f} s"}


def clock_warmup(torch, step, ms):
    """Run the step, untimed, for about `ms` milliseconds before anything is
    measured: a GPU that has been idle runs its first tens of milliseconds of
    MFMA work at a lower clock (the llama1b step takes 0.399-0.405 ms after a
    few warm-up steps and 0.366-0.369 ms after ~200 ms of work). Returns what
    was run, for the JSON line."""
    if ms <= 0:
        return {"ms": 0.0, "steps": 0}
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for i in range(10):
            step(n + i)
        torch.cuda.synchronize()
        n += 10
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "steps": n}


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
    # the capture left the GPU idle: warm its clock up again on the replays
    args.graph_clock_warmup = clock_warmup(torch, lambda i: graphs[i % len(graphs)].replay(), args.clock_warmup_ms)
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    args.graphs = graphs
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
    ws = attn.bwd_workspace(q, k)  # the backward's workspace (None when the shape needs none)

    # the step's launches in order. Default: the backward with the preprocess
    # folded into the dQ pass (attn_bwd_dq_delta computes D, then
    # attn_bwd_dkdv reads it: the launches of attn_bwd_fused, issued as two
    # calls so that each kernel has its own events); --separate-preprocess:
    # attn_bwd_preprocess, then the two passes of attn_bwd.
    order = (["rope"] if args.rope else []) + (["fwd", "pre", "dkdv", "dq"] if args.separate_preprocess
                                                else ["fwd", "dq", "dkdv"])

    def launch_one(name):
        if name == "rope":
            attn.attn_rope(q, k, qa, ka, rb)
        elif name == "fwd":
            attn.attn_fwd(qa, ka, v, o, lse, scale, sl, cz)
        elif name == "pre":
            attn.attn_bwd_preprocess(o, do, delta, sl)
        elif name == "dkdv":
            attn.attn_bwd_dkdv(qa, ka, v, do, lse, delta, dk, dv, scale, sl, cz, rb, ws)
        elif args.separate_preprocess:
            attn.attn_bwd_dq(qa, ka, v, do, lse, delta, dq, scale, sl, cz, rb)
        else:
            attn.attn_bwd_dq_delta(qa, ka, v, o, do, lse, delta, dq, scale, sl, cz, rb)

    def step(ev=None):
        # ev[i] is recorded before launch i, ev[len(order)] after the last
        for i, name in enumerate(order):
            if ev is not None:
                ev[i].record()
            launch_one(name)
        if ev is not None:
            ev[len(order)].record()

    warm = clock_warmup(torch, lambda i: step(), args.clock_warmup_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    g_step = None
    launch = "eager"
    if not args.eager:
        # the same launches captured in one HIP graph and replayed (the
        # default: no host-side launch cost in the timed step)
        def capture():
            return attn.capture_step(q, k, v, do, o, lse, delta, dq, dk, dv, scale, sl, causal, ws,
                                     fused=not args.separate_preprocess, rope_base=rb, q_rot=qa if args.rope else None,
                                     k_rot=ka if args.rope else None)
        g_step = time_graph_replays(torch, [capture], args)
        launch = "hip graph" if g_step is not None else "eager (graph capture failed)"
    # per-kernel times: an eager pass with HIP events on the library's stream,
    # right after the timed replays so that the GPU is still at its sustained
    # clock (with --eager it is the timed region itself). After graph timing
    # the pass is queued behind at least 30 ms of replays of the step, which
    # keep the GPU busy while the host enqueues it (a few ms for the default
    # steps): the events then time the kernels back to back, not the host's
    # launch gaps.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)] for _ in range(args.steps)]
    if g_step is not None:
        for i in range(max(10, math.ceil(30.0 / g_step))):
            args.graphs[i % len(args.graphs)].replay()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in events) / args.steps  # ms per launch
           for i, n in enumerate(order)}
    # per-step event times (first to last launch of the step): median, min, p90
    step_ev = sorted(ev[0].elapsed_time(ev[-1]) for ev in events)
    step_stats = {"median": round(step_ev[len(step_ev) // 2], 4), "min": round(step_ev[0], 4),
                  "p90": round(step_ev[min(len(step_ev) - 1, (9 * len(step_ev)) // 10)], 4)}
    ms_step = wall * 1e3 / args.steps
    if g_step is not None:
        log(f"graph step {g_step:.4f} ms; eager pass {step_stats['median']:.4f} ms per step by its events")
        ms_step = g_step
    tflops = fl["total"] / (ms_step * 1e-3) / 1e12

    # roofline of the dominant kernel (the RoPE pre-pass is priced in hbm_rotated)
    dom = max((n for n in order if n != "rope"), key=per.get)
    if dom == "pre":
        alg_bytes = 2.0 * B * S * Hq * d * 2 + B * Hq * S * 4.0
        achieved = alg_bytes / (per[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        share = {"fwd": fl["fwd"], "dkdv": fl["bwd_dkdv"], "dq": fl["bwd_dq"]}[dom]
        achieved = share / (per[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    roof["kernel"] = KERNEL_NAMES[dom]
    roof["ms_per_launch"] = per[dom]
    roof["traffic"] = read_traffic(dom, w.name) if (causal and not args.rope) else None
    label = {n: KERNEL_NAMES.get(n, "rope_kernel") for n in order}
    if not args.separate_preprocess:
        label["dq"] = "bwd_dq_kernel (computes D)"

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": dict(w.describe(), causal=causal, launch=launch, step_launches=[label[n] for n in order],
                       valid_pairs_per_head=fl["pairs_per_head"],
                       algorithmic_gflop_per_step=round(fl["total"] / 1e9, 3),
                       rope_base=rb if args.rope else None),
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "clock_warmup": {"before_eager_pass": warm, "before_graph_timing": getattr(args, "graph_clock_warmup", None)},
        "step_event_ms": step_stats,
        "kernel_ms": {label[n]: round(per[n], 4) for n in order},
        "kernel_tflops": {label[n]: round(s / (per[n] * 1e-3) / 1e12, 1)
                          for n, s in (("fwd", fl["fwd"]), ("dkdv", fl["bwd_dkdv"]), ("dq", fl["bwd_dq"]))},
        "roofline": roof,
    }
    if not args.no_hbm:
        result["hbm_rotated"] = hbm_rotated(torch, attn, q, k, do, o, sl, rb if args.rope else 0.0, args)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget, causal, rb)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def hbm_rotated(torch, attn, q, k, do, o, sl, rope_base, args):
    """HBM throughput of the bandwidth-bound kernels on inputs that are not in
    the 256 MB last-level cache: enough copies of the preprocess's O and dO
    (and of the RoPE pre-pass's q and k) that the set rotated through exceeds
    three times the cache and holds at least four copies. Each launch reads a
    copy the previous launches have pushed out; HIP events on the library's
    stream time replays of a HIP graph holding one launch per copy. Algorithmic bytes: preprocess 2 * (B*S*Hq*d*2)
    read + B*Hq*S*4 written; RoPE (B*S*(Hq+Hkv)*d*2) read + the same written.
    A plain device copy timed the same way gives the bandwidth the box
    sustains for reference."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    out = {}

    def timed(n_copies, launch):
        # one launch per copy, captured in a HIP graph so that host-side
        # launch cost cannot set the pace; the graph is replayed and timed
        for i in range(n_copies):  # eager pass (checks the arguments)
            launch(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_copies):
                launch(i)
        graph.replay()
        torch.cuda.synchronize()
        replays = 5
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(replays):
            graph.replay()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / (replays * n_copies)

    pre_read = 2.0 * B * S * Hq * d * 2
    pre_bytes = pre_read + B * Hq * S * 4.0
    copies = max(4, math.ceil(3 * MALL_BYTES / pre_read) + 1)
    sets = [(o.clone(), do.clone(), torch.empty(B, Hq, S, device=q.device)) for _ in range(copies)]
    ms = timed(copies, lambda i: attn.attn_bwd_preprocess(sets[i][0], sets[i][1], sets[i][2], sl))
    out["preprocess_kernel"] = {"gbs": round(pre_bytes / (ms * 1e-3) / 1e9, 1),
                                "frac_of_8tbs": round(pre_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                                "ms_per_launch": round(ms, 5), "bytes_per_launch": pre_bytes,
                                "input_copies_rotated": copies}
    del sets
    if rope_base:
        rope_bytes = 2.0 * B * S * (Hq + Hkv) * d * 2
        copies = max(4, math.ceil(3 * MALL_BYTES / (rope_bytes / 2)) + 1)
        rsets = [(q.clone(), k.clone(), torch.empty_like(q), torch.empty_like(k)) for _ in range(copies)]
        ms = timed(copies, lambda i: attn.attn_rope(*rsets[i], rope_base))
        out["rope_kernel"] = {"gbs": round(rope_bytes / (ms * 1e-3) / 1e9, 1),
                              "frac_of_8tbs": round(rope_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                              "ms_per_launch": round(ms, 5), "bytes_per_launch": rope_bytes,
                              "input_copies_rotated": copies}
        del rsets
    # reference: a plain device copy (torch's copy kernel) of 512 MiB, read
    # and written once per launch (the pair is larger than the cache)
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device=q.device).fill_(1)
    dst = torch.empty_like(src)
    ms = timed(2, lambda i: (dst if i == 0 else src).copy_(src if i == 0 else dst))
    out["device_copy"] = {"gbs": round(2.0 * n / (ms * 1e-3) / 1e9, 1), "bytes_per_launch": 2.0 * n,
                          "kernel": "torch copy_ (512 MiB each way)"}
    del src, dst
    torch.cuda.synchronize()
    return out


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
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
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

    warm = clock_warmup(torch, step, args.clock_warmup_ms)
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
        "clock_warmup": {"before_eager_pass": warm, "before_graph_timing": getattr(args, "graph_clock_warmup", None)},
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
    ap.add_argument("--no-hbm", action="store_true",
                    help="skip the rotated-input HBM measurement of the preprocess (and RoPE) kernels")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work in cpu_baseline")
    ap.add_argument("--clock-warmup-ms", type=float, default=250.0,
                    help="untimed runs of the step for this long before anything is measured, so that the GPU "
                         "runs at its sustained clock (0: only the --warmup steps)")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as eager launches from Python instead of replays of its captured HIP graph")
    ap.add_argument("--graph", action="store_true",
                    help="(the default) time replays of the step captured in one HIP graph")
    ap.add_argument("--non-causal", action="store_true",
                    help="bidirectional attention (causal = 0): every key of the valid prefix, all pairs priced")
    ap.add_argument("--separate-preprocess", action="store_true",
                    help="the backward as attn_bwd_preprocess + attn_bwd (4 launches per step) instead of the "
                         "default attn_bwd_dq_delta + attn_bwd_dkdv (the launches of attn_bwd_fused)")
    ap.add_argument("--rope", action="store_true",
                    help="rotary position embedding: attn_rope pre-pass, backward with the fused adjoint")
    ap.add_argument("--rope-base", type=float, default=10000.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (each GPU would run its own "
              "(sequence, kv-head) units independently); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.workload is None:
        args.workload = "decode_llama1b" if args.decode else "llama1b"
    if args.decode:
        run_decode(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
