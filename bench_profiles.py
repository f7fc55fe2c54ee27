#!/usr/bin/env python3
"""rocprofv3 post-processing for bench.py: turns profiler output into the short
text summaries kept under profiles/, and provides the plain device copy whose
counters calibrate the HBM byte counts.

    python bench_profiles.py --copy-calibration          (run under rocprofv3 --pmc)
    python bench_profiles.py --trace DIR --workload W    profiles/<kernel>_<W>_trace.txt
    python bench_profiles.py --pmc FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR --workload W
                                                         profiles/<kernel>_<W>_pmc.txt
    python bench_profiles.py --sq DIR [DIR ...] --workload W
                                                         profiles/<kernel>_<W>_sq.txt

Every summary records the command that produced its data (--command) and the
hash of the kernel sources it was taken on; bench.py uses a _pmc.txt traffic
figure only while that hash matches the current sources.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

from bench import KERNEL_NAMES, ROOT, kernel_source_sha, log

# kernels that appear in traces beside the four of the step and the decode pair
TRACE_EXTRA = {"reduce": "dkdv_reduce_kernel", "rope": "rope_kernel"}


def _pmc_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


# The dK/dV pass's kernel under either of its implementations (at d=128 the
# role split has its own name); both are filed under the pass's name.
KERNEL_ALIASES = {"bwd_dkdv_kernel": ("bwd_dkdv_kernel", "bwd_dkdv_roles_kernel")}


def _is_kernel(name, kname):
    return any(alias in name for alias in KERNEL_ALIASES.get(kname, (kname,)))


def _avg_counter(rows, match, counter):
    """Mean over dispatches of one counter for the kernels `match` names
    (a counter reported per XCD or per instance is summed per dispatch)."""
    vals = {}
    for r in rows:
        if _is_kernel(r.get("Kernel_Name", ""), match) and r.get("Counter_Name") == counter:
            key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(vals))
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return (sum(vals.values()) / len(vals), len(vals)) if vals else (None, 0)


OUT_DIR = os.path.join(ROOT, "profiles")


def _profiles_path(kname, workload, kind):
    os.makedirs(OUT_DIR, exist_ok=True)
    return os.path.join(OUT_DIR, f"{kname}_{workload}_{kind}.txt")


def pmc_summary(args):
    """HBM bytes per dispatch from four rocprofv3 --pmc runs: FETCH_SIZE and
    WRITE_SIZE (KiB) of the bench, and of a plain copy of known size whose
    counts give the factor from counter KiB to bytes moved."""
    fetch, write = _pmc_rows(args.pmc[0]), _pmc_rows(args.pmc[1])
    cfetch, cwrite = _pmc_rows(args.pmc[2]), _pmc_rows(args.pmc[3])
    copy_bytes = float(args.copy_bytes)
    # the copy kernel reads and writes copy_bytes each
    cf, _ = _avg_counter(cfetch, args.copy_kernel, "FETCH_SIZE")
    cw, _ = _avg_counter(cwrite, args.copy_kernel, "WRITE_SIZE")
    if cf is None or cw is None:
        sys.exit("no copy-kernel counters in the calibration runs")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    for kname in list(KERNEL_NAMES.values()) + list(TRACE_EXTRA.values()):
        fk, n1 = _avg_counter(fetch, kname, "FETCH_SIZE")
        wk, n2 = _avg_counter(write, kname, "WRITE_SIZE")
        if fk is None or wk is None:
            continue
        traffic = fk * 1024.0 * f_scale + wk * 1024.0 * w_scale
        path = _profiles_path(kname, args.workload, "pmc")
        with open(path, "w") as out:
            out.write(f"# HBM traffic of {kname} on workload {args.workload} (rocprofv3 --pmc)\n")
            out.write(f"# commands: {args.command}\n")
            out.write(f"kernel_source_sha256_16: {kernel_source_sha()}\n")
            out.write(f"dispatches_fetch: {n1}\ndispatches_write: {n2}\n")
            out.write(f"fetch_kib_per_dispatch: {fk:.1f}\nwrite_kib_per_dispatch: {wk:.1f}\n")
            out.write(f"copy_bytes: {copy_bytes:.0f}\n")
            out.write(f"copy_fetch_kib: {cf:.1f}\ncopy_write_kib: {cw:.1f}\n")
            out.write(f"scale_fetch: {f_scale:.4f}\nscale_write: {w_scale:.4f}\n")
            out.write(f"fetch_bytes_per_dispatch: {fk * 1024.0 * f_scale:.0f}\n")
            out.write(f"write_bytes_per_dispatch: {wk * 1024.0 * w_scale:.0f}\n")
            out.write(f"traffic_bytes_per_dispatch: {traffic:.0f}\n")
        log(f"wrote {path}: {traffic / 1e6:.1f} MB per dispatch")


def sq_summary(args):
    """SQ counters averaged per dispatch (any split over runs), with derived
    utilisation: MFMA busy and VALU active per SIMD (the SQ counters sum over
    SIMDs; VALU activity counts quad-cycles), GRBM_GUI_ACTIVE summed over the
    8 XCDs."""
    rows = []
    for d in args.sq:
        rows += _pmc_rows(d)
    counters = sorted({r["Counter_Name"] for r in rows})
    for kname in list(KERNEL_NAMES.values()) + list(TRACE_EXTRA.values()):
        vals = {}
        for c in counters:
            v, n = _avg_counter(rows, kname, c)
            if v is not None:
                vals[c] = (v, n)
        if not vals:
            continue
        path = _profiles_path(kname, args.workload, "sq")
        with open(path, "w") as out:
            out.write(f"# SQ counters of {kname} on workload {args.workload} (per dispatch, mean over dispatches)\n")
            out.write(f"# commands: {args.command}\n")
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
            if "SQ_WAIT_ANY" in vals and "SQ_WAVE_CYCLES" in vals:
                out.write(f"wait_any_fraction_of_wave_cycles: "
                          f"{vals['SQ_WAIT_ANY'][0] / vals['SQ_WAVE_CYCLES'][0]:.3f}\n")
            if "SQ_INSTS_MFMA" in vals:
                out.write(f"mfma_flop_executed: {vals['SQ_INSTS_MFMA'][0] * 32768:.4g}  "
                          f"(32x32x16 bf16 = 32768 flop each)\n")
        log(f"wrote {path}")


def _kernel_stats(trace_dir):
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_stats.csv under {trace_dir}")
    return list(csv.DictReader(open(files[0])))


def _write_trace(kname, w, row, command, lines):
    avg_us = float(row["AverageNs"]) / 1e3
    path = _profiles_path(kname, w.name, "trace")
    with open(path, "w") as out:
        out.write(f"# rocprofv3 kernel-trace summary: {kname} on workload {w.name} {w.describe()}\n")
        out.write(f"# command: {command}\n")
        out.write(f"kernel: {row['Name']}\n")
        out.write(f"kernel_source_sha256_16: {kernel_source_sha()}\n")
        out.write(f"calls: {row['Calls']}\n")
        out.write(f"average_us: {avg_us:.2f}\nmin_us: {float(row['MinNs']) / 1e3:.2f}\n"
                  f"max_us: {float(row['MaxNs']) / 1e3:.2f}\n")
        for line in lines(avg_us):
            out.write(line + "\n")
    log(f"wrote {path}: {avg_us:.1f} us")


def trace_summary(args):
    """Per-kernel average launch time from a rocprofv3 --kernel-trace --stats
    run, priced in algorithmic flops (the MFMA kernels) or bytes (the rest)."""
    from attn_workloads import DECODE_WORKLOADS, WORKLOADS, algorithmic_flops, dkdv_split_parts, workload_inputs
    if args.workload in DECODE_WORKLOADS:
        return decode_trace_summary(args)
    w = WORKLOADS[args.workload]
    seqlens = workload_inputs(w).seqlens if w.padded else None
    fl = algorithmic_flops(w, seqlens, not args.non_causal)
    share = {"fwd_kernel": fl["fwd"], "bwd_dkdv_kernel": fl["bwd_dkdv"], "bwd_dq_kernel": fl["bwd_dq"]}
    B, S, Hq, Hkv, d = w.B, w.S, w.Hq, w.Hkv, w.d
    kv_bf16 = B * S * Hkv * d * 2.0
    # dK/dV partials: each key row's block was split into its own number of
    # parts; the reduce pass reads that many fp32 (dK, dV) rows per key row
    per_block = dkdv_split_parts(B, S, Hq, Hkv, not args.non_causal)
    parts = sum(per_block) / len(per_block)
    rows = [min(128, S - 128 * kb) for kb in range(len(per_block))]
    partial_bytes = sum(p * r for p, r in zip(per_block, rows)) * B * Hkv * d * 4 * 2.0
    alg_bytes = {
        "preprocess_kernel": 2.0 * B * S * Hq * d * 2 + B * Hq * S * 4.0,
        "dkdv_reduce_kernel": partial_bytes + 2 * kv_bf16,
        "rope_kernel": 2.0 * B * S * (Hq + Hkv) * d * 2,
    }
    names = list(KERNEL_NAMES.values()) + list(TRACE_EXTRA.values())
    for row in _kernel_stats(args.trace):
        kname = next((k for k in names if _is_kernel(row["Name"], k)), None)
        if kname is None:
            continue
        if kname in share:
            def lines(avg_us, f=share[kname], kname=kname):
                out = [f"algorithmic_gflop_per_launch: {f / 1e9:.3f}",
                       f"achieved_tflops_at_average: {f / (avg_us * 1e-6) / 1e12:.1f}"]
                if kname == "bwd_dq_kernel":
                    out.append("note: in the benchmark's default step this pass also computes D = rowsum(dO*O) "
                               "(attn_bwd_dq_delta); with --separate-preprocess it reads D")
                if kname == "bwd_dkdv_kernel" and parts > 1:
                    out.append(f"note: this shape splits its key blocks' query ranges over {per_block} "
                               f"parts; the dK/dV call is this kernel plus dkdv_reduce_kernel")
                return out
        else:
            def lines(avg_us, b=alg_bytes[kname], kname=kname):
                out = [f"algorithmic_bytes_per_launch: {b:.0f}",
                       f"achieved_gbs_at_average: {b / (avg_us * 1e-6) / 1e9:.1f}"]
                if kname == "dkdv_reduce_kernel":
                    out.append(f"parts per key block: {per_block} (fp32 dK and dV partials read, "
                               f"bf16 dK and dV written)")
                return out
        _write_trace(kname, w, row, args.command, lines)


def decode_trace_summary(args):
    from attn_workloads import DECODE_WORKLOADS, decode_bytes, decode_workload_inputs
    w = DECODE_WORKLOADS[args.workload]
    nb = decode_bytes(w.B, w.Sq, w.Smax, w.Hq, w.Hkv, w.d, decode_workload_inputs(w).cache_lens)
    alg = {"decode_split_kernel": nb["cache"] + w.B * w.Sq * w.Hq * w.d * 2,
           "decode_merge_kernel": w.B * w.Sq * w.Hq * (w.d * 2 + 4)}
    for row in _kernel_stats(args.trace):
        kname = next((k for k in alg if k in row["Name"]), None)
        if kname is None:
            continue

        def lines(avg_us, b=alg[kname]):
            return [f"algorithmic_bytes_per_launch: {b:.0f}",
                    f"achieved_gbs_at_average: {b / (avg_us * 1e-6) / 1e9:.1f}"]
        _write_trace(kname, w, row, args.command, lines)


def copy_calibration(args):
    """A plain device copy of --copy-bytes bytes, five times: read and written
    once each per copy, the known quantity the counters are scaled by."""
    import torch
    n = int(args.copy_bytes)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="llama1b")
    ap.add_argument("--non-causal", action="store_true", help="the traced run was bidirectional")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--copy-bytes", type=float, default=1 << 30)
    ap.add_argument("--copy-kernel", default="copy")
    ap.add_argument("--pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--sq", nargs="+", metavar="DIR")
    ap.add_argument("--trace", metavar="TRACE_DIR")
    ap.add_argument("--command", default="", help="command line recorded in the written summaries")
    ap.add_argument("--out", default=None, help="directory for the summaries (default: profiles/)")
    args = ap.parse_args()
    if args.out:
        global OUT_DIR
        OUT_DIR = args.out
    if args.copy_calibration:
        copy_calibration(args)
    elif args.pmc:
        pmc_summary(args)
    elif args.sq:
        sq_summary(args)
    elif args.trace:
        trace_summary(args)
    else:
        ap.error("one of --copy-calibration, --pmc, --sq, --trace")


if __name__ == "__main__":
    main()
