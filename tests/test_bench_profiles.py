"""CPU: the rocprofv3 post-processing in bench_profiles.py, on small counter
and kernel-statistics files written here (no profiler, no GPU)."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(w.fieldnames, r)))


def _run(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench_profiles.py"), *args],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    return r


def _fields(path):
    out = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def test_pmc_summary_scales_by_the_copy(tmp_path):
    d = tmp_path
    # two dispatches of the dK/dV kernel; a counter split over two XCD rows of
    # one dispatch is summed; the copy of 1 MiB reads 2048 KiB by the counter
    # (scale 0.5) and writes 1024 KiB (scale 1)
    _counters(d / "f", [(1, "void attn::bwd_dkdv_kernel<64,1,2,2>(attn::BwdArgs)", "FETCH_SIZE", 100),
                        (1, "void attn::bwd_dkdv_kernel<64,1,2,2>(attn::BwdArgs)", "FETCH_SIZE", 100),
                        (2, "void attn::bwd_dkdv_kernel<64,1,2,2>(attn::BwdArgs)", "FETCH_SIZE", 400)])
    _counters(d / "w", [(1, "void attn::bwd_dkdv_kernel<64,1,2,2>(attn::BwdArgs)", "WRITE_SIZE", 50),
                        (2, "void attn::bwd_dkdv_kernel<64,1,2,2>(attn::BwdArgs)", "WRITE_SIZE", 150)])
    _counters(d / "cf", [(1, "copy_kernel", "FETCH_SIZE", 2048)])
    _counters(d / "cw", [(1, "copy_kernel", "WRITE_SIZE", 1024)])
    out = d / "out"
    _run("--pmc", str(d / "f"), str(d / "w"), str(d / "cf"), str(d / "cw"), "--copy-bytes", str(1 << 20),
         "--workload", "llama1b", "--out", str(out), "--command", "test")
    f = _fields(out / "bwd_dkdv_kernel_llama1b_pmc.txt")
    assert float(f["fetch_kib_per_dispatch"]) == 300.0      # (200 + 400) / 2
    assert float(f["write_kib_per_dispatch"]) == 100.0
    assert float(f["scale_fetch"]) == 0.5 and float(f["scale_write"]) == 1.0
    assert float(f["traffic_bytes_per_dispatch"]) == 300 * 1024 * 0.5 + 100 * 1024
    assert len(f["kernel_source_sha256_16"]) == 16


def test_sq_summary_derived_fractions(tmp_path):
    d = tmp_path
    k = "void attn::fwd_kernel<64,2,2,4,1>(attn::FwdArgs)"
    _counters(d / "a", [(1, k, "GRBM_GUI_ACTIVE", 8000), (1, k, "SQ_VALU_MFMA_BUSY_CYCLES", 512000),
                        (1, k, "SQ_ACTIVE_INST_VALU", 128000), (1, k, "SQ_WAVE_CYCLES", 1000),
                        (1, k, "SQ_WAIT_ANY", 250), (1, k, "SQ_INSTS_MFMA", 10)])
    out = d / "out"
    _run("--sq", str(d / "a"), "--workload", "llama1b", "--out", str(out))
    f = _fields(out / "fwd_kernel_llama1b_sq.txt")
    assert float(f["elapsed_cycles_per_xcd"]) == 1000       # 8000 over 8 XCDs
    assert float(f["mfma_busy_fraction"]) == 0.5            # 512000 / (1000 * 1024 SIMDs)
    assert float(f["valu_active_fraction"]) == 0.5          # 4 * 128000 / (1000 * 1024)
    assert float(f["wait_any_fraction_of_wave_cycles"]) == 0.25
    assert f["mfma_flop_executed"].split()[0] == "3.277e+05"


def test_trace_summary_prices_kernels(tmp_path):
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writerow(["void attn::fwd_kernel<64,1,2,4,2>(attn::FwdArgs)", 10, 100000, 10000, 50, 9000, 11000])
        w.writerow(["void attn::preprocess_kernel<64>(attn::PreArgs)", 10, 20000, 2000, 10, 1900, 2100])
        w.writerow(["void attn::dkdv_reduce_kernel<64>(attn::BwdArgs)", 10, 20000, 2000, 10, 1900, 2100])
    out = tmp_path / "out"
    _run("--trace", str(d), "--workload", "tiny", "--out", str(out))
    sys.path.insert(0, ROOT)
    from attn_workloads import WORKLOADS, algorithmic_flops
    w = WORKLOADS["tiny"]
    f = _fields(out / "fwd_kernel_tiny_trace.txt")
    assert float(f["average_us"]) == 10.0
    fl = algorithmic_flops(w, None)["fwd"]
    assert abs(float(f["achieved_tflops_at_average"]) - fl / 1e-5 / 1e12) < 0.1
    p = _fields(out / "preprocess_kernel_tiny_trace.txt")
    pre = 2.0 * w.B * w.S * w.Hq * w.d * 2 + w.B * w.Hq * w.S * 4.0
    assert float(p["algorithmic_bytes_per_launch"]) == pre
    assert os.path.exists(out / "dkdv_reduce_kernel_tiny_trace.txt")


def test_kernel_hash_ignores_comments_and_layout(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    a = "int f(int x) {  // doubles\n  return 2 * x; /* plain\n product */ }\n"
    b = "int f(int x) { return 2 * x; }"
    c = "int f(int x) { return 3 * x; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(b) != bench._code_only(c)
    assert len(bench.kernel_source_sha()) == 16
