"""Build the gfx950 attention library in-tree with hipcc.

    python -m causal_attention_fwd_amd.build        # writes causal_attention_fwd_amd/libattn_mi355x.so

The library is plain HIP C++ compiled for gfx950 only; no torch headers are
involved. Packed-fp32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["attn_kernels.hip", "attn_api.cpp", "attn_plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_command(out_path: str = LIB_PATH, extra=()) -> list:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-result",
           "-I", INCLUDE, "-I", CSRC]
    cmd += list(extra)
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", out_path]
    return cmd


def build(verbose: bool = False, out_path: str = LIB_PATH, extra=()) -> str:
    """Compile the library (always recompiles) and return its path."""
    cmd = compile_command(out_path + ".tmp", extra)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = [ln for ln in (res.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(out_path + ".tmp", out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
