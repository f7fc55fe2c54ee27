"""CPU: the C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

attn_api.cpp (validation) and attn_plan.cpp (grid limits, decode plan) are
compiled with g++ -fsanitize=address,undefined together with stub launchers
(tests/c/launch_stub.cpp: they check the arguments a real launch would pass
and count launches) and a plain-C driver (tests/c/abi_sanitize.c) that makes
valid calls, invalid calls of every kind and calls with extreme sizes. The run
must be clean: every expectation met and no sanitizer report. No GPU and no
HIP compiler are involved (host code only; the ROCm headers supply the HIP
runtime types).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_attention_fwd_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def test_abi_validation_is_sanitizer_clean(tmp_path):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++/gcc or the ROCm headers are not available")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "attn_api.cpp"), os.path.join(CSRC, "attn_plan.cpp"),
                os.path.join(ROOT, "tests", "c", "launch_stub.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([gxx, *SAN, "-std=c++17", "-Wall", *inc, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    obj = str(tmp_path / "abi_sanitize.o")
    subprocess.run([gcc, *SAN, "-std=c11", "-Wall", "-Werror", *inc, "-c",
                    os.path.join(ROOT, "tests", "c", "abi_sanitize.c"), "-o", obj], check=True)
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run([gxx, *SAN, *objs, obj, "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "abi_sanitize ok" in res.stdout, out
