"""C-ABI checks that need no GPU (CPU only).

The library loads here (ROCm is installed even without a device), exports every
function include/attn.h declares, and rejects invalid calls with the documented
status code before any HIP call. No call in this file reaches a kernel launch:
every call made with placeholder pointers fails host validation first.
"""
import ctypes
import os
import re
import subprocess

import pytest

import causal_attention_fwd_amd as attn
from attn_workloads import dkdv_split_parts as dealt_parts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.library_path()):
        from causal_attention_fwd_amd import build as b
        b.build()
    return attn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(attn_[a-z_]+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(attn.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", attn.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (attn_[a-z_]+)$", out, re.M))
    assert set(declared_functions()) <= exported


def test_status_strings(lib):
    for code, name in attn.STATUS.items():
        assert attn.attn_status_string(code).startswith(name)
    assert "UNKNOWN" in attn.attn_status_string(99)


def _shape(**kw):
    base = dict(B=2, S=128, Hq=4, Hkv=2, d=64, scale=0.125, seqlens_ptr=None, causal=1, rope_base=0.0,
                q_stride=None, kv_stride=None, o_stride=None)
    base.update(kw)
    return attn.make_shape(base["B"], base["S"], base["Hq"], base["Hkv"], base["d"], base["scale"],
                           base["seqlens_ptr"], base["causal"], base["rope_base"], base["q_stride"],
                           base["kv_stride"], base["o_stride"])


P = ctypes.c_void_p
GOOD = 0x10000          # placeholder, 16-byte aligned (never dereferenced: validation fails first)
ODD = 0x10008           # 8-byte aligned only


def _fwd(lib, shape, ptrs=(GOOD,) * 5):
    return lib.attn_fwd(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs], P(0))


def _bwd(lib, shape, ptrs=(GOOD,) * 9, ws=None, ws_bytes=0):
    return lib.attn_bwd(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs],
                        P(ws), ctypes.c_size_t(ws_bytes), P(0))


def _dkdv(lib, shape, ptrs=(GOOD,) * 8):
    return lib.attn_bwd_dkdv(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs], None, 0,
                             P(0))


def _dq(lib, shape, ptrs=(GOOD,) * 7):
    return lib.attn_bwd_dq(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs], P(0))


def _rope(lib, shape, ptrs=(GOOD,) * 4):
    return lib.attn_rope(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs], P(0))


def _fused(lib, shape, ptrs=(GOOD,) * 10, ws=None, ws_bytes=0):
    return lib.attn_bwd_fused(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs],
                              P(ws), ctypes.c_size_t(ws_bytes), P(0))


def _dq_delta(lib, shape, ptrs=(GOOD,) * 8):
    return lib.attn_bwd_dq_delta(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs], P(0))


def _pre(lib, shape, ptrs=(GOOD,) * 3):
    return lib.attn_bwd_preprocess(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs], P(0))


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 1), (dict(S=0), 1), (dict(Hq=0), 1), (dict(Hkv=0), 1), (dict(S=-5), 1),
    (dict(Hq=6, Hkv=4), 1), (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1),
    (dict(scale=0.0), 1), (dict(scale=-0.1), 1),
    (dict(d=32), 2), (dict(d=96), 2), (dict(d=256), 2), (dict(causal=2), 1), (dict(causal=-1), 1),
    (dict(seqlens_ptr=GOOD + 2), 3),
    (dict(rope_base=-1.0), 1), (dict(rope_base=float("nan")), 1), (dict(rope_base=float("inf")), 1),
    (dict(q_stride=(128 * 4 * 64, 4 * 64, 60)), 3), (dict(kv_stride=(-8, 128, 64)), 3),
    (dict(o_stride=(8, 8, 4)), 3), (dict(q_stride=(1 << 40, (1 << 22) + 8, 64)), 2),
    (dict(kv_stride=(0, (1 << 22) + 64, 64)), 2),
    (dict(B=2 ** 30, S=2 ** 20), 2), (dict(Hq=2 ** 17, Hkv=1), 2), (dict(Hq=2 ** 16, Hkv=2 ** 16, d=128), 2),
])
def test_invalid_shapes_rejected(lib, kw, code):
    shape = _shape(**kw)
    assert _rope(lib, shape) == code
    assert _fused(lib, shape) == code
    assert _fwd(lib, shape) == code
    assert _pre(lib, shape) == code
    assert _bwd(lib, shape) == code
    assert _dkdv(lib, shape) == code
    assert _dq(lib, shape) == code


def test_null_shape_and_pointers(lib):
    assert _fwd(lib, None) == 1
    assert _pre(lib, None) == 1
    assert _bwd(lib, None) == 1
    for i in range(5):
        ptrs = [GOOD] * 5
        ptrs[i] = 0
        assert _fwd(lib, _shape(), ptrs) == 1
    for i in range(3):
        ptrs = [GOOD] * 3
        ptrs[i] = 0
        assert _pre(lib, _shape(), ptrs) == 1
    for i in range(9):
        ptrs = [GOOD] * 9
        ptrs[i] = 0
        assert _bwd(lib, _shape(), ptrs) == 1
    for i in range(8):
        ptrs = [GOOD] * 8
        ptrs[i] = 0
        assert _dkdv(lib, _shape(), ptrs) == 1
    for i in range(7):
        ptrs = [GOOD] * 7
        ptrs[i] = 0
        assert _dq(lib, _shape(), ptrs) == 1
    assert _dkdv(lib, None) == 1
    assert _dq(lib, None) == 1


def test_misaligned_pointers(lib):
    for i in range(5):
        ptrs = [GOOD] * 5
        ptrs[i] = ODD
        assert _fwd(lib, _shape(), ptrs) == 3
    for i in range(9):
        ptrs = [GOOD] * 9
        ptrs[i] = ODD
        assert _bwd(lib, _shape(), ptrs) == 3
    for i in range(8):
        ptrs = [GOOD] * 8
        ptrs[i] = ODD
        assert _dkdv(lib, _shape(), ptrs) == 3


def test_workspace_bytes_is_linear_not_quadratic(lib):
    for S in (128, 4096, 16384, 1 << 20):
        shape = _shape(B=1, S=S, Hq=32, Hkv=8, d=128)
        ws = lib.attn_bwd_workspace_bytes(ctypes.byref(shape))
        assert ws <= 1 * S * 32 * 128 * 4
    assert lib.attn_bwd_workspace_bytes(None) == 0


@pytest.mark.parametrize("B,S,Hq,Hkv,causal", [(2, 1024, 12, 4, 1), (2, 1024, 12, 4, 0), (1, 1000, 8, 1, 1),
                                               (3, 333, 4, 2, 1), (1, 128, 2, 2, 1), (4, 2048, 32, 8, 1),
                                               (2, 1281, 12, 4, 1)])
def test_split_workspace_holds_the_most_parts_of_any_block(lib, B, S, Hq, Hkv, causal):
    parts = dealt_parts(B, S, Hq, Hkv, causal)
    shape = _shape(B=B, S=S, Hq=Hq, Hkv=Hkv, d=64, causal=causal)
    split = sum(parts) > len(parts)
    want = 2 * max(parts) * B * S * Hkv * 64 * 4 if split else 0  # fp32 dK and dV partials
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(shape)) == want
    if causal and want:
        # the first blocks, which meet the most query tiles, get the most workgroups
        assert parts[0] >= parts[-1] and sum(parts) % len(parts) == 0


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_fwd(q, q, q, q, lse, 0.125)


def test_product_path_never_uses_the_oracle():
    pkg = os.path.join(ROOT, "causal_attention_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


# ------------------------------------------------------------------ decode

def _dshape(**kw):
    base = dict(B=2, Sq=1, Smax=256, Hq=8, Hkv=2, d=64, scale=0.125, lens_ptr=None, rope_base=0.0)
    base.update(kw)
    return attn.make_decode_shape(base["B"], base["Sq"], base["Smax"], base["Hq"], base["Hkv"], base["d"],
                                  base["scale"], base["lens_ptr"], base["rope_base"])


def _dec(lib, shape, ptrs=(GOOD,) * 5, ws=None, ws_bytes=0):
    return lib.attn_decode(ctypes.byref(shape) if shape is not None else None, *[P(p) for p in ptrs],
                           P(ws), ctypes.c_size_t(ws_bytes), P(0))


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 1), (dict(Sq=0), 1), (dict(Smax=0), 1), (dict(Hq=0), 1), (dict(Hkv=0), 1), (dict(Smax=-3), 1),
    (dict(Hq=6, Hkv=4), 1), (dict(scale=float("nan")), 1), (dict(scale=0.0), 1), (dict(scale=-1.0), 1),
    (dict(d=32), 2), (dict(d=96), 2), (dict(rope_base=-1.0), 1), (dict(rope_base=float("nan")), 1),
    (dict(lens_ptr=GOOD + 2), 3), (dict(Hq=2 ** 16, Hkv=2 ** 16, d=128), 2),
    (dict(B=2 ** 20, Sq=64, Hq=64, Hkv=8, Smax=2 ** 16), 2),
])
def test_decode_invalid_shapes_rejected(lib, kw, code):
    shape = _dshape(**kw)
    assert _dec(lib, shape, ws=GOOD, ws_bytes=1 << 40) == code
    assert lib.attn_decode_workspace_bytes(ctypes.byref(shape)) == 0


def test_decode_pointers_and_workspace(lib):
    assert _dec(lib, None) == 1
    assert lib.attn_decode_workspace_bytes(None) == 0
    shape = _dshape()
    need = lib.attn_decode_workspace_bytes(ctypes.byref(shape))
    assert need > 0
    for i in range(5):
        ptrs = [GOOD] * 5
        ptrs[i] = 0
        assert _dec(lib, shape, ptrs, GOOD, need) == 1
        ptrs[i] = ODD
        assert _dec(lib, shape, ptrs, GOOD, need) == 3
    assert _dec(lib, shape, ws=None, ws_bytes=need) == 4
    assert _dec(lib, shape, ws=GOOD, ws_bytes=need - 1) == 4
    assert _dec(lib, shape, ws=ODD, ws_bytes=need) == 4


def test_decode_workspace_bytes_bounded_by_waves_and_units(lib):
    # one fp32 partial (d values + LSE) per query row and (wave, unit) slot;
    # the wave count is capped, so the workspace does not grow with the cache
    def ws(**kw):
        return lib.attn_decode_workspace_bytes(ctypes.byref(_dshape(**kw)))
    for B, Sq, Hq, Hkv, d in ((4, 1, 32, 8, 64), (3, 8, 32, 4, 128), (2, 5, 20, 2, 64)):
        R = Sq * Hq // Hkv
        RB = -(-R // 32)
        RU, U = (R if RB == 1 else 32), B * Hkv * RB
        big = [ws(B=B, Sq=Sq, Smax=Smax, Hq=Hq, Hkv=Hkv, d=d) for Smax in (1 << 14, 1 << 16, 1 << 20)]
        assert big[0] == big[1] == big[2]
        assert big[0] <= 256 + 256 + U * 8 + 256 + (1024 + U) * RU * (d + 1) * 4
        # a one-tile cache needs one wave per unit at most
        small = ws(B=B, Sq=Sq, Smax=64, Hq=Hq, Hkv=Hkv, d=d)
        assert small <= 256 + 256 + U * 8 + 256 + (2 * U) * RU * (d + 1) * 4


def test_rope_requires_a_base_and_valid_pointers(lib):
    assert _rope(lib, None) == 1
    assert _rope(lib, _shape()) == 1                      # rope_base = 0: nothing to rotate with
    shape = _shape(rope_base=10000.0)
    for i in range(4):
        ptrs = [GOOD] * 4
        ptrs[i] = 0
        assert _rope(lib, shape, ptrs) == 1
        ptrs[i] = ODD
        assert _rope(lib, shape, ptrs) == 3
    # a rope base is accepted by every attention entry point (validation only)
    assert _fwd(lib, _shape(rope_base=10000.0, d=96)) == 2


def test_strides_accepted_when_valid(lib):
    # a fused QKV projection output [B, S, Hq + 2 Hkv, d]: q, k, v are views
    B, S, Hq, Hkv, d = 2, 128, 4, 2, 64
    W = (Hq + 2 * Hkv) * d
    shape = _shape(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, q_stride=(S * W, W, d), kv_stride=(S * W, W, d),
                   o_stride=(S * Hq * d, Hq * d, d))
    # validation passes; a null pointer then stops the call before any launch
    assert _fwd(lib, shape, (0, GOOD, GOOD, GOOD, GOOD)) == 1
    # the same layout with one stride off the 8-element grid is refused
    bad = _shape(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, q_stride=(S * W, W + 4, d))
    assert _fwd(lib, bad) == 3


def test_fused_backward_pointers(lib):
    assert _fused(lib, None) == 1
    for i in range(10):
        ptrs = [GOOD] * 10
        ptrs[i] = 0
        assert _fused(lib, _shape(), ptrs) == 1
        ptrs[i] = ODD
        assert _fused(lib, _shape(), ptrs) == 3


def test_dq_delta_pointers_and_shapes(lib):
    assert _dq_delta(lib, None) == 1
    for i in range(8):
        ptrs = [GOOD] * 8
        ptrs[i] = 0
        assert _dq_delta(lib, _shape(), ptrs) == 1
        ptrs[i] = ODD
        assert _dq_delta(lib, _shape(), ptrs) == 3
    assert _dq_delta(lib, _shape(d=96)) == 2
    assert _dq_delta(lib, _shape(Hq=6, Hkv=4)) == 1


def test_plain_c_client_and_struct_layouts(lib, tmp_path):
    """include/attn.h compiles as C99 with gcc and links against the library;
    the struct layouts it reports are the ones the ctypes binding uses."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    exe = tmp_path / "abi_check"
    src = os.path.join(ROOT, "tests", "c", "abi_check.c")
    lib_path = attn.library_path()
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__", src, "-o", str(exe), lib_path, "-Wl,-rpath," + os.path.dirname(lib_path)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    vals = {}
    for line in out.splitlines():
        parts = line.split()
        for key, val in zip(parts[0::2], parts[1::2]):
            vals[key] = val
    assert int(vals["attn_shape"]) == ctypes.sizeof(attn.AttnShape)
    for f in ("rope_base", "q_stride", "kv_stride", "o_stride", "seqlens"):
        assert int(out.split(f + " ")[1].split()[0]) == getattr(attn.AttnShape, f).offset, f
    assert int(vals["attn_decode_shape"]) == ctypes.sizeof(attn.AttnDecodeShape)
    assert int(vals["cache_lens"]) == attn.AttnDecodeShape.cache_lens.offset
    dline = [l for l in out.splitlines() if l.startswith("attn_decode_shape")][0].split()
    assert int(dline[dline.index("rope_base") + 1]) == attn.AttnDecodeShape.rope_base.offset
    for c_name, f in (("dq_stride", "q_stride"), ("dkv_stride", "kv_stride"), ("do_stride", "o_stride")):
        assert int(dline[dline.index(c_name) + 1]) == getattr(attn.AttnDecodeShape, f).offset, f
    assert vals["fwd_bad_dim"] == "2" and vals["fwd_null_ptr"] == "1" and vals["fwd_bad_stride"] == "3"
    assert "ATTN_ERR_INVALID_ARG" in out
