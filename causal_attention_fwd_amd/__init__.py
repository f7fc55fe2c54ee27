"""Python binding of the gfx950 fused causal attention library (libattn_mi355x.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/attn.h. PyTorch supplies device
memory and the current stream. There is no CPU fallback: if the library is not
built, or a tensor is not on a GPU, the call raises.

Entry points (same names as the C ABI):
    attn_rope(q, k, q_rot, k_rot, rope_base=10000.0, seqlens=None)
    attn_fwd(q, k, v, o, lse, scale, seqlens=None)
    attn_bwd_preprocess(o, d_o, delta, seqlens=None)
    attn_bwd_workspace_bytes(B, S, Hq, Hkv, d)
    attn_bwd(q, k, v, d_o, lse, delta, dq, dk, dv, scale, seqlens=None, workspace=None)
    attn_bwd_dkdv(q, k, v, d_o, lse, delta, dk, dv, scale, seqlens=None, workspace=None)
    attn_bwd_dq(q, k, v, d_o, lse, delta, dq, scale, seqlens=None)
    attn_bwd_fused(q, k, v, o, d_o, lse, delta, dq, dk, dv, scale, seqlens=None, workspace=None)
    attn_bwd_dq_delta(q, k, v, o, d_o, lse, delta, dq, scale, seqlens=None)
    attn_decode_workspace_bytes(B, Sq, Smax, Hq, Hkv, d)
    attn_decode(q, k_cache, v_cache, o, lse, scale, cache_lens=None, workspace=None)
    attn_decode_noalloc(q, k_cache, v_cache, o, lse, scale, cache_lens=None)
    attn_status_string(code)
and allocating conveniences `rope(...)`, `forward(...)`, `backward(...)`, `decode(...)`.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["attn_rope", "rope", "attn_bwd_fused", "attn_bwd_dq_delta", "capture_decode", "attn_fwd", "attn_bwd_preprocess", "attn_bwd_workspace_bytes", "attn_bwd",
           "attn_bwd_dkdv", "attn_bwd_dq", "bwd_workspace", "attn_decode_workspace_bytes", "attn_decode", "attn_decode_noalloc", "attn_status_string",
           "forward", "backward", "decode", "capture_step", "AttnError", "library_path", "load_library",
           "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libattn_mi355x.so"

STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_MISALIGNED",
          4: "ATTN_ERR_WORKSPACE", 5: "ATTN_ERR_HIP"}

# The symbols include/attn.h declares.
EXPORTED = ("attn_rope", "attn_fwd", "attn_bwd_preprocess", "attn_bwd_workspace_bytes", "attn_bwd", "attn_bwd_dkdv",
            "attn_bwd_dq", "attn_bwd_fused", "attn_bwd_dq_delta", "attn_decode_workspace_bytes", "attn_decode", "attn_decode_noalloc",
            "attn_status_string")


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {attn_status_string(code)} (status {code})")


class AttnShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float),
                ("causal", ctypes.c_int32), ("seqlens", ctypes.c_void_p), ("rope_base", ctypes.c_float),
                ("q_stride", ctypes.c_int64 * 3), ("kv_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3)]


class AttnDecodeShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("cache_len", ctypes.c_int32),
                ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float), ("cache_lens", ctypes.c_void_p), ("rope_base", ctypes.c_float),
                ("q_stride", ctypes.c_int64 * 3), ("kv_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3)]


def library_path() -> str:
    return os.environ.get("ATTN_MI355X_LIB", os.path.join(_HERE, LIB_NAME))


_lib = None


def load_library():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m causal_attention_fwd_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    shp = ctypes.POINTER(AttnShape)
    lib.attn_fwd.argtypes = [shp, vp, vp, vp, vp, vp, vp]
    lib.attn_fwd.restype = i32
    lib.attn_bwd_preprocess.argtypes = [shp, vp, vp, vp, vp]
    lib.attn_bwd_preprocess.restype = i32
    lib.attn_bwd_workspace_bytes.argtypes = [shp]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_dkdv.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_bwd_dkdv.restype = i32
    lib.attn_bwd_dq.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_bwd_dq.restype = i32
    dshp = ctypes.POINTER(AttnDecodeShape)
    lib.attn_decode_workspace_bytes.argtypes = [dshp]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode.argtypes = [dshp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_decode.restype = i32
    lib.attn_decode_noalloc.argtypes = [dshp, vp, vp, vp, vp, vp, vp]
    lib.attn_decode_noalloc.restype = i32
    lib.attn_bwd_fused.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_bwd_fused.restype = i32
    lib.attn_bwd_dq_delta.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_bwd_dq_delta.restype = i32
    lib.attn_rope.argtypes = [shp, vp, vp, vp, vp, vp]
    lib.attn_rope.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_status_string(code: int) -> str:
    return load_library().attn_status_string(int(code)).decode()


def make_shape(B: int, S: int, Hq: int, Hkv: int, d: int, scale: float, seqlens_ptr: Optional[int] = None,
               causal: int = 1, rope_base: float = 0.0, q_stride=None, kv_stride=None, o_stride=None) -> AttnShape:
    """Stride triples are (sequence, position, head) in elements; None means dense."""
    tri = lambda x: (ctypes.c_int64 * 3)(*(x if x is not None else (0, 0, 0)))  # noqa: E731
    return AttnShape(int(B), int(S), int(Hq), int(Hkv), int(d), float(scale), int(causal),
                     ctypes.c_void_p(seqlens_ptr) if seqlens_ptr else None, float(rope_base or 0.0),
                     tri(q_stride), tri(kv_stride), tri(o_stride))


# ------------------------------------------------------------------ torch marshalling

def _torch():
    import torch
    return torch


def _check_gpu(name, t, dtype, shape=None, strided=False):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}); there is no CPU path")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if strided:
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be 4-D with its last dimension contiguous")
        _reject_expanded(name, t)
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _reject_expanded(name, t):
    """An expanded view (stride 0 on a dimension of size > 1) lets one row of
    memory stand for many; the kernels would read or write it as distinct rows
    (outputs would race), so such views are refused."""
    if any(t.shape[i] > 1 and t.stride(i) == 0 for i in range(3)):
        raise ValueError(f"{name} has an expanded (stride-0) dimension; pass a tensor with real strides "
                         f"(e.g. .contiguous())")


def _dense_triple(t):
    """Element strides of a dense [B, S, H, d] tensor of t's shape."""
    _, S, H, d = t.shape
    return (S * H * d, H * d, d)


def _strides(group, tensors):
    """The (sequence, position, head) element strides the tensors of one stride
    group share (the C ABI takes one triple per group). The stride of a size-1
    dimension never moves an address, so it is taken as the dense one: the
    triple then never reads as the all-zero "dense" marker by accident, and
    tensors that differ only there still share a triple."""
    got = None
    for name, t in tensors:
        dense = _dense_triple(t)
        st = tuple(dense[i] if t.shape[i] == 1 else int(t.stride(i)) for i in range(3))
        if got is None:
            got = st
        elif st != got:
            raise ValueError(f"{name} must have the same strides as the other {group} tensors")
    return got


def _shape_from(q, k, scale, seqlens, causal=1, rope_base=0.0, qg=(), kvg=(), og=()):
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,S,Hq,d] and k [B,S,Hkv,d]")
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    sl = None
    if seqlens is not None:
        sl = _check_gpu("seqlens", seqlens, torch.int32, (B,))
    qs = _strides("q", qg) if qg else None
    ks = _strides("k/v", kvg) if kvg else None
    os_ = _strides("o", og) if og else None
    return make_shape(B, S, Hq, Hkv, d, scale, sl, causal, rope_base, qs, ks, os_), (B, S, Hq, Hkv, d)


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _call(fn, where, *args):
    code = fn(*args)
    if code != 0:
        raise AttnError(code, where)


def attn_rope(q, k, q_rot, k_rot, rope_base: float = 10000.0, seqlens=None):
    """q_rot, k_rot <- q and k rotated by the rotary position embedding."""
    torch = _torch()
    shape, (B, S, Hq, Hkv, d) = _shape_from(q, k, 1.0, seqlens, 1, rope_base,
                                            qg=[("q", q), ("q_rot", q_rot)], kvg=[("k", k), ("k_rot", k_rot)])
    ptrs = [_check_gpu("q", q, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("k", k, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("q_rot", q_rot, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("k_rot", k_rot, torch.bfloat16, (B, S, Hkv, d), True)]
    _call(load_library().attn_rope, "attn_rope", ctypes.byref(shape), *[ctypes.c_void_p(p) for p in ptrs],
          _stream())


def attn_fwd(q, k, v, o, lse, scale: float, seqlens=None, causal: int = 1):
    """O, LSE <- attention forward (writes into `o` and `lse`)."""
    torch = _torch()
    shape, (B, S, Hq, Hkv, d) = _shape_from(q, k, scale, seqlens, causal, 0.0, qg=[("q", q)],
                                            kvg=[("k", k), ("v", v)], og=[("o", o)])
    ptrs = [_check_gpu("q", q, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("k", k, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("v", v, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("o", o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("lse", lse, torch.float32, (B, Hq, S))]
    _call(load_library().attn_fwd, "attn_fwd", ctypes.byref(shape), *[ctypes.c_void_p(p) for p in ptrs], _stream())


def attn_bwd_preprocess(o, d_o, delta, seqlens=None):
    """D <- rowsum(dO * O) (writes into `delta`)."""
    torch = _torch()
    if o.dim() != 4:
        raise ValueError("o must be [B,S,Hq,d]")
    B, S, Hq, d = o.shape
    sl = _check_gpu("seqlens", seqlens, torch.int32, (B,)) if seqlens is not None else None
    shape = make_shape(B, S, Hq, Hq, d, 1.0, sl, o_stride=_strides("o", [("o", o), ("d_o", d_o)]))
    ptrs = [_check_gpu("o", o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("d_o", d_o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("delta", delta, torch.float32, (B, Hq, S))]
    _call(load_library().attn_bwd_preprocess, "attn_bwd_preprocess", ctypes.byref(shape),
          *[ctypes.c_void_p(p) for p in ptrs], _stream())


def attn_bwd_workspace_bytes(B: int, S: int, Hq: int, Hkv: int, d: int) -> int:
    shape = make_shape(B, S, Hq, Hkv, d, 1.0 / math.sqrt(d))
    return int(load_library().attn_bwd_workspace_bytes(ctypes.byref(shape)))


def attn_bwd(q, k, v, d_o, lse, delta, dq, dk, dv, scale: float, seqlens=None, workspace=None, causal: int = 1,
             rope_base: float = 0.0):
    """dQ, dK, dV <- attention backward (writes into `dq`, `dk`, `dv`). With
    rope_base > 0, q and k are the rotated tensors and dq, dk come back with
    respect to the unrotated ones."""
    torch = _torch()
    shape, (B, S, Hq, Hkv, d) = _shape_from(q, k, scale, seqlens, causal, rope_base, qg=[("q", q)],
                                            kvg=[("k", k), ("v", v), ("dk", dk), ("dv", dv)],
                                            og=[("d_o", d_o), ("dq", dq)])
    ptrs = [_check_gpu("q", q, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("k", k, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("v", v, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("d_o", d_o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("lse", lse, torch.float32, (B, Hq, S)),
            _check_gpu("delta", delta, torch.float32, (B, Hq, S)),
            _check_gpu("dq", dq, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("dk", dk, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("dv", dv, torch.bfloat16, (B, S, Hkv, d), True)]
    ws_ptr, ws_bytes = _workspace_arg(workspace, q, k)
    _call(load_library().attn_bwd, "attn_bwd", ctypes.byref(shape), *[ctypes.c_void_p(p) for p in ptrs],
          ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes), _stream())


def _bwd_common(q, k, v, d_o, lse, delta, scale, seqlens, causal, rope_base, kv_out=(), o_out=()):
    torch = _torch()
    shape, (B, S, Hq, Hkv, d) = _shape_from(q, k, scale, seqlens, causal, rope_base, qg=[("q", q)],
                                            kvg=[("k", k), ("v", v)] + list(kv_out),
                                            og=[("d_o", d_o)] + list(o_out))
    ptrs = [_check_gpu("q", q, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("k", k, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("v", v, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("d_o", d_o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("lse", lse, torch.float32, (B, Hq, S)),
            _check_gpu("delta", delta, torch.float32, (B, Hq, S))]
    return shape, (B, S, Hq, Hkv, d), ptrs


def _workspace_arg(workspace, q, k):
    """(pointer, bytes) of the backward workspace; when none is given and the
    shape needs one, a torch tensor is allocated on q's stream (stream-ordered
    reuse by torch's allocator keeps it valid until the kernels have run)."""
    if workspace is None:
        workspace = bwd_workspace(q, k)
        if workspace is None:
            return None, 0
    return _check_gpu("workspace", workspace, workspace.dtype), workspace.numel() * workspace.element_size()


def attn_bwd_dkdv(q, k, v, d_o, lse, delta, dk, dv, scale: float, seqlens=None, causal: int = 1,
                  rope_base: float = 0.0, workspace=None):
    """dK, dV <- the key-block pass of the backward (writes into `dk`, `dv`;
    `workspace` must hold attn_bwd_workspace_bytes() bytes when that is
    nonzero)."""
    torch = _torch()
    shape, (B, S, Hq, Hkv, d), ptrs = _bwd_common(q, k, v, d_o, lse, delta, scale, seqlens, causal, rope_base,
                                                  kv_out=[("dk", dk), ("dv", dv)])
    ptrs += [_check_gpu("dk", dk, torch.bfloat16, (B, S, Hkv, d), True),
             _check_gpu("dv", dv, torch.bfloat16, (B, S, Hkv, d), True)]
    ws_ptr, ws_bytes = _workspace_arg(workspace, q, k)
    _call(load_library().attn_bwd_dkdv, "attn_bwd_dkdv", ctypes.byref(shape),
          *[ctypes.c_void_p(p) for p in ptrs], ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes), _stream())


def bwd_workspace(q, k):
    """A workspace tensor of attn_bwd_workspace_bytes() bytes for q and k's
    shapes, or None when none is needed."""
    torch = _torch()
    B, S, Hq, d = q.shape
    need = attn_bwd_workspace_bytes(B, S, Hq, k.shape[2], d)
    return torch.empty(need, dtype=torch.uint8, device=q.device) if need else None


def attn_bwd_dq(q, k, v, d_o, lse, delta, dq, scale: float, seqlens=None, causal: int = 1,
                rope_base: float = 0.0):
    """dQ <- the query-block pass of the backward (writes into `dq`)."""
    torch = _torch()
    shape, (B, S, Hq, Hkv, d), ptrs = _bwd_common(q, k, v, d_o, lse, delta, scale, seqlens, causal, rope_base,
                                                  o_out=[("dq", dq)])
    ptrs += [_check_gpu("dq", dq, torch.bfloat16, (B, S, Hq, d), True)]
    _call(load_library().attn_bwd_dq, "attn_bwd_dq", ctypes.byref(shape),
          *[ctypes.c_void_p(p) for p in ptrs], _stream())


def attn_bwd_fused(q, k, v, o, d_o, lse, delta, dq, dk, dv, scale: float, seqlens=None, workspace=None,
                   causal: int = 1, rope_base: float = 0.0):
    """D, dQ, dK, dV <- the backward with the preprocess folded into the dQ
    pass (writes `delta` as well as the gradients)."""
    torch = _torch()
    shape, (B, S, Hq, Hkv, d) = _shape_from(q, k, scale, seqlens, causal, rope_base, qg=[("q", q)],
                                            kvg=[("k", k), ("v", v), ("dk", dk), ("dv", dv)],
                                            og=[("o", o), ("d_o", d_o), ("dq", dq)])
    ptrs = [_check_gpu("q", q, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("k", k, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("v", v, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("o", o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("d_o", d_o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("lse", lse, torch.float32, (B, Hq, S)),
            _check_gpu("delta", delta, torch.float32, (B, Hq, S)),
            _check_gpu("dq", dq, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("dk", dk, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("dv", dv, torch.bfloat16, (B, S, Hkv, d), True)]
    ws_ptr, ws_bytes = _workspace_arg(workspace, q, k)
    _call(load_library().attn_bwd_fused, "attn_bwd_fused", ctypes.byref(shape), *[ctypes.c_void_p(p) for p in ptrs],
          ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes), _stream())


def attn_bwd_dq_delta(q, k, v, o, d_o, lse, delta, dq, scale: float, seqlens=None, causal: int = 1,
                      rope_base: float = 0.0):
    """D, dQ <- the dQ pass with the preprocess folded in (writes `delta` and
    `dq`); followed by attn_bwd_dkdv it is attn_bwd_fused."""
    torch = _torch()
    shape, (B, S, Hq, Hkv, d) = _shape_from(q, k, scale, seqlens, causal, rope_base, qg=[("q", q)],
                                            kvg=[("k", k), ("v", v)],
                                            og=[("o", o), ("d_o", d_o), ("dq", dq)])
    ptrs = [_check_gpu("q", q, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("k", k, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("v", v, torch.bfloat16, (B, S, Hkv, d), True),
            _check_gpu("o", o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("d_o", d_o, torch.bfloat16, (B, S, Hq, d), True),
            _check_gpu("lse", lse, torch.float32, (B, Hq, S)),
            _check_gpu("delta", delta, torch.float32, (B, Hq, S)),
            _check_gpu("dq", dq, torch.bfloat16, (B, S, Hq, d), True)]
    _call(load_library().attn_bwd_dq_delta, "attn_bwd_dq_delta", ctypes.byref(shape),
          *[ctypes.c_void_p(p) for p in ptrs], _stream())


# ------------------------------------------------------------------ decode

def make_decode_shape(B: int, Sq: int, Smax: int, Hq: int, Hkv: int, d: int, scale: float,
                      cache_lens_ptr: Optional[int] = None, rope_base: float = 0.0, q_stride=None,
                      kv_stride=None, o_stride=None) -> AttnDecodeShape:
    """Stride triples are (sequence, position, head) in elements; None means dense."""
    tri = lambda x: (ctypes.c_int64 * 3)(*(x if x is not None else (0, 0, 0)))  # noqa: E731
    return AttnDecodeShape(int(B), int(Sq), int(Smax), int(Hq), int(Hkv), int(d), float(scale),
                           ctypes.c_void_p(cache_lens_ptr) if cache_lens_ptr else None, float(rope_base or 0.0),
                           tri(q_stride), tri(kv_stride), tri(o_stride))


def attn_decode_workspace_bytes(B: int, Sq: int, Smax: int, Hq: int, Hkv: int, d: int) -> int:
    shape = make_decode_shape(B, Sq, Smax, Hq, Hkv, d, 1.0 / math.sqrt(d))
    return int(load_library().attn_decode_workspace_bytes(ctypes.byref(shape)))


def _decode_args(q, k_cache, v_cache, o, lse, scale, cache_lens, rope_base):
    torch = _torch()
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [B,Sq,Hq,d] and the caches [B,Smax,Hkv,d]")
    B, Sq, Hq, d = q.shape
    Smax, Hkv = k_cache.shape[1], k_cache.shape[2]
    lens = _check_gpu("cache_lens", cache_lens, torch.int32, (B,)) if cache_lens is not None else None
    shape = make_decode_shape(B, Sq, Smax, Hq, Hkv, d, scale, lens, rope_base, _strides("q", [("q", q)]),
                              _strides("cache", [("k_cache", k_cache), ("v_cache", v_cache)]),
                              _strides("o", [("o", o)]))
    ptrs = [_check_gpu("q", q, torch.bfloat16, (B, Sq, Hq, d), True),
            _check_gpu("k_cache", k_cache, torch.bfloat16, (B, Smax, Hkv, d), True),
            _check_gpu("v_cache", v_cache, torch.bfloat16, (B, Smax, Hkv, d), True),
            _check_gpu("o", o, torch.bfloat16, (B, Sq, Hq, d), True),
            _check_gpu("lse", lse, torch.float32, (B, Hq, Sq))]
    return shape, ptrs


def attn_decode_noalloc(q, k_cache, v_cache, o, lse, scale: float, cache_lens=None, rope_base: float = 0.0):
    """attn_decode without a workspace: the library's static per-GPU scratch
    (ATTN_DECODE_SCRATCH_BYTES) holds the partials; nothing is allocated.
    Calls that overlap on one GPU race (the scratch is shared)."""
    shape, ptrs = _decode_args(q, k_cache, v_cache, o, lse, scale, cache_lens, rope_base)
    _call(load_library().attn_decode_noalloc, "attn_decode_noalloc", ctypes.byref(shape),
          *[ctypes.c_void_p(p) for p in ptrs], _stream())


def attn_decode(q, k_cache, v_cache, o, lse, scale: float, cache_lens=None, workspace=None, rope_base: float = 0.0):
    """O, LSE <- decode attention of q [B,Sq,Hq,d] against the caches [B,Smax,Hkv,d]
    (with rope_base > 0 the queries are rotated at their positions; the cache
    holds rotated keys)."""
    torch = _torch()
    shape, ptrs = _decode_args(q, k_cache, v_cache, o, lse, scale, cache_lens, rope_base)
    ws, nbytes = None, 0
    if workspace is not None:
        ws = _check_gpu("workspace", workspace, torch.uint8)
        nbytes = workspace.numel()
    _call(load_library().attn_decode, "attn_decode", ctypes.byref(shape), *[ctypes.c_void_p(p) for p in ptrs],
          ctypes.c_void_p(ws), ctypes.c_size_t(nbytes), _stream())


def decode(q, k_cache, v_cache, scale: Optional[float] = None, cache_lens=None, rope_base: float = 0.0):
    """Returns (O, LSE) of decode attention as new tensors (allocates the workspace)."""
    torch = _torch()
    B, Sq, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(B, Sq, k_cache.shape[1], Hq, k_cache.shape[2], d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    attn_decode(q, k_cache, v_cache, o, lse, scale, cache_lens, ws, rope_base)
    return o, lse


# ------------------------------------------------------------------ allocating conveniences

def forward(q, k, v, scale: Optional[float] = None, seqlens=None, causal: bool = True):
    """Returns (O, LSE) as new tensors."""
    torch = _torch()
    B, S, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, o, lse, scale, seqlens, int(causal))
    return o, lse


def rope(q, k, rope_base: float = 10000.0):
    """Returns (q_rot, k_rot) as new tensors."""
    torch = _torch()
    # q_rot shares q's strides and k_rot k's (one stride triple per group)
    q_rot = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    k_rot = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    attn_rope(q, k, q_rot, k_rot, rope_base)
    return q_rot, k_rot


def backward(q, k, v, o, d_o, lse, scale: Optional[float] = None, seqlens=None, causal: bool = True,
             rope_base: float = 0.0):
    """Returns (dQ, dK, dV, D) as new tensors (runs the preprocess, then the
    backward). With rope_base > 0, q and k are the rotated tensors from rope()
    and dQ, dK are the gradients with respect to the unrotated ones."""
    torch = _torch()
    B, S, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    delta = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    attn_bwd_preprocess(o, d_o, delta, seqlens)
    ws = bwd_workspace(q, k)
    # dQ shares dO's strides and dK, dV share K's (one stride triple per group)
    dq = torch.empty_strided(d_o.shape, d_o.stride(), dtype=q.dtype, device=q.device)
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    dv = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    attn_bwd(q, k, v, d_o, lse, delta, dq, dk, dv, scale, seqlens, ws, int(causal), rope_base)
    return dq, dk, dv, delta


# ------------------------------------------------------------------ graph capture

def capture_step(q, k, v, d_o, o, lse, delta, dq, dk, dv, scale: float, seqlens=None, causal: bool = True,
                 workspace=None, fused: bool = False, rope_base: float = 0.0, q_rot=None, k_rot=None):
    """Capture one training step of the path -- attn_fwd, attn_bwd_preprocess,
    attn_bwd (its dK/dV and dQ launches) -- into a HIP graph (torch.cuda.CUDAGraph)
    and return it; ``graph.replay()`` then reruns all four kernels with one
    launch, on the tensors given here (refill them in place between replays).

    The library is capture-safe: every entry point only enqueues kernels on the
    current stream (no allocation, no synchronisation, no memset), so the graph
    holds exactly the four kernel nodes (three with fused=True: attn_fwd then
    attn_bwd_fused; one more, the attn_rope pre-pass into q_rot / k_rot, with
    rope_base > 0). Shapes, pointers, scale, seqlens and causal are fixed at
    capture time."""
    cz = int(bool(causal))
    if rope_base and (q_rot is None or k_rot is None):
        raise ValueError("rope_base needs the q_rot and k_rot buffers")
    qa, ka = (q_rot, k_rot) if rope_base else (q, k)
    if workspace is None:
        workspace = bwd_workspace(q, k)  # allocated before the capture, bound to the graph

    def step():
        if rope_base:
            attn_rope(q, k, q_rot, k_rot, rope_base)
        attn_fwd(qa, ka, v, o, lse, scale, seqlens, cz)
        if fused:
            attn_bwd_fused(qa, ka, v, o, d_o, lse, delta, dq, dk, dv, scale, seqlens, workspace, cz, rope_base)
        else:
            attn_bwd_preprocess(o, d_o, delta, seqlens)
            attn_bwd(qa, ka, v, d_o, lse, delta, dq, dk, dv, scale, seqlens, workspace, cz, rope_base)
    graph = _capture(step)
    graph.attn_workspace = workspace  # kept alive as long as the graph
    return graph


def _capture(step):
    """One eager run of `step` on a side stream (loads the library and checks
    the arguments outside the capture), then the capture."""
    torch = _torch()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    return graph


def capture_decode(q, k_cache, v_cache, o, lse, scale: float, cache_lens=None, workspace=None,
                   rope_base: float = 0.0):
    """Capture one attn_decode call (its split and merge launches) into a HIP
    graph and return it. A serving loop refills q, the caches and cache_lens
    in place and replays; the workspace is bound at capture time (it must be
    at least attn_decode_workspace_bytes for these shapes)."""
    return _capture(lambda: attn_decode(q, k_cache, v_cache, o, lse, scale, cache_lens, workspace, rope_base))
