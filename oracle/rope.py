"""CPU oracle for rotary position embedding (RoPE) in front of attention.

TEST INFRASTRUCTURE ONLY (like oracle/attention.py): only the tests, the smoke
check and the benchmark's CPU-baseline leg may use it, and it shares no code
with the HIP kernels.

What it computes. "AxiomLM" (PyPI page), "Key Features" lists rotary position
embeddings among its modern-architecture modules, and "8. Standalone Modern
Architectural Modules" precomputes the rotation frequencies for a head size and
a maximum position (dim=64, end=1024) and applies them to q [2,1024,12,64] and
k [2,1024,4,64] before attention. The pages print no formula and no base; the
plain reading is the original rotary embedding with complex-style pairs
(the name of the precomputed table, freqs_cis, is that of the complex form):
  element pairs (x_2i, x_2i+1), i < d/2,
  frequency     theta_i = base^(-2i/d), base = 10000,
  angle         a = p * theta_i at token position p (0 for the first token),
  rotation      x'_2i   = x_2i cos a - x_2i+1 sin a
                x'_2i+1 = x_2i sin a + x_2i+1 cos a,
applied to every query and key head; values are not rotated. The rotation is
orthogonal, so its adjoint (what the backward pass applies to the gradients
of the rotated q and k) is the rotation by -a.

Gradients: with q_r = R q and k_r = R k, attention's dQ_r and dK_r map back to
dQ = R^T dQ_r and dK = R^T dK_r; dV is unchanged.

Storage. In a bf16 pipeline ("Axis", Zyora Labs page, feature list: bf16
storage, fp32 accumulation) the rotated q and k are tensors like any other and
are stored in bf16 before attention reads them. ``bf16_storage=True`` rounds
them to the nearest bf16 value (ties to even) at that point; the rest stays in
the oracle's precision.
"""
from __future__ import annotations

import numpy as np

from . import attention

__all__ = ["ROPE_BASE", "frequencies", "rotate", "round_bf16", "forward", "backward", "decode"]

ROPE_BASE = 10000.0


def frequencies(d: int, base: float = ROPE_BASE) -> np.ndarray:
    """theta_i = base^(-2i/d) for i = 0 .. d/2 - 1 (fp64)."""
    if d % 2:
        raise ValueError("RoPE needs an even head size")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d)


def rotate(x, base: float = ROPE_BASE, positions=None, inverse: bool = False, dtype=np.float64):
    """Rotate the pairs of x [B, S, H, d] by position * theta_i.

    positions: length-S token positions (default 0 .. S-1). inverse=True
    rotates by the negative angle (the adjoint)."""
    x = np.asarray(x, dtype=dtype)
    B, S, H, d = x.shape
    pos = np.arange(S, dtype=np.float64) if positions is None else np.asarray(positions, dtype=np.float64)
    ang = np.outer(pos, frequencies(d, base))          # [S, d/2]
    if inverse:
        ang = -ang
    c = np.cos(ang).astype(dtype)[None, :, None, :]
    s = np.sin(ang).astype(dtype)[None, :, None, :]
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


def round_bf16(x):
    """Nearest bf16 value (8 significant bits, ties to even) of each finite
    normal-range element, kept in x's dtype."""
    x = np.asarray(x)
    m, e = np.frexp(x)                     # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e).astype(x.dtype)


def _rotated(q, k, base, dtype, bf16_storage):
    qr, kr = rotate(q, base, dtype=dtype), rotate(k, base, dtype=dtype)
    if bf16_storage:
        qr, kr = round_bf16(qr), round_bf16(kr)
    return qr, kr


def forward(q, k, v, scale: float, seqlens=None, base: float = ROPE_BASE, dtype=np.float64, causal: bool = True,
            bf16_storage: bool = False):
    """Attention of the rotated q and k (oracle/attention.py's forward)."""
    qr, kr = _rotated(q, k, base, dtype, bf16_storage)
    return attention.forward(qr, kr, v, scale, seqlens, dtype=dtype, causal=causal)


def backward(q, k, v, do, scale: float, seqlens=None, base: float = ROPE_BASE, dtype=np.float64,
             causal: bool = True, bf16_storage: bool = False):
    """Forward and backward of attention(rope(q), rope(k), v).

    Returns oracle/attention.py's backward dict with dQ and dK taken back
    through the rotation's adjoint (gradients with respect to the unrotated
    q and k), plus the rotated inputs as "Qrot" and "Krot"."""
    qr, kr = _rotated(q, k, base, dtype, bf16_storage)
    ref = attention.backward(qr, kr, v, do, scale, seqlens, dtype=dtype, causal=causal)
    ref["dQ"] = rotate(ref["dQ"], base, inverse=True, dtype=dtype)
    ref["dK"] = rotate(ref["dK"], base, inverse=True, dtype=dtype)
    ref["Qrot"], ref["Krot"] = qr, kr
    return ref


def decode(q, k_cache, v_cache, scale: float, cache_lens=None, base: float = ROPE_BASE, dtype=np.float64,
           bf16_storage: bool = False):
    """Decode attention (oracle/attention.py's decode) with the new queries
    rotated at their positions: query t of sequence b sits at position
    p = L_b - Sq + t, the position its key was rotated at when it entered the
    cache, so the cache holds keys already rotated and is used as it is.
    ``bf16_storage`` rounds the rotated queries to bf16 (see the header)."""
    q = np.asarray(q, dtype=dtype)
    B, Sq, Hq, d = q.shape
    lens = attention.lengths(B, np.asarray(k_cache).shape[1], cache_lens)
    qr = np.empty_like(q)
    for b in range(B):
        pos = lens[b] - Sq + np.arange(Sq)
        qr[b:b + 1] = rotate(q[b:b + 1], base, positions=pos, dtype=dtype)
    if bf16_storage:
        qr = round_bf16(qr)
    return attention.decode(qr, k_cache, v_cache, scale, cache_lens, dtype=dtype)
