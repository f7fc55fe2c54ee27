"""CPU oracle for causal scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP kernels and never receives a value produced by
them.

What it computes (the plain definition, materialising every probability):
  * "Axis" (Zyora Labs page), feature list: fused flash attention forward and
    backward whose probabilities never reach memory; bf16 storage with fp32
    accumulation. The fused method reaches the same result as the plain
    softmax attention below up to rounding order, so the oracle is that plain
    definition written out, in fp64 by default.
  * "Axis" (Rust/cuTile page), "Training building blocks": the attention program
    is causal attention checked by central differences; "Conformance with
    PyTorch": operators are checked against an independent oracle
    reimplemented from the documented formula.
  * "AxiomLM" (PyPI page), "Key Features": grouped-query attention, kv heads
    shared by consecutive groups of query heads (head h reads kv head h // G).
  * "Axis" (Rust/cuTile page), "Sudoku as an acceptance test": its transformer
    uses bidirectional multi-head attention, the same softmax attention with
    no causal restriction (``causal=False`` below: every key of the valid
    prefix, j < L, enters every row's sum instead of j <= i).

The pages never print the formula; this is the textbook reading. For one
sequence with valid prefix length L (right padding) and one query head:
  s_ij  = scale * <q_i, k_j>                 for j <= i < L
  LSE_i = log sum_{j <= i} exp(s_ij)         (-inf on padded rows i >= L)
  P_ij  = exp(s_ij) / sum_{j' <= i} exp(s_ij'), 0 for j > i and outside [0, L)
  O_i   = sum_{j <= i} P_ij v_j              (0 on padded rows)
  D_i   = <dO_i, O_i>                        (0 on padded rows)
  dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i)
  dQ_i  = scale * sum_j dS_ij k_j
  dK_j  = scale * sum_{h in group} sum_i dS_ij q_i
  dV_j  = sum_{h in group} sum_i P_ij dO_i
With causal=False every "j <= i" above reads "j < L".
These are the exact gradients of f = sum(O * dO) with respect to Q, K, V.
Only positions inside the valid prefix ever enter a sum, so whatever a padded
position holds (even NaN) cannot reach an output.

Layouts: Q, O, dO, dQ are [B, S, Hq, d]; K, V, dK, dV are [B, S, Hkv, d];
LSE and D are [B, Hq, S]. ``seqlens`` (length-B integers or None) gives each
sequence's valid prefix length L_b; values are clamped into [0, S].
"""
from __future__ import annotations

import numpy as np

__all__ = ["forward", "backward", "preprocess", "probabilities", "lengths", "decode"]


def lengths(B: int, S: int, seqlens):
    """Valid prefix length of each sequence, clamped into [0, S]."""
    if seqlens is None:
        return [S] * B
    vals = [int(x) for x in np.asarray(seqlens).reshape(-1).tolist()]
    if len(vals) != B:
        raise ValueError("seqlens must have one entry per sequence")
    return [min(max(x, 0), S) for x in vals]


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("Q, K, V must be [B, S, H, d]")
    B, S, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != S or k.shape[3] != d:
        raise ValueError("K and V must be [B, S, Hkv, d] matching Q")
    Hkv = k.shape[2]
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, S, Hq, Hkv, d


def probabilities(qh, kh, scale: float, dtype=np.float64, causal: bool = True):
    """Softmax of one (sequence, query head) over its valid prefix.

    qh, kh: [L, d] (the valid prefix only). Returns (P [L, L], lse [L]).
    Causal: every row i has at least the key j = 0, so every row is a proper
    distribution over keys 0..i; entries above the diagonal are exactly 0.
    Not causal: every row is a distribution over all L keys."""
    qh = np.asarray(qh, dtype=dtype)
    kh = np.asarray(kh, dtype=dtype)
    L = qh.shape[0]
    allowed = np.tril(np.ones((L, L), dtype=bool)) if causal else np.ones((L, L), dtype=bool)
    s = (qh @ kh.T) * dtype(scale)
    s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=1) if L > 0 else np.zeros((0,), dtype=dtype)
    e = np.exp(s - m[:, None])          # exactly 0 above the diagonal
    denom = np.sum(e, axis=1)
    P = e / denom[:, None]
    lse = m + np.log(denom)
    return P.astype(dtype), lse.astype(dtype)


def forward(q, k, v, scale: float, seqlens=None, dtype=np.float64, causal: bool = True):
    """Attention forward: returns (O [B,S,Hq,d], LSE [B,Hq,S]) in ``dtype``."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, S, Hq, Hkv, d = _check(q, k, v)
    G = Hq // Hkv
    lens = lengths(B, S, seqlens)
    O = np.zeros((B, S, Hq, d), dtype=dtype)
    LSE = np.full((B, Hq, S), -np.inf, dtype=dtype)
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            g = h // G
            P, lse = probabilities(q[b, :L, h, :], k[b, :L, g, :], scale, dtype, causal)
            O[b, :L, h, :] = P @ np.asarray(v[b, :L, g, :], dtype=dtype)
            LSE[b, h, :L] = lse
    return O, LSE


def preprocess(o, do, seqlens=None, dtype=np.float64):
    """Row dot product D[b, h, i] = <dO[b,i,h,:], O[b,i,h,:]> (0 on padded rows)."""
    o = np.asarray(o)
    do = np.asarray(do)
    if o.shape != do.shape or o.ndim != 4:
        raise ValueError("O and dO must be [B, S, Hq, d] of equal shape")
    B, S, Hq, d = o.shape
    lens = lengths(B, S, seqlens)
    D = np.zeros((B, Hq, S), dtype=dtype)
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            D[b, h, :L] = np.sum(np.asarray(do[b, :L, h, :], dtype=dtype)
                                 * np.asarray(o[b, :L, h, :], dtype=dtype), axis=1)
    return D


def backward(q, k, v, do, scale: float, seqlens=None, dtype=np.float64, causal: bool = True):
    """Attention backward from scratch (the forward is recomputed here).

    Returns a dict with O, LSE, D, dQ, dK, dV (all in ``dtype``)."""
    q, k, v, do = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(do)
    B, S, Hq, Hkv, d = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must match Q")
    G = Hq // Hkv
    lens = lengths(B, S, seqlens)
    O = np.zeros((B, S, Hq, d), dtype=dtype)
    LSE = np.full((B, Hq, S), -np.inf, dtype=dtype)
    D = np.zeros((B, Hq, S), dtype=dtype)
    dQ = np.zeros((B, S, Hq, d), dtype=dtype)
    dK = np.zeros((B, S, Hkv, d), dtype=dtype)
    dV = np.zeros((B, S, Hkv, d), dtype=dtype)
    sc = dtype(scale)
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            g = h // G
            qh = np.asarray(q[b, :L, h, :], dtype=dtype)
            kh = np.asarray(k[b, :L, g, :], dtype=dtype)
            vh = np.asarray(v[b, :L, g, :], dtype=dtype)
            doh = np.asarray(do[b, :L, h, :], dtype=dtype)
            P, lse = probabilities(qh, kh, scale, dtype, causal)
            oh = P @ vh
            Dh = np.sum(doh * oh, axis=1)
            dP = doh @ vh.T
            dS = P * (dP - Dh[:, None])
            O[b, :L, h, :] = oh
            LSE[b, h, :L] = lse
            D[b, h, :L] = Dh
            dQ[b, :L, h, :] = sc * (dS @ kh)
            dK[b, :L, g, :] += sc * (dS.T @ qh)
            dV[b, :L, g, :] += P.T @ doh
    return {"O": O, "LSE": LSE, "D": D, "dQ": dQ, "dK": dK, "dV": dV}


def decode(q, k_cache, v_cache, scale: float, cache_lens=None, dtype=np.float64):
    """Attention of a few new queries against a key/value cache (inference).

    "AxiomLM" (PyPI page), "Key Features" and "Zero-Overhead Inference &
    Streaming Generation": a state-cached key/value decode engine whose step
    touches only the cache, with grouped kv heads ("Benchmarks": 4-head GQA to
    shrink the cache). The pages give no formula; the plain reading: sequence
    b holds L_b cached positions, the last Sq of which belong to the Sq new
    queries (their keys and values are already in the cache), so query t sits
    at position p = L_b - Sq + t and attends to the cached keys j <= p (causal
    among the new queries; with Sq = 1 the query sees the whole cache):
      s_j = scale * <q_t, k_j>,  LSE_t = ln sum_{j <= p} exp(s_j),
      O_t = sum_{j <= p} exp(s_j - LSE_t) v_j.
    A query with p < 0 (L_b < Sq - t) sees no key: O_t = 0, LSE_t = -inf.

    q: [B, Sq, Hq, d]; k_cache, v_cache: [B, Smax, Hkv, d]; cache_lens:
    length-B integers (clamped into [0, Smax]) or None (= Smax).
    Returns (O [B, Sq, Hq, d], LSE [B, Hq, Sq]) in ``dtype``."""
    q, k_cache, v_cache = np.asarray(q), np.asarray(k_cache), np.asarray(v_cache)
    if q.ndim != 4 or k_cache.ndim != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, Sq, Hq, d] and the caches [B, Smax, Hkv, d]")
    B, Sq, Hq, d = q.shape
    Bc, Smax, Hkv, dc = k_cache.shape
    if Bc != B or dc != d or Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("cache shape does not match q")
    G = Hq // Hkv
    lens = lengths(B, Smax, cache_lens)
    O = np.zeros((B, Sq, Hq, d), dtype=dtype)
    LSE = np.full((B, Hq, Sq), -np.inf, dtype=dtype)
    sc = dtype(scale)
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            g = h // G
            for t in range(Sq):
                p = L - Sq + t
                if p < 0:
                    continue
                kk = np.asarray(k_cache[b, :p + 1, g, :], dtype=dtype)
                vv = np.asarray(v_cache[b, :p + 1, g, :], dtype=dtype)
                s_ = (kk @ np.asarray(q[b, t, h, :], dtype=dtype)) * sc
                m = np.max(s_)
                e = np.exp(s_ - m)
                den = np.sum(e)
                O[b, t, h, :] = (e / den) @ vv
                LSE[b, h, t] = m + np.log(den)
    return O, LSE
