"""Seeded synthetic workloads for causal attention (shared by tests and bench).

This module only draws random inputs, names the workload shapes and counts
(valid pairs, flops, bytes, the split dK/dV pass's workgroups per key block).
It holds none of the attention arithmetic, so both the CPU oracle and the GPU
path can take their inputs from here without sharing any of the method's code.

Shapes follow the pages' workloads:
  * tiny        - a single tile, two heads (a sanity case the oracle runs in ms)
  * gqa124m     - "AxiomLM" (PyPI page), the 124M-class GQA model config in
                  "Quick Start" (12 query heads, 4 kv heads, block 1024) and the
                  q/k shapes (2,1024,12,64)/(2,1024,4,64) in "8. Standalone
                  Modern Architectural Modules"
  * llama1b     - "Axis" (Zyora Labs page): compile_model(batch=4, seq=2048,
                  dtype="bf16"), 1B-class Llama with grouped kv heads (32/8)
  * padded      - a right-padded batch, valid length uniform in [S/2, S]
  * longseq     - one long 16K sequence; Axis (Zyora Labs) states that memory
                  stays flat as sequence length grows

Recipe (also stated in the design doc): generator = torch.Generator('cpu') seeded
with 20260000 + index (index 1..5 in the order above); draw Q, K, V, dO as
fp32 standard normals in [B, S, H, d] order, scale dO by its stated sigma,
round to bf16 (round-to-nearest-even), and for the padded workload draw the
per-sequence valid lengths last with randint(S//2, S+1).

Decode workloads (attention of a few new queries against a key/value cache):
  * decode_llama1b - the llama1b heads (32 query, 8 kv, d 64), 32 sequences,
                     cache capacity 8192, one new query each, cache lengths
                     uniform in [Smax/4, Smax] (a serving batch of mixed
                     lengths; the AxiomLM pages describe a cached-state decode
                     engine for grouped-kv-head models without sizes)
Recipe: generator seeded with 20260100 + index; draw q [B, Sq, Hq, d], then the
k and v caches [B, Smax, Hkv, d] as fp32 standard normals, round to bf16, then
the cache lengths with randint(lo, hi + 1).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed index (1-based)
    B: int
    S: int
    Hq: int
    Hkv: int
    d: int
    do_sigma: float = 1.0
    padded: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 20260000 + self.index

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "S": self.S, "Hq": self.Hq,
                "Hkv": self.Hkv, "d": self.d, "causal": True,
                "padded": self.padded, "dO_sigma": self.do_sigma}


WORKLOADS = {
    "tiny": Workload("tiny", 1, B=1, S=128, Hq=2, Hkv=2, d=64),
    "gqa124m": Workload("gqa124m", 2, B=2, S=1024, Hq=12, Hkv=4, d=64),
    "llama1b": Workload("llama1b", 3, B=4, S=2048, Hq=32, Hkv=8, d=64, do_sigma=0.1),
    "padded": Workload("padded", 4, B=8, S=4096, Hq=16, Hkv=16, d=128, padded=True),
    "longseq": Workload("longseq", 5, B=1, S=16384, Hq=32, Hkv=8, d=128),
}


@dataclasses.dataclass
class Inputs:
    q: torch.Tensor        # [B, S, Hq, d] bf16 (CPU)
    k: torch.Tensor        # [B, S, Hkv, d] bf16
    v: torch.Tensor        # [B, S, Hkv, d] bf16
    do: torch.Tensor       # [B, S, Hq, d] bf16
    seqlens: Optional[torch.Tensor]  # int32 [B] or None
    scale: float


def make_inputs(B: int, S: int, Hq: int, Hkv: int, d: int, seed: int,
                do_sigma: float = 1.0, padded: bool = False,
                scale: Optional[float] = None,
                seqlen_range: Optional[tuple] = None) -> Inputs:
    """Draw bf16-rounded N(0,1) inputs in the recipe's order.

    ``seqlen_range`` (lo, hi inclusive) overrides the default padded range
    [S//2, S]; it is used by edge-case tests (e.g. zero-length sequences).
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    q = torch.randn(B, S, Hq, d, generator=gen, dtype=torch.float32)
    k = torch.randn(B, S, Hkv, d, generator=gen, dtype=torch.float32)
    v = torch.randn(B, S, Hkv, d, generator=gen, dtype=torch.float32)
    do = torch.randn(B, S, Hq, d, generator=gen, dtype=torch.float32)
    if do_sigma != 1.0:
        do = do * do_sigma
    seqlens = None
    if padded:
        lo, hi = seqlen_range if seqlen_range is not None else (S // 2, S)
        seqlens = torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)
    return Inputs(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16),
                  v=v.to(torch.bfloat16), do=do.to(torch.bfloat16),
                  seqlens=seqlens, scale=(1.0 / math.sqrt(d)) if scale is None else float(scale))


def workload_inputs(w: Workload) -> Inputs:
    return make_inputs(w.B, w.S, w.Hq, w.Hkv, w.d, w.seed, do_sigma=w.do_sigma, padded=w.padded)


def valid_pairs(S: int, B: int, seqlens=None, causal: bool = True) -> int:
    """Number of (i, j) query/key pairs with j <= i < L_b (causal) or with
    i, j < L_b (bidirectional), summed over the batch.

    Pure counting (no attention arithmetic): used to price algorithmic work.
    """
    lens = [S] * B if seqlens is None else [int(L) for L in seqlens.tolist()]
    if causal:
        return int(sum(L * (L + 1) // 2 for L in lens))
    return int(sum(L * L for L in lens))


def algorithmic_flops(w_or_shape, seqlens=None, causal: bool = True) -> dict:
    """Algorithmic flop counts: 4*d per valid pair per query head (QK^T and PV)
    forward; backward 2.5x that (five GEMMs incl. the QK^T recompute).
    Per-kernel shares: dK/dV kernel 8*d (S, dP, dV, dK), dQ kernel 2*d (dQ)."""
    if isinstance(w_or_shape, Workload):
        B, S, Hq, d = w_or_shape.B, w_or_shape.S, w_or_shape.Hq, w_or_shape.d
    else:
        B, S, Hq, d = w_or_shape
    pairs = valid_pairs(S, B, seqlens, causal)
    fwd = 4.0 * d * Hq * pairs
    return {"pairs_per_head": pairs, "fwd": fwd, "bwd": 2.5 * fwd, "total": 3.5 * fwd,
            "bwd_dkdv": 2.0 * fwd, "bwd_dq": 0.5 * fwd}


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    index: int
    B: int
    Sq: int
    Smax: int
    Hq: int
    Hkv: int
    d: int
    len_lo: int
    len_hi: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 20260100 + self.index

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "Sq": self.Sq, "Smax": self.Smax, "Hq": self.Hq,
                "Hkv": self.Hkv, "d": self.d, "cache_len_range": [self.len_lo, self.len_hi]}


DECODE_WORKLOADS = {
    "decode_llama1b": DecodeWorkload("decode_llama1b", 1, B=32, Sq=1, Smax=8192, Hq=32, Hkv=8, d=64,
                                     len_lo=2048, len_hi=8192),
}


@dataclasses.dataclass
class DecodeInputs:
    q: torch.Tensor                  # [B, Sq, Hq, d] bf16 (CPU)
    k_cache: torch.Tensor            # [B, Smax, Hkv, d] bf16
    v_cache: torch.Tensor            # [B, Smax, Hkv, d] bf16
    cache_lens: Optional[torch.Tensor]  # int32 [B] or None (= Smax)
    scale: float


def make_decode_inputs(B: int, Sq: int, Smax: int, Hq: int, Hkv: int, d: int, seed: int,
                       len_range: Optional[tuple] = None, scale: Optional[float] = None) -> DecodeInputs:
    """Draw bf16-rounded N(0,1) decode inputs; ``len_range`` (lo, hi inclusive)
    draws per-sequence cache lengths, None leaves every cache full."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    q = torch.randn(B, Sq, Hq, d, generator=gen, dtype=torch.float32)
    k = torch.randn(B, Smax, Hkv, d, generator=gen, dtype=torch.float32)
    v = torch.randn(B, Smax, Hkv, d, generator=gen, dtype=torch.float32)
    lens = None
    if len_range is not None:
        lo, hi = len_range
        lens = torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)
    return DecodeInputs(q=q.to(torch.bfloat16), k_cache=k.to(torch.bfloat16), v_cache=v.to(torch.bfloat16),
                        cache_lens=lens, scale=(1.0 / math.sqrt(d)) if scale is None else float(scale))


def decode_workload_inputs(w: DecodeWorkload) -> DecodeInputs:
    return make_decode_inputs(w.B, w.Sq, w.Smax, w.Hq, w.Hkv, w.d, w.seed, (w.len_lo, w.len_hi))


def decode_bytes(B: int, Sq: int, Smax: int, Hq: int, Hkv: int, d: int, cache_lens=None) -> dict:
    """Algorithmic HBM bytes of one decode call: every valid cached key and
    value row read once (bf16), the queries read and the outputs written once
    (bf16), one fp32 LSE per query row. Pure counting."""
    lens = [Smax] * B if cache_lens is None else [min(max(int(L), 0), Smax) for L in cache_lens.tolist()]
    cache = sum(lens) * Hkv * d * 2 * 2
    qo = B * Sq * Hq * d * 2 * 2 + B * Sq * Hq * 4
    return {"cache": cache, "q_o_lse": qo, "total": cache + qo}


def dkdv_split_parts(B: int, S: int, Hq: int, Hkv: int, causal: bool = True) -> list:
    """Workgroups per 128-key block of the split dK/dV pass, from the rule the
    library documents (all ones when there is no split): each (sequence, kv
    head) gets parts * nkb workgroups, parts = min(ceil(256 / blocks), a quarter
    of the first block's (head, query tile) iterations, 8); every block gets
    one and the rest go in proportion to the blocks' query tiles (ceil(S/64) -
    2*kb under the causal mask, all equal without it). Pure counting, used to
    check the library's workspace size and to price its reduce pass."""
    nkb = (S + 127) // 128
    units = nkb * B * Hkv
    if units >= 256:
        return [1] * nkb
    parts = min((256 + units - 1) // units, max(1, (S + 63) // 64 * (Hq // Hkv) // 4), 8)
    n64 = (S + 63) // 64
    w = [n64 - 2 * kb if causal else 1 for kb in range(nkb)]
    extra = (parts - 1) * nkb
    cum, first = 0, []
    for kb in range(nkb + 1):
        first.append(kb + extra * cum // sum(w))
        if kb < nkb:
            cum += w[kb]
    return [first[kb + 1] - first[kb] for kb in range(nkb)]
