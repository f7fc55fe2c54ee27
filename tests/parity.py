"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare.

Tolerances (per tensor, over the compared slice):
  O, dQ, dK, dV : relative Frobenius error <= 1e-2 and max |gpu - ref| <= 5e-2
  LSE           : identical -inf pattern, max |gpu - ref| <= 1e-3 on finite rows
  D             : relative Frobenius error <= 1e-2 (D is computed from the bf16 O)
and no NaN/Inf anywhere in the GPU outputs except LSE's -inf on padded rows.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import causal_attention_fwd_amd as attn
import oracle

TOL_REL_FRO = 1e-2
TOL_MAX_ABS = 5e-2
TOL_LSE = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu(inp):
    dev = torch.device("cuda")
    t = {k: getattr(inp, k).to(dev).contiguous() for k in ("q", "k", "v", "do")}
    t["seqlens"] = inp.seqlens.to(dev) if inp.seqlens is not None else None
    return t


def run_gpu(inp, t=None, causal=True, bench_order=False):
    """fwd -> preprocess -> bwd on the GPU; returns host fp32 numpy arrays.
    bench_order: the benchmark's launch sequence instead, fwd ->
    attn_bwd_dq_delta (dQ, forming D) -> attn_bwd_dkdv (reading that D)."""
    t = t or to_gpu(inp)
    o, lse = attn.forward(t["q"], t["k"], t["v"], inp.scale, t["seqlens"], causal=causal)
    if bench_order:
        delta = torch.full_like(lse, float("nan"))
        dq = torch.full_like(t["q"], float("nan"))
        dk, dv = torch.full_like(t["k"], float("nan")), torch.full_like(t["v"], float("nan"))
        attn.attn_bwd_dq_delta(t["q"], t["k"], t["v"], o, t["do"], lse, delta, dq, inp.scale, t["seqlens"],
                               int(causal))
        attn.attn_bwd_dkdv(t["q"], t["k"], t["v"], t["do"], lse, delta, dk, dv, inp.scale, t["seqlens"],
                           int(causal))
    else:
        dq, dk, dv, delta = attn.backward(t["q"], t["k"], t["v"], o, t["do"], lse, inp.scale, t["seqlens"],
                                          causal=causal)
    torch.cuda.synchronize()
    host = lambda x: x.float().cpu().numpy()  # noqa: E731
    return {"O": host(o), "LSE": host(lse), "D": host(delta), "dQ": host(dq), "dK": host(dk), "dV": host(dv)}


def host_inputs(inp):
    q, k, v, do = (x.float().numpy() for x in (inp.q, inp.k, inp.v, inp.do))
    sl = inp.seqlens.numpy() if inp.seqlens is not None else None
    return q, k, v, do, sl


def oracle_unit(inp, b, hkv, dtype=np.float64, causal=True):
    """Oracle on one (sequence, kv head) unit: the kv head and its query-head group."""
    q, k, v, do, sl = host_inputs(inp)
    G = q.shape[2] // k.shape[2]
    hs = slice(hkv * G, (hkv + 1) * G)
    sub_sl = None if sl is None else sl[b:b + 1]
    ref = oracle.backward(q[b:b + 1, :, hs], k[b:b + 1, :, hkv:hkv + 1], v[b:b + 1, :, hkv:hkv + 1],
                          do[b:b + 1, :, hs], inp.scale, sub_sl, dtype=dtype, causal=causal)
    return ref


def slice_unit(gpu, b, hkv, G):
    hs = slice(hkv * G, (hkv + 1) * G)
    return {"O": gpu["O"][b:b + 1, :, hs], "dQ": gpu["dQ"][b:b + 1, :, hs],
            "dK": gpu["dK"][b:b + 1, :, hkv:hkv + 1], "dV": gpu["dV"][b:b + 1, :, hkv:hkv + 1],
            "LSE": gpu["LSE"][b:b + 1, hs], "D": gpu["D"][b:b + 1, hs]}


def metrics(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    return float(rel), float(np.max(np.abs(diff))) if diff.size else 0.0


def compare(gpu, ref, label=""):
    """Assert the parity bar; returns a dict of the measured errors."""
    report = {}
    for key in ("O", "dQ", "dK", "dV"):
        g = gpu[key]
        assert np.all(np.isfinite(g)), f"{label} {key}: non-finite GPU values"
        rel, mx = metrics(g, ref[key])
        report[key] = (rel, mx)
        assert rel <= TOL_REL_FRO and mx <= TOL_MAX_ABS, f"{label} {key}: rel_fro={rel:.3e} max_abs={mx:.3e}"
    g, r = gpu["LSE"], np.asarray(ref["LSE"], dtype=np.float64)
    assert not np.any(np.isnan(g)), f"{label} LSE: NaN"
    assert np.array_equal(np.isneginf(g), np.isneginf(r)), f"{label} LSE: -inf pattern differs"
    assert not np.any(np.isposinf(g)), f"{label} LSE: +inf"
    fin = np.isfinite(r)
    mx = float(np.max(np.abs(g[fin] - r[fin]))) if np.any(fin) else 0.0
    report["LSE"] = (0.0, mx)
    assert mx <= TOL_LSE, f"{label} LSE: max_abs={mx:.3e}"
    assert np.all(np.isfinite(gpu["D"])), f"{label} D: non-finite"
    rel, mx = metrics(gpu["D"], ref["D"])
    report["D"] = (rel, mx)
    assert rel <= TOL_REL_FRO, f"{label} D: rel_fro={rel:.3e}"
    say(f"  {label}: " + "  ".join(f"{k} rel={v[0]:.2e} max={v[1]:.2e}" for k, v in report.items()))
    return report


def whole_output_identities(inp, gpu, causal=True, label=""):
    """Checks over every (sequence, kv head) unit at any size, on the GPU's
    outputs (host arrays) in fp64:
      * D_i = sum_c dO_ic O_ic from the GPU's own bf16 O (to fp32 summation);
      * every O row lies in the range of the V rows it sees (prefix for
        causal), widened by the bf16 roundings of P and O;
      * sum_j dV_j = sum over the group's heads of sum_i dO_i, and
        sum_j dK_j = 0 (every valid row of P sums to one and sum_j dS_ij = 0),
        within a multiple of the bf16 rounding noise.
    A skipped or repeated tile, a wrong mask, LSE or D breaks one of them."""
    q, k, v, do, sl = host_inputs(inp)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    O, D, dK, dV = (np.asarray(gpu[n], dtype=np.float64) for n in ("O", "D", "dK", "dV"))
    worst = {"D": 0.0, "O": 0.0, "dV": 0.0, "dK": 0.0}
    for b in range(B):
        L = int(sl[b]) if sl is not None else S
        if L == 0:
            continue
        dob = do[b, :L].astype(np.float64)                     # [L, Hq, d]
        ob = O[b, :L]
        prod = dob * ob
        dref = prod.sum(axis=-1).T                              # [Hq, L]
        dtol = 1e-5 * np.abs(prod).sum(axis=-1).T + 1e-30
        err = np.abs(D[b, :, :L] - dref)
        assert np.all(err <= dtol), f"{label} D: b={b} max err {err.max():.3e}"
        worst["D"] = max(worst["D"], float((err / dtol).max()))
        for g in range(Hkv):
            vb = v[b, :L, g].astype(np.float64)                 # [L, d]
            if causal:
                hi, lo = np.maximum.accumulate(vb, axis=0), np.minimum.accumulate(vb, axis=0)
            else:
                hi, lo = np.broadcast_to(vb.max(axis=0), vb.shape), np.broadcast_to(vb.min(axis=0), vb.shape)
            tol = 2.0 ** -7 * float(np.abs(vb).max())
            hs = slice(g * G, (g + 1) * G)
            og = ob[:, hs]                                      # [L, G, d]
            over = max(float((og - hi[:, None]).max()), float((lo[:, None] - og).max()))
            assert over <= tol, f"{label} O outside the range of its visible V rows: b={b} g={g} by {over:.3e}"
            worst["O"] = max(worst["O"], over / tol)
            sdv = dV[b, :L, g].sum(axis=0)
            sdo = dob[:, hs].sum(axis=(0, 1))
            noise_v = (np.linalg.norm(dV[b, :L, g]) + np.linalg.norm(dob[:, hs])) * 2.0 ** -7
            ev = float(np.linalg.norm(sdv - sdo))
            assert ev <= noise_v, f"{label} sum dV != sum dO: b={b} g={g} {ev:.3e} > {noise_v:.3e}"
            worst["dV"] = max(worst["dV"], ev / noise_v)
            sdk = dK[b, :L, g].sum(axis=0)
            dterm = np.abs(prod[:, hs]).sum(axis=-1) * 2.0 ** -9          # [L, G]
            qn2 = (q[b, :L, hs].astype(np.float64) ** 2).sum(axis=-1)      # [L, G]
            noise_k = np.linalg.norm(dK[b, :L, g]) * 2.0 ** -7 + 4 * inp.scale * np.sqrt((dterm ** 2 * qn2).sum())
            ek = float(np.linalg.norm(sdk))
            assert ek <= noise_k, f"{label} sum dK != 0: b={b} g={g} {ek:.3e} > {noise_k:.3e}"
            worst["dK"] = max(worst["dK"], ek / noise_k)
    say(f"  {label} identities over every unit (largest fraction of its bound): "
        + "  ".join(f"{k} {v:.2f}" for k, v in worst.items()))

