"""GPU: attn_decode_noalloc, the allocation-free decode entry point.

It must give exactly attn_decode's results (same kernels, same work split; its
partials live in the library's static per-GPU scratch instead of a caller
workspace), on two calls in a row with the second smaller than the first (the
scratch keeps the previous call's contents), and both must meet the oracle's
parity bar. A problem whose workspace would exceed the scratch is refused
before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import causal_attention_fwd_amd as attn
import oracle
from attn_workloads import make_decode_inputs
from parity import TOL_LSE, TOL_MAX_ABS, TOL_REL_FRO, metrics, say

pytestmark = pytest.mark.gpu


def _run_both(inp, rope_base=0.0):
    dev = torch.device("cuda")
    q = inp.q.to(dev).contiguous()
    k = inp.k_cache.to(dev).contiguous()
    v = inp.v_cache.to(dev).contiguous()
    lens = inp.cache_lens.to(dev) if inp.cache_lens is not None else None
    ref_o, ref_l = attn.decode(q, k, v, inp.scale, lens, rope_base)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"), device=dev)
    attn.attn_decode_noalloc(q, k, v, o, lse, inp.scale, lens, rope_base)
    torch.cuda.synchronize()
    return o, lse, ref_o, ref_l


def _check_oracle(o, lse, inp, label):
    lens = inp.cache_lens.numpy() if inp.cache_lens is not None else None
    ro, rl = oracle.decode(inp.q.float().numpy(), inp.k_cache.float().numpy(), inp.v_cache.float().numpy(),
                           inp.scale, lens)
    go, gl = o.float().cpu().numpy(), lse.float().cpu().numpy()
    rel, mx = metrics(go, ro)
    assert rel <= TOL_REL_FRO and mx <= TOL_MAX_ABS, f"{label} O: rel_fro={rel:.3e} max_abs={mx:.3e}"
    rl = np.asarray(rl, dtype=np.float64)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{label}: LSE -inf pattern differs"
    fin = np.isfinite(rl)
    lmx = float(np.max(np.abs(gl[fin] - rl[fin]))) if np.any(fin) else 0.0
    assert lmx <= TOL_LSE, f"{label} LSE: max_abs={lmx:.3e}"
    say(f"  {label}: O rel={rel:.2e} max={mx:.2e} LSE max={lmx:.2e}")


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def test_noalloc_decode_matches_workspace_decode_twice_shrinking():
    # first call: a serving-sized batch of mixed lengths; second: a smaller one
    cases = [(16, 2, 6000, 32, 8, 64, (1000, 6000), 8101), (3, 1, 900, 8, 2, 128, (0, 900), 8102)]
    for B, Sq, Smax, Hq, Hkv, d, rng, seed in cases:
        say(f"noalloc decode B={B} Sq={Sq} Smax={Smax} Hq={Hq} Hkv={Hkv} d={d} lens={rng} seed={seed}")
        need = attn.attn_decode_workspace_bytes(B, Sq, Smax, Hq, Hkv, d)
        assert 0 < need <= 32 << 20
        inp = make_decode_inputs(B, Sq, Smax, Hq, Hkv, d, seed, rng)
        o, lse, ref_o, ref_l = _run_both(inp)
        np.testing.assert_array_equal(_bits(o), _bits(ref_o))
        np.testing.assert_array_equal(_bits(lse), _bits(ref_l))
        _check_oracle(o, lse, inp, f"noalloc B={B} Smax={Smax}")


def test_noalloc_decode_refuses_problems_beyond_its_scratch():
    B, Sq, Smax, Hq, Hkv, d = 64, 64, 64, 64, 64, 128
    need = attn.attn_decode_workspace_bytes(B, Sq, Smax, Hq, Hkv, d)
    assert need > 32 << 20
    dev = torch.device("cuda")
    q = torch.zeros(B, Sq, Hq, d, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(B, Smax, Hkv, d, dtype=torch.bfloat16, device=dev)
    o = torch.zeros_like(q)
    lse = torch.zeros(B, Hq, Sq, device=dev)
    with pytest.raises(attn.AttnError) as ei:
        attn.attn_decode_noalloc(q, kc, kc, o, lse, 1.0 / d ** 0.5)
    assert ei.value.code == 4
    assert float(o.abs().max()) == 0.0  # nothing was enqueued
