"""GPU parity of attn_bwd_fused (the backward preprocess folded into dQ).

The dQ pass computes D = rowsum(dO * O) from the O and dO rows it loads,
writes it, and the dK/dV pass reads it. Compared with the oracle at the
training path's tolerances, and with the separate preprocess + attn_bwd path:
D agrees to fp32 summation order, and so do the gradients.
"""
import numpy as np
import pytest
import torch

import causal_attention_fwd_amd as attn
from attn_workloads import make_inputs
from parity import compare, host_inputs, say

import oracle
from oracle import rope as oracle_rope

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def fused_run(inp, causal=True, rope_base=0.0):
    q, k, v, do = (getattr(inp, n).to(DEV).contiguous() for n in ("q", "k", "v", "do"))
    sl = inp.seqlens.to(DEV) if inp.seqlens is not None else None
    if rope_base:
        q, k = attn.rope(q, k, rope_base)
    o, lse = attn.forward(q, k, v, inp.scale, sl, causal=causal)
    delta = torch.full_like(lse, float("nan"))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    attn.attn_bwd_fused(q, k, v, o, do, lse, delta, dq, dk, dv, inp.scale, sl, None, int(causal), rope_base)
    sep = attn.backward(q, k, v, o, do, lse, inp.scale, sl, causal=causal, rope_base=rope_base)
    torch.cuda.synchronize()
    host = lambda x: x.float().cpu().numpy()  # noqa: E731
    got = {"O": host(o), "LSE": host(lse), "D": host(delta), "dQ": host(dq), "dK": host(dk), "dV": host(dv)}
    ref_sep = {"dQ": host(sep[0]), "dK": host(sep[1]), "dV": host(sep[2]), "D": host(sep[3])}
    return got, ref_sep


CASES = [
    # B, S, Hq, Hkv, d, causal, padded range
    (1, 1, 1, 1, 64, True, None),
    (2, 130, 4, 2, 64, True, None),
    (3, 257, 6, 3, 128, True, (0, 257)),
    (2, 300, 8, 2, 64, False, (100, 300)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_S{}_H{}-{}_d{}_{}".format(
    *c[:5], "causal" if c[5] else "bidir"))
def test_fused_backward(case):
    B, S, Hq, Hkv, d, causal, rng = case
    say(f"fused bwd B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} causal={causal} pad={rng}")
    inp = make_inputs(B, S, Hq, Hkv, d, 5150 + S + d, padded=rng is not None, seqlen_range=rng)
    got, sep = fused_run(inp, causal)
    q, k, v, do, sl = host_inputs(inp)
    compare(got, oracle.backward(q, k, v, do, inp.scale, sl, causal=causal), f"fused{case}")
    assert np.all(np.isfinite(got["D"]))
    np.testing.assert_allclose(got["D"], sep["D"], rtol=1e-5, atol=1e-6)
    for key in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(got[key], sep[key], rtol=0, atol=2e-2, err_msg=key)


def test_fused_backward_with_rope():
    inp = make_inputs(2, 200, 4, 1, 64, 5199)
    got, sep = fused_run(inp, True, 10000.0)
    q, k, v, do, sl = host_inputs(inp)
    ref = oracle_rope.backward(q, k, v, do, inp.scale, sl, 10000.0, bf16_storage=True)
    compare(got, ref, "fused-rope")


def test_fused_backward_rope_d128_padded_bidirectional():
    say("fused bwd with RoPE, d=128, padded, bidirectional")
    inp = make_inputs(2, 190, 4, 2, 128, 5211, padded=True, seqlen_range=(60, 190))
    got, sep = fused_run(inp, False, 10000.0)
    q, k, v, do, sl = host_inputs(inp)
    ref = oracle_rope.backward(q, k, v, do, inp.scale, sl, 10000.0, causal=False, bf16_storage=True)
    compare(got, ref, "fused-rope-d128-bidir")
    np.testing.assert_allclose(got["D"], sep["D"], rtol=1e-5, atol=1e-6)
    for key in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(got[key], sep[key], rtol=0, atol=2e-2, err_msg=key)


@pytest.mark.timeout(600)
def test_fused_backward_llama1b_units():
    B, S, Hq, Hkv, d = 4, 2048, 32, 8, 64
    say(f"fused bwd llama1b B={B} S={S}")
    inp = make_inputs(B, S, Hq, Hkv, d, 20260003, do_sigma=0.1)
    got, sep = fused_run(inp)
    np.testing.assert_allclose(got["D"], sep["D"], rtol=1e-5, atol=1e-6)
    q, k, v, do, sl = host_inputs(inp)
    G = Hq // Hkv
    for b, g in [(0, 0), (3, 7)]:
        hs = slice(g * G, (g + 1) * G)
        ref = oracle.backward(q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1],
                              do[b:b + 1, :, hs], inp.scale, None)
        unit = {"O": got["O"][b:b + 1, :, hs], "dQ": got["dQ"][b:b + 1, :, hs],
                "dK": got["dK"][b:b + 1, :, g:g + 1], "dV": got["dV"][b:b + 1, :, g:g + 1],
                "LSE": got["LSE"][b:b + 1, hs], "D": got["D"][b:b + 1, hs]}
        compare(unit, ref, f"fused-llama1b[b={b},g={g}]")


SPLIT_CASES = [
    # B, S, Hq, Hkv, d, causal, padded range, rope base
    (2, 130, 4, 2, 64, True, None, 0.0),
    (3, 257, 6, 3, 128, True, (0, 257), 0.0),
    (2, 300, 8, 2, 64, False, (100, 300), 10000.0),
    (2, 1000, 64, 16, 64, True, (500, 1000), 0.0),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B{}_S{}_H{}-{}_d{}_{}{}".format(
    *c[:5], "causal" if c[5] else "bidir", "_rope" if c[7] else ""))
def test_dq_delta_then_dkdv_is_the_fused_backward(case):
    """attn_bwd_dq_delta then attn_bwd_dkdv on one stream: the launches of
    attn_bwd_fused, so the same bits, and the oracle's gradients and D."""
    B, S, Hq, Hkv, d, causal, rng, rb = case
    say(f"dq_delta + dkdv B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} causal={causal} pad={rng} rope={rb}")
    inp = make_inputs(B, S, Hq, Hkv, d, 5300 + S + d, padded=rng is not None, seqlen_range=rng)
    q, k, v, do = (getattr(inp, n).to(DEV).contiguous() for n in ("q", "k", "v", "do"))
    sl = inp.seqlens.to(DEV) if inp.seqlens is not None else None
    if rb:
        q, k = attn.rope(q, k, rb)
    o, lse = attn.forward(q, k, v, inp.scale, sl, causal=causal)
    outs = []
    for split in (True, False):
        delta = torch.full_like(lse, float("nan"))
        dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
        if split:
            attn.attn_bwd_dq_delta(q, k, v, o, do, lse, delta, dq, inp.scale, sl, int(causal), rb)
            attn.attn_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, inp.scale, sl, int(causal), rb)
        else:
            attn.attn_bwd_fused(q, k, v, o, do, lse, delta, dq, dk, dv, inp.scale, sl, None, int(causal), rb)
        outs.append((delta, dq, dk, dv))
    torch.cuda.synchronize()
    for name, a, b in zip(("D", "dQ", "dK", "dV"), *outs):
        # bitwise: the bf16 / fp32 bit patterns (NaN-safe)
        bits = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(bits).cpu(), b.view(bits).cpu()), name
    host = lambda x: x.float().cpu().numpy()  # noqa: E731
    delta, dq, dk, dv = outs[0]
    got = {"O": host(o), "LSE": host(lse), "D": host(delta), "dQ": host(dq), "dK": host(dk), "dV": host(dv)}
    qh, kh, vh, doh, slh = host_inputs(inp)
    if rb:
        ref = oracle_rope.backward(qh, kh, vh, doh, inp.scale, slh, rb, causal=causal, bf16_storage=True)
    else:
        ref = oracle.backward(qh, kh, vh, doh, inp.scale, slh, causal=causal)
    compare(got, ref, f"dq_delta{case}")
