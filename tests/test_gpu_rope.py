"""GPU parity of rotary position embedding with attention.

attn_rope rotates q and k once (compared with the oracle's fp64 rotation up to
the bf16 rounding of its output, also at positions past 2^16 where the angle
must be reduced accurately); the forward and backward then run on the rotated
tensors with rope_base set, and the backward's dQ and dK leave through the
rotation's adjoint. Whole steps are compared with oracle.rope.backward
(pinned in test_oracle_rope.py) with the rotated q and k stored in bf16 as the
bf16 pipeline stores them (unrounded, the bf16 rounding of the rotated inputs
alone moves LSE by up to ~1e-2), at the parity tolerances of the training
path.
"""
import numpy as np
import pytest
import torch

import causal_attention_fwd_amd as attn
from attn_workloads import make_inputs
from parity import compare, say, slice_unit

import oracle
from oracle import rope as oracle_rope

pytestmark = pytest.mark.gpu

BASE = 10000.0


def run_gpu_rope(inp, causal=True, base=BASE):
    dev = torch.device("cuda")
    q, k, v, do = (getattr(inp, n).to(dev).contiguous() for n in ("q", "k", "v", "do"))
    sl = inp.seqlens.to(dev) if inp.seqlens is not None else None
    q_rot, k_rot = attn.rope(q, k, base)
    o, lse = attn.forward(q_rot, k_rot, v, inp.scale, sl, causal=causal)
    dq, dk, dv, delta = attn.backward(q_rot, k_rot, v, o, do, lse, inp.scale, sl, causal=causal, rope_base=base)
    torch.cuda.synchronize()
    host = lambda x: x.float().cpu().numpy()  # noqa: E731
    return {"O": host(o), "LSE": host(lse), "D": host(delta), "dQ": host(dq), "dK": host(dk), "dV": host(dv),
            "Qrot": host(q_rot), "Krot": host(k_rot)}


def check_rotation(got, ref, label):
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    # bf16 rounding of the output (half an ulp: 2^-9 relative) plus fp32 and
    # hardware sine/cosine error far below it
    bound = np.abs(ref) * 2.0 ** -8 + 1e-5 * (np.max(np.abs(ref)) + 1e-30)
    worst = float(np.max(err - bound))
    assert worst <= 0.0, f"{label}: rotation error exceeds bf16 rounding by {worst:.3e}"
    say(f"  {label}: max |err| = {float(np.max(err)):.3e}")


@pytest.mark.parametrize("B,S,H,d", [(2, 300, 3, 64), (1, 70000, 1, 128), (1, 65, 2, 128)])
def test_rotation_matches_oracle(B, S, H, d):
    say(f"rope rotation B={B} S={S} H={H} d={d}")
    gen = torch.Generator().manual_seed(S + d)
    x = torch.randn(B, S, H, d, generator=gen).bfloat16()
    y = torch.randn(B, S, 1, d, generator=gen).bfloat16()
    dev = torch.device("cuda")
    qr, kr = attn.rope(x.to(dev), y.to(dev), BASE)
    torch.cuda.synchronize()
    check_rotation(qr.float().cpu().numpy(), oracle_rope.rotate(x.float().numpy(), BASE), "q_rot")
    check_rotation(kr.float().cpu().numpy(), oracle_rope.rotate(y.float().numpy(), BASE), "k_rot")


def test_rotation_other_base():
    gen = torch.Generator().manual_seed(3)
    x = torch.randn(1, 500, 2, 64, generator=gen).bfloat16()
    dev = torch.device("cuda")
    qr, kr = attn.rope(x.to(dev), x[:, :, :1].contiguous().to(dev), 500000.0)
    torch.cuda.synchronize()
    check_rotation(qr.float().cpu().numpy(), oracle_rope.rotate(x.float().numpy(), 500000.0), "q_rot base 5e5")


FUZZ = [
    # B, S, Hq, Hkv, d, causal, padded-length range or None
    (1, 1, 1, 1, 64, True, None),
    (2, 63, 4, 2, 64, True, None),
    (1, 65, 2, 2, 128, True, None),
    (3, 127, 8, 1, 64, False, None),
    (2, 200, 6, 2, 128, True, (1, 200)),
    (3, 300, 4, 1, 64, True, (0, 300)),
    (2, 257, 2, 2, 128, False, (100, 257)),
]


@pytest.mark.parametrize("case", FUZZ, ids=lambda c: "B{}_S{}_H{}-{}_d{}_{}_{}".format(
    *c[:5], "causal" if c[5] else "bidir", "pad" if c[6] else "dense"))
def test_rope_attention_every_element(case):
    B, S, Hq, Hkv, d, causal, rng = case
    seed = 8000 + B * 7 + S * 13 + Hq * 17 + d
    say(f"rope case B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} causal={causal} pad={rng} seed={seed}")
    inp = make_inputs(B, S, Hq, Hkv, d, seed, padded=rng is not None, seqlen_range=rng)
    gpu = run_gpu_rope(inp, causal)
    q, k, v, do = (getattr(inp, n).float().numpy() for n in ("q", "k", "v", "do"))
    sl = inp.seqlens.numpy() if inp.seqlens is not None else None
    ref = oracle_rope.backward(q, k, v, do, inp.scale, sl, BASE, causal=causal, bf16_storage=True)
    compare(gpu, ref, f"rope{case}")
    check_rotation(gpu["Qrot"], oracle_rope.rotate(q, BASE), "q_rot")
    check_rotation(gpu["Krot"], oracle_rope.rotate(k, BASE), "k_rot")


@pytest.mark.timeout(600)
def test_rope_llama1b_units():
    B, S, Hq, Hkv, d = 4, 2048, 32, 8, 64
    say(f"rope large B={B} S={S} Hq={Hq} Hkv={Hkv} d={d}")
    inp = make_inputs(B, S, Hq, Hkv, d, 20260003, do_sigma=0.1)
    gpu = run_gpu_rope(inp)
    q, k, v, do = (getattr(inp, n).float().numpy() for n in ("q", "k", "v", "do"))
    G = Hq // Hkv
    for b, g in [(0, 0), (3, 7)]:
        hs = slice(g * G, (g + 1) * G)
        ref = oracle_rope.backward(q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1],
                                   do[b:b + 1, :, hs], inp.scale, None, BASE, bf16_storage=True)
        compare(slice_unit(gpu, b, g, G), ref, f"rope-llama1b[b={b},g={g}]")


def test_rope_zero_base_is_plain_attention():
    # rope_base = 0 in the backward leaves dQ and dK as the plain kernels give them
    inp = make_inputs(1, 130, 2, 1, 64, 91)
    dev = torch.device("cuda")
    q, k, v, do = (getattr(inp, n).to(dev).contiguous() for n in ("q", "k", "v", "do"))
    o, lse = attn.forward(q, k, v, inp.scale)
    a = attn.backward(q, k, v, o, do, lse, inp.scale)
    b = attn.backward(q, k, v, o, do, lse, inp.scale, rope_base=0.0)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ref = oracle.backward(*(getattr(inp, n).float().numpy() for n in ("q", "k", "v", "do")), inp.scale)
    np.testing.assert_allclose(a[0].float().cpu().numpy(), ref["dQ"], atol=5e-2, rtol=0)
