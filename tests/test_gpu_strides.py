"""GPU parity of strided tensors (the shape's q/kv/o stride triples).

The kernels address every row through (sequence, position, head) strides, so
views give the same arithmetic as dense copies: these tests compare strided
runs bitwise with runs on contiguous copies of the same values, and with the
oracle. Layouts: Q, K, V as views into one fused projection output
[B, S, Hq + 2 Hkv, d] (gradients into a fused buffer of the same layout), O /
dO / dQ with padding between positions and every other sequence of a larger
batch, and the RoPE pre-pass on views.
"""
import numpy as np
import pytest
import torch

import causal_attention_fwd_amd as attn
from attn_workloads import make_inputs
from parity import compare, host_inputs, say

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def dense_run(q, k, v, do, scale, sl, causal=True, rope_base=0.0):
    q, k, v, do = (x.contiguous() for x in (q, k, v, do))
    if rope_base:
        q, k = attn.rope(q, k, rope_base)
    o, lse = attn.forward(q, k, v, scale, sl, causal=causal)
    dq, dk, dv, delta = attn.backward(q, k, v, o, do, lse, scale, sl, causal=causal, rope_base=rope_base)
    return o, lse, dq, dk, dv


def same(a, b):
    assert torch.equal(a.contiguous().view(torch.int16) if a.dtype == torch.bfloat16 else a.contiguous(),
                       b.contiguous().view(torch.int16) if b.dtype == torch.bfloat16 else b.contiguous())


@pytest.mark.parametrize("B,S,Hq,Hkv,d,causal,padded", [
    (2, 300, 4, 2, 64, True, False),
    (1, 257, 8, 1, 128, True, True),
    (2, 200, 6, 3, 64, False, True),
    (2, 1000, 64, 16, 64, True, True),   # large-grid forward and dQ blocks
])
def test_fused_qkv_views(B, S, Hq, Hkv, d, causal, padded):
    say(f"fused qkv B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} causal={causal} padded={padded}")
    inp = make_inputs(B, S, Hq, Hkv, d, 4242 + S, padded=padded)
    H = Hq + 2 * Hkv
    fused = torch.empty(B, S, H, d, dtype=torch.bfloat16, device=DEV)
    fused[:, :, :Hq] = inp.q.to(DEV)
    fused[:, :, Hq:Hq + Hkv] = inp.k.to(DEV)
    fused[:, :, Hq + Hkv:] = inp.v.to(DEV)
    q, k, v = fused[:, :, :Hq], fused[:, :, Hq:Hq + Hkv], fused[:, :, Hq + Hkv:]
    do = inp.do.to(DEV)
    sl = inp.seqlens.to(DEV) if inp.seqlens is not None else None
    o, lse = attn.forward(q, k, v, inp.scale, sl, causal=causal)
    dfused = torch.zeros_like(fused)
    dq = torch.empty_like(do)
    dk, dv = dfused[:, :, Hq:Hq + Hkv], dfused[:, :, Hq + Hkv:]
    delta = torch.empty_like(lse)
    attn.attn_bwd_preprocess(o, do, delta, sl)
    attn.attn_bwd(q, k, v, do, lse, delta, dq, dk, dv, inp.scale, sl, None, int(causal))
    ref = dense_run(q, k, v, do, inp.scale, sl, causal)
    torch.cuda.synchronize()
    for got, want in zip((o, lse, dq, dk, dv), ref):
        same(got, want)
    # the query slots of the gradient buffer were never written
    assert torch.count_nonzero(dfused[:, :, :Hq]) == 0
    host = lambda x: x.float().cpu().numpy()  # noqa: E731
    gpu = {"O": host(o), "LSE": host(lse), "D": host(delta), "dQ": host(dq), "dK": host(dk), "dV": host(dv)}
    qn, kn, vn, don, sln = host_inputs(inp)
    compare(gpu, oracle.backward(qn, kn, vn, don, inp.scale, sln, causal=causal), "fused-qkv")


def test_padded_positions_and_batch_stride():
    B, S, Hq, Hkv, d = 2, 190, 4, 2, 64
    say(f"strided o/do/dq and every-other-sequence views B={B} S={S}")
    inp = make_inputs(2 * B, S, Hq, Hkv, d, 4343)
    qb, kb, vb, dob = (getattr(inp, n).to(DEV) for n in ("q", "k", "v", "do"))
    q, k, v, do_src = qb[::2], kb[::2], vb[::2], dob[::2]          # batch stride doubled
    big_o = torch.empty(B, S, Hq + 3, d, dtype=torch.bfloat16, device=DEV)  # padded positions
    big_do = torch.empty(B, S, Hq + 3, d, dtype=torch.bfloat16, device=DEV)
    big_dq = torch.empty(B, S, Hq + 3, d, dtype=torch.bfloat16, device=DEV)
    o, do, dq = big_o[:, :, :Hq], big_do[:, :, :Hq], big_dq[:, :, :Hq]
    do.copy_(do_src)
    lse = torch.empty(B, Hq, S, device=DEV)
    attn.attn_fwd(q, k, v, o, lse, inp.scale)
    delta = torch.empty_like(lse)
    attn.attn_bwd_preprocess(o, do, delta)
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=DEV)
    dv = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=DEV)
    attn.attn_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, inp.scale)
    attn.attn_bwd_dq(q, k, v, do, lse, delta, dq, inp.scale)
    ref = dense_run(q, k, v, do, inp.scale, None)
    torch.cuda.synchronize()
    for got, want in zip((o, lse, dq, dk, dv), ref):
        same(got, want)


def test_rope_on_views():
    B, S, Hq, Hkv, d = 2, 150, 4, 1, 64
    inp = make_inputs(B, S, Hq, Hkv, d, 4444)
    H = Hq + 2 * Hkv
    fused = torch.empty(B, S, H, d, dtype=torch.bfloat16, device=DEV)
    fused[:, :, :Hq] = inp.q.to(DEV)
    fused[:, :, Hq:Hq + Hkv] = inp.k.to(DEV)
    fused[:, :, Hq + Hkv:] = inp.v.to(DEV)
    q, k, v = fused[:, :, :Hq], fused[:, :, Hq:Hq + Hkv], fused[:, :, Hq + Hkv:]
    q_rot, k_rot = attn.rope(q, k, 10000.0)
    qd, kd = attn.rope(q.contiguous(), k.contiguous(), 10000.0)
    do = inp.do.to(DEV)
    o, lse = attn.forward(q_rot, k_rot, v, inp.scale)
    dq, dk, dv, _ = attn.backward(q_rot, k_rot, v, o, do, lse, inp.scale, rope_base=10000.0)
    ref = dense_run(q, k, v, do, inp.scale, None, True, 10000.0)
    torch.cuda.synchronize()
    same(q_rot, qd)
    same(k_rot, kd)
    for got, want in zip((o, lse, dq, dk, dv), ref):
        same(got, want)


def test_fused_backward_on_views():
    """attn_bwd_fused (dQ pass reading O for D) with every group strided: Q, K, V
    views into a projection output, O / dO / dQ views into one wider buffer,
    dK / dV into a gradient buffer of the projection's layout; bitwise equal to
    the same call on dense copies."""
    B, S, Hq, Hkv, d = 2, 260, 4, 2, 64
    say(f"fused backward on views B={B} S={S} Hq={Hq} Hkv={Hkv} d={d}")
    inp = make_inputs(B, S, Hq, Hkv, d, 4545, padded=True, seqlen_range=(70, 260))
    sl = inp.seqlens.to(DEV)
    H = Hq + 2 * Hkv
    proj = torch.empty(B, S, H, d, dtype=torch.bfloat16, device=DEV)
    proj[:, :, :Hq] = inp.q.to(DEV)
    proj[:, :, Hq:Hq + Hkv] = inp.k.to(DEV)
    proj[:, :, Hq + Hkv:] = inp.v.to(DEV)
    q, k, v = proj[:, :, :Hq], proj[:, :, Hq:Hq + Hkv], proj[:, :, Hq + Hkv:]
    obuf = torch.empty(B, S, 3 * Hq, d, dtype=torch.bfloat16, device=DEV)  # O | dO | dQ side by side
    o, do, dq = obuf[:, :, :Hq], obuf[:, :, Hq:2 * Hq], obuf[:, :, 2 * Hq:]
    do.copy_(inp.do.to(DEV))
    dproj = torch.zeros_like(proj)
    dk, dv = dproj[:, :, Hq:Hq + Hkv], dproj[:, :, Hq + Hkv:]
    lse = torch.empty(B, Hq, S, device=DEV)
    delta = torch.empty_like(lse)
    attn.attn_fwd(q, k, v, o, lse, inp.scale, sl)
    attn.attn_bwd_fused(q, k, v, o, do, lse, delta, dq, dk, dv, inp.scale, sl)
    # the same call on dense copies
    qc, kc, vc, doc = (x.contiguous() for x in (q, k, v, do))
    oc, lc = torch.empty_like(qc), torch.empty_like(lse)
    dc = torch.empty_like(lse)
    dqc, dkc, dvc = torch.empty_like(qc), torch.empty_like(kc), torch.empty_like(vc)
    attn.attn_fwd(qc, kc, vc, oc, lc, inp.scale, sl)
    attn.attn_bwd_fused(qc, kc, vc, oc, doc, lc, dc, dqc, dkc, dvc, inp.scale, sl)
    torch.cuda.synchronize()
    for got, want in zip((o, lse, delta, dq, dk, dv), (oc, lc, dc, dqc, dkc, dvc)):
        same(got, want)
    assert torch.count_nonzero(dproj[:, :, :Hq]) == 0
    host = lambda x: x.float().cpu().numpy()  # noqa: E731
    gpu = {"O": host(o), "LSE": host(lse), "D": host(delta), "dQ": host(dq), "dK": host(dk), "dV": host(dv)}
    qn, kn, vn, don, sln = host_inputs(inp)
    compare(gpu, oracle.backward(qn, kn, vn, don, inp.scale, sln), "fused-bwd-views")
