"""GPU: the whole step captured in one HIP graph (torch.cuda.CUDAGraph).

The graph is replayed several times, with the program's own eager work, new
inputs copied in place and synchronisations between replays, and every replay
is compared bit for bit with an eager run of the same entry points on the same
inputs (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import causal_attention_fwd_amd as attn
from attn_workloads import make_inputs
from parity import say

pytestmark = pytest.mark.gpu


def _eager(t, scale, sl, causal):
    o, lse = attn.forward(t["q"], t["k"], t["v"], scale, sl, causal=causal)
    dq, dk, dv, delta = attn.backward(t["q"], t["k"], t["v"], o, t["do"], lse, scale, sl, causal=causal)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "D": delta, "dQ": dq, "dK": dk, "dV": dv}


@pytest.mark.parametrize("causal,padded", [(True, False), (True, True), (False, True)])
def test_graph_replays_match_eager(causal, padded):
    B, S, Hq, Hkv, d = 2, 384, 8, 2, 64
    say(f"graph capture: B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} causal={causal} padded={padded}")
    dev = torch.device("cuda")
    inputs = [make_inputs(B, S, Hq, Hkv, d, 900 + i, padded=padded, seqlen_range=(200, 384)) for i in range(3)]
    # buffers the graph is bound to
    buf = {n: getattr(inputs[0], n).to(dev).contiguous() for n in ("q", "k", "v", "do")}
    sl = inputs[0].seqlens.to(dev) if padded else None
    o = torch.empty_like(buf["q"])
    lse = torch.empty(B, Hq, S, device=dev)
    delta = torch.empty(B, Hq, S, device=dev)
    dq, dk, dv = torch.empty_like(buf["q"]), torch.empty_like(buf["k"]), torch.empty_like(buf["v"])
    scale = inputs[0].scale
    graph = attn.capture_step(buf["q"], buf["k"], buf["v"], buf["do"], o, lse, delta, dq, dk, dv, scale, sl, causal)
    outs = {"O": o, "LSE": lse, "D": delta, "dQ": dq, "dK": dk, "dV": dv}
    for rep in range(6):
        inp = inputs[rep % 3]
        for n in ("q", "k", "v", "do"):
            buf[n].copy_(getattr(inp, n).to(dev))
        if padded:
            sl.copy_(inp.seqlens.to(dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {key: val.clone() for key, val in outs.items()}
        # eager work between replays, on separate tensors
        t = {n: getattr(inp, n).to(dev).contiguous() for n in ("q", "k", "v", "do")}
        ref = _eager(t, scale, inp.seqlens.to(dev) if padded else None, causal)
        for key in got:
            bits = torch.int16 if got[key].dtype == torch.bfloat16 else torch.int32
            np.testing.assert_array_equal(got[key].view(bits).cpu().numpy(), ref[key].view(bits).cpu().numpy(),
                                          err_msg=f"replay {rep} {key}")
        say(f"  replay {rep}: all six outputs bitwise equal to eager")
