"""GPU: the whole step captured in one HIP graph (torch.cuda.CUDAGraph).

The graph is replayed several times, with the program's own eager work, new
inputs copied in place and synchronisations between replays. Every replay is
checked twice: against the oracle (oracle.backward, oracle.rope.backward or
oracle.decode in fp64) on that replay's own inputs, to the parity bar of
tests/parity.py, and bit for bit against an eager run of the same entry
points on the same inputs (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import causal_attention_fwd_amd as attn
import oracle
from attn_workloads import make_inputs
from oracle import rope as oracle_rope
from parity import compare, say


def _oracle_step(inp, causal, rope_base):
    """The oracle's forward and backward on one replay's inputs (host fp64)."""
    q, k, v, do = (getattr(inp, n).float().numpy() for n in ("q", "k", "v", "do"))
    sl = inp.seqlens.numpy() if inp.seqlens is not None else None
    if rope_base:
        # the rotated q and k are bf16 tensors in the pipeline
        return oracle_rope.backward(q, k, v, do, inp.scale, sl, rope_base, causal=causal, bf16_storage=True)
    return oracle.backward(q, k, v, do, inp.scale, sl, causal=causal)

pytestmark = pytest.mark.gpu


def _eager(t, scale, sl, causal, fused=False, rope_base=0.0):
    q, k = attn.rope(t["q"], t["k"], rope_base) if rope_base else (t["q"], t["k"])
    o, lse = attn.forward(q, k, t["v"], scale, sl, causal=causal)
    if fused:
        delta = torch.empty_like(lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(t["v"])
        attn.attn_bwd_fused(q, k, t["v"], o, t["do"], lse, delta, dq, dk, dv, scale, sl, None, int(causal),
                            rope_base)
    else:
        dq, dk, dv, delta = attn.backward(q, k, t["v"], o, t["do"], lse, scale, sl, causal=causal,
                                          rope_base=rope_base)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "D": delta, "dQ": dq, "dK": dk, "dV": dv}


@pytest.mark.parametrize("causal,padded,fused,rope_base,large", [(True, False, False, 0.0, False),
                                                                 (True, True, False, 0.0, False),
                                                                 (False, True, False, 0.0, False),
                                                                 (True, True, True, 0.0, False),
                                                                 (True, False, False, 10000.0, False),
                                                                 (True, True, True, 10000.0, False),
                                                                 (True, True, False, 0.0, True)])
def test_graph_replays_match_eager(causal, padded, fused, rope_base, large):
    # large: enough blocks for the large-grid forward and dQ kernels
    B, S, Hq, Hkv, d = (2, 1000, 64, 16, 64) if large else (2, 384, 8, 2, 64)
    say(f"graph capture: B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} causal={causal} padded={padded} fused={fused} "
        f"rope={rope_base}")
    dev = torch.device("cuda")
    rng = (500, 1000) if large else (200, 384)
    inputs = [make_inputs(B, S, Hq, Hkv, d, 900 + i, padded=padded, seqlen_range=rng) for i in range(3)]
    # buffers the graph is bound to
    buf = {n: getattr(inputs[0], n).to(dev).contiguous() for n in ("q", "k", "v", "do")}
    sl = inputs[0].seqlens.to(dev) if padded else None
    o = torch.empty_like(buf["q"])
    lse = torch.empty(B, Hq, S, device=dev)
    delta = torch.empty(B, Hq, S, device=dev)
    dq, dk, dv = torch.empty_like(buf["q"]), torch.empty_like(buf["k"]), torch.empty_like(buf["v"])
    scale = inputs[0].scale
    q_rot, k_rot = (torch.empty_like(buf["q"]), torch.empty_like(buf["k"])) if rope_base else (None, None)
    graph = attn.capture_step(buf["q"], buf["k"], buf["v"], buf["do"], o, lse, delta, dq, dk, dv, scale, sl, causal,
                              fused=fused, rope_base=rope_base, q_rot=q_rot, k_rot=k_rot)
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
        host = {key: val.float().cpu().numpy() for key, val in got.items()}
        compare(host, _oracle_step(inp, causal, rope_base), f"replay {rep} vs oracle")
        # eager work between replays, on separate tensors
        t = {n: getattr(inp, n).to(dev).contiguous() for n in ("q", "k", "v", "do")}
        ref = _eager(t, scale, inp.seqlens.to(dev) if padded else None, causal, fused, rope_base)
        for key in got:
            bits = torch.int16 if got[key].dtype == torch.bfloat16 else torch.int32
            np.testing.assert_array_equal(got[key].view(bits).cpu().numpy(), ref[key].view(bits).cpu().numpy(),
                                          err_msg=f"replay {rep} {key}")
        say(f"  replay {rep}: all six outputs bitwise equal to eager")


def _check_decode_oracle(o, lse, inp, rope_base, label):
    from parity import TOL_LSE, TOL_MAX_ABS, TOL_REL_FRO, metrics
    lens = inp.cache_lens.numpy() if inp.cache_lens is not None else None
    args = (inp.q.float().numpy(), inp.k_cache.float().numpy(), inp.v_cache.float().numpy(), inp.scale, lens)
    ro, rl = (oracle_rope.decode(*args, base=rope_base, bf16_storage=True) if rope_base else oracle.decode(*args))
    go, gl = o.float().cpu().numpy(), lse.float().cpu().numpy()
    assert np.all(np.isfinite(go)), f"{label}: non-finite O"
    rel, mx = metrics(go, ro)
    assert rel <= TOL_REL_FRO and mx <= TOL_MAX_ABS, f"{label} O: rel_fro={rel:.3e} max_abs={mx:.3e}"
    rl = np.asarray(rl, dtype=np.float64)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{label}: LSE -inf pattern differs"
    fin = np.isfinite(rl)
    lmx = float(np.max(np.abs(gl[fin] - rl[fin]))) if np.any(fin) else 0.0
    assert lmx <= TOL_LSE, f"{label} LSE: max_abs={lmx:.3e}"
    say(f"  {label}: O rel={rel:.2e} max={mx:.2e} LSE max={lmx:.2e}")


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_decode_graph_replays_match_eager(rope_base):
    from attn_workloads import make_decode_inputs
    B, Sq, Smax, Hq, Hkv, d = 8, 2, 3000, 16, 4, 64
    say(f"decode graph capture: B={B} Sq={Sq} Smax={Smax} rope={rope_base}")
    dev = torch.device("cuda")
    inputs = [make_decode_inputs(B, Sq, Smax, Hq, Hkv, d, 950 + i, (1, Smax)) for i in range(3)]
    q = inputs[0].q.to(dev).contiguous()
    kc, vc = inputs[0].k_cache.to(dev).contiguous(), inputs[0].v_cache.to(dev).contiguous()
    lens = inputs[0].cache_lens.to(dev)
    o, lse = torch.empty_like(q), torch.empty(B, Hq, Sq, device=dev)
    ws = torch.empty(attn.attn_decode_workspace_bytes(B, Sq, Smax, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    scale = inputs[0].scale
    graph = attn.capture_decode(q, kc, vc, o, lse, scale, lens, ws, rope_base)
    for rep in range(6):
        inp = inputs[rep % 3]
        q.copy_(inp.q.to(dev))
        kc.copy_(inp.k_cache.to(dev))
        vc.copy_(inp.v_cache.to(dev))
        lens.copy_(inp.cache_lens.to(dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = o.clone(), lse.clone()
        _check_decode_oracle(got_o, got_l, inp, rope_base, f"decode replay {rep} vs oracle")
        ro, rl = attn.decode(inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev), scale,
                             inp.cache_lens.to(dev), rope_base)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got_o.view(torch.int16).cpu().numpy(), ro.view(torch.int16).cpu().numpy())
        np.testing.assert_array_equal(got_l.view(torch.int32).cpu().numpy(), rl.view(torch.int32).cpu().numpy())
        say(f"  decode replay {rep}: bitwise equal to eager")
