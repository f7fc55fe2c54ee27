"""CPU: the whole-output identities the full-size GPU parity tests apply to
every unit. They must hold for the oracle's own outputs stored as the GPU
stores them (bf16 O, dK, dV; D from that O in fp32), and fail for planted
mistakes of the kinds they exist to catch."""
import numpy as np
import pytest
import torch

import oracle
from attn_workloads import make_inputs
from parity import host_inputs, whole_output_identities


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _as_gpu(inp, causal=True):
    """Oracle outputs rounded as the GPU path stores them."""
    q, k, v, do, sl = host_inputs(inp)
    ref = oracle.backward(q, k, v, do, inp.scale, sl, causal=causal)
    out = {n: _bf16(ref[n]) for n in ("O", "dQ", "dK", "dV")}
    out["LSE"] = np.asarray(ref["LSE"], dtype=np.float32)
    # D from the stored (bf16) O, in fp32, zero on padded rows
    D = np.einsum("bshd,bshd->bhs", do.astype(np.float32), out["O"]).astype(np.float32)
    if sl is not None:
        for b, L in enumerate(sl.tolist()):
            D[b, :, L:] = 0.0
    out["D"] = D
    return out


CASES = [(2, 300, 4, 2, 64, None), (3, 257, 4, 1, 128, (60, 257))]


@pytest.mark.parametrize("case", CASES, ids=["dense_d64", "padded_d128"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "bidirectional"])
def test_identities_hold_for_the_oracle(case, causal):
    B, S, Hq, Hkv, d, rng = case
    inp = make_inputs(B, S, Hq, Hkv, d, 77, padded=rng is not None, seqlen_range=rng)
    whole_output_identities(inp, _as_gpu(inp, causal), causal=causal, label="oracle")


def _planted(kind, out, inp):
    out = {k: v.copy() for k, v in out.items()}
    if kind == "skipped key tile in dV":
        out["dV"][0, 64:128] = 0.0
    elif kind == "skipped key tile in dK":
        out["dK"][1, 128:192] = 0.0
    elif kind == "row sees a later key":
        # row 3 of head 0 (four visible keys) also attends key 200 with half the weight
        v = inp.v.float().numpy()
        out["O"][0, 3, 0] = _bf16(0.5 * out["O"][0, 3, 0] + 0.5 * v[0, 200, 0])
    elif kind == "D from the wrong O":
        out["D"][0, 1, 5] *= 1.01
    elif kind == "dK without the -D term":
        # dS = P dP instead of P (dP - D): dK_j gains scale * sum_h sum_i P_ij D_i Q_i
        q, k, v, do, sl = host_inputs(inp)
        B, S, Hq, _ = q.shape
        G = Hq // k.shape[2]
        lse = np.asarray(out["LSE"], dtype=np.float64)
        mask = np.tril(np.ones((S, S), dtype=bool))
        for b in range(B):
            for h in range(Hq):
                g = h // G
                s = inp.scale * q[b, :, h].astype(np.float64) @ k[b, :, g].astype(np.float64).T
                P = np.where(mask, np.exp(s - lse[b, h][:, None]), 0.0)
                extra = inp.scale * P.T @ (out["D"][b, h][:, None] * q[b, :, h].astype(np.float64))
                out["dK"][b, :, g] = _bf16(out["dK"][b, :, g] + extra)
    return out


@pytest.mark.parametrize("kind", ["skipped key tile in dV", "skipped key tile in dK", "row sees a later key",
                                  "D from the wrong O", "dK without the -D term"])
def test_identities_catch_planted_mistakes(kind):
    inp = make_inputs(2, 300, 4, 2, 64, 78)
    out = _planted(kind, _as_gpu(inp), inp)
    with pytest.raises(AssertionError):
        whole_output_identities(inp, out, label=kind)
