"""GPU parity of the forward's online softmax under score spikes.

The forward keeps, per row, a reference maximum it last rescaled to and takes
exponents against it; only when a tile's row maximum exceeds the reference by
more than 2^8 (base 2) are O and l rescaled. Random inputs almost never
rescale after the first tile; these cases plant score spikes in later tiles
(tens of nats above everything else the row sees, and moderate ones) so that
some waves of some blocks rescale late and others not, and compare the
forward's outputs with the oracle at the usual tolerances. Only the forward's
outputs are compared: the planted keys are large (|k| up to ~240), and the
backward's absolute error bound is not meant for gradients of that size (the
backward kernels are checked elsewhere).
"""
import numpy as np
import pytest
import torch

from attn_workloads import make_inputs
from parity import TOL_LSE, TOL_MAX_ABS, TOL_REL_FRO, host_inputs, metrics, run_gpu, say

import oracle

pytestmark = pytest.mark.gpu


def plant_spikes(inp, rows, key, strength, heads=None):
    """Make query rows `rows` of every sequence (and the given heads) score
    `strength` (scaled, natural units) against key `key`, above everything
    else they see."""
    q, k = inp.q.float(), inp.k.float()
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    heads = range(Hq) if heads is None else heads
    for b in range(B):
        for h in heads:
            u = q[b, rows, h].mean(dim=0)
            u = u / u.norm()
            q[b, rows, h] = u * 4.0 + 0.05 * q[b, rows, h]
            k[b, key, h // G] = u * (strength / (4.0 * inp.scale))
    inp.q.copy_(q.to(torch.bfloat16))
    inp.k.copy_(k.to(torch.bfloat16))


CASES = [
    # B, S, Hq, Hkv, d, causal, spike rows, spike key, strength (natural units)
    (1, 300, 2, 1, 64, True, slice(200, 232), 150, 60.0),    # far past 2^20: starts over
    (2, 520, 4, 2, 64, False, slice(0, 16), 400, 60.0),
    (1, 260, 2, 2, 128, True, slice(130, 140), 129, 80.0),
    (1, 300, 2, 1, 64, True, slice(200, 232), 150, 10.0),    # 2^14: absorbed by the first path
    (2, 400, 4, 1, 64, True, slice(300, 301), 299, 13.0),
    # large-grid forward blocks (256 rows; at d=64 each wave holds two 32-row
    # query tiles): a late spike, one confined to the second tile of a wave
    # (rows 608-639 of block rows 512-767 are wave 1's second tile), a
    # bidirectional one and a d=128 one
    (2, 1000, 64, 16, 64, True, slice(600, 632), 590, 60.0),
    (2, 1000, 64, 16, 64, True, slice(610, 620), 600, 20.0),
    (2, 1000, 64, 16, 64, False, slice(0, 16), 900, 60.0),
    (1, 1000, 64, 16, 128, True, slice(700, 720), 650, 80.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_S{}_H{}-{}_d{}_{}_x{:g}".format(
    *c[:5], "causal" if c[5] else "bidir", c[8]))
def test_forward_with_score_spikes(case):
    B, S, Hq, Hkv, d, causal, rows, key, strength = case
    seed = 9100 + S + d + int(strength)
    say(f"softmax paths B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} causal={causal} rows={rows} key={key} "
        f"strength={strength} seed={seed}")
    inp = make_inputs(B, S, Hq, Hkv, d, seed)
    plant_spikes(inp, rows, key, strength, heads=[0])
    gpu = run_gpu(inp, causal=causal)
    q, k, v, do, sl = host_inputs(inp)
    ref = oracle.backward(q, k, v, do, inp.scale, sl, causal=causal)
    # the spike dominates the planted rows: their outputs are (nearly) v_key
    r0 = rows.start
    if not causal or r0 >= key:
        assert np.max(np.abs(ref["O"][0, r0, 0] - v[0, key, 0])) < 0.05
    rel, mx = metrics(gpu["O"], ref["O"])
    assert np.all(np.isfinite(gpu["O"]))
    assert rel <= TOL_REL_FRO and mx <= TOL_MAX_ABS, f"O: rel_fro={rel:.3e} max_abs={mx:.3e}"
    lse = np.asarray(ref["LSE"], dtype=np.float64)
    fin = np.isfinite(lse)
    assert np.array_equal(np.isneginf(gpu["LSE"]), np.isneginf(lse))
    lmx = float(np.max(np.abs(gpu["LSE"][fin] - lse[fin])))
    assert lmx <= TOL_LSE, f"LSE: max_abs={lmx:.3e}"
    say(f"  spikes: O rel={rel:.2e} max={mx:.2e}  LSE max={lmx:.2e}")
