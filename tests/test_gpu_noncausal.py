"""GPU parity of bidirectional (non-causal) attention, causal = 0 in the ABI.

The same kernels with no tile skipping and no diagonal mask, against the
oracle's causal=False path (pinned in test_oracle_noncausal.py): small shapes
element by element, larger ones on whole (sequence, kv head) units, plus the
padding contract.
"""
import numpy as np
import pytest

from attn_workloads import make_inputs
from parity import compare, host_inputs, oracle_unit, run_gpu, say, slice_unit

import oracle

pytestmark = pytest.mark.gpu

FUZZ = [
    # B, S, Hq, Hkv, d, padded-length range or None
    (1, 1, 1, 1, 64, None),
    (1, 17, 2, 1, 64, None),
    (2, 63, 4, 2, 64, None),
    (1, 65, 2, 2, 128, None),
    (3, 127, 8, 1, 64, None),
    (2, 129, 6, 2, 64, None),
    (1, 200, 8, 2, 128, None),
    (3, 300, 4, 1, 64, (0, 300)),
    (3, 257, 2, 2, 128, (1, 257)),
    (2, 1000, 6, 3, 64, (500, 1000)),
    # large-grid forward and dQ blocks, ragged lengths (as in the causal fuzz)
    (2, 1000, 64, 16, 64, (500, 1000)),
    (1, 1000, 64, 16, 128, (700, 1000)),
]


@pytest.mark.parametrize("case", FUZZ, ids=lambda c: "B{}_S{}_H{}-{}_d{}_{}".format(*c[:5], "pad" if c[5] else "dense"))
def test_noncausal_every_element(case):
    B, S, Hq, Hkv, d, rng = case
    seed = 5000 + B * 7 + S * 13 + Hq * 17 + d
    say(f"non-causal case B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} pad={rng} seed={seed}")
    inp = make_inputs(B, S, Hq, Hkv, d, seed, padded=rng is not None, seqlen_range=rng)
    gpu = run_gpu(inp, causal=False)
    q, k, v, do, sl = host_inputs(inp)
    compare(gpu, oracle.backward(q, k, v, do, inp.scale, sl, causal=False), f"noncausal{case}")


@pytest.mark.parametrize("B,S,Hq,Hkv,d,padded,units", [
    (2, 1024, 12, 4, 64, False, [(0, 0), (1, 3)]),
    (4, 2048, 32, 8, 64, False, [(0, 0), (3, 7)]),
    (2, 4096, 16, 16, 128, True, [(0, 0), (1, 15)]),
])
@pytest.mark.timeout(600)
def test_noncausal_large_units(B, S, Hq, Hkv, d, padded, units):
    seed = 6000 + B + S + Hq + d
    say(f"non-causal large B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} padded={padded} seed={seed}")
    inp = make_inputs(B, S, Hq, Hkv, d, seed, padded=padded)
    gpu = run_gpu(inp, causal=False)
    G = Hq // Hkv
    for b, hkv in units:
        say(f"  unit b={b} kv_head={hkv}")
        ref = oracle_unit(inp, b, hkv, np.float64, causal=False)
        compare(slice_unit(gpu, b, hkv, G), ref, f"noncausal-large[b={b},g={hkv}]")
    if inp.seqlens is not None:
        for b, L in enumerate(inp.seqlens.tolist()):
            for key in ("O", "dQ", "dK", "dV"):
                assert np.all(gpu[key][b, L:] == 0.0), (key, b)
            assert np.all(np.isneginf(gpu["LSE"][b, :, L:]))


def test_noncausal_nan_padding_and_last_row():
    say("non-causal contract: NaN-filled padding, and the last valid row equals the causal one")
    B, S, Hq, Hkv, d = 3, 333, 4, 2, 128
    inp = make_inputs(B, S, Hq, Hkv, d, 37, padded=True, seqlen_range=(100, 300))
    clean = run_gpu(inp, causal=False)
    causal = run_gpu(inp, causal=True)
    for b, L in enumerate(inp.seqlens.tolist()):
        # row L-1 sees every valid key in both forms (same kernel arithmetic up to tile order)
        np.testing.assert_allclose(clean["O"][b, L - 1], causal["O"][b, L - 1], atol=2e-2, rtol=0)
        np.testing.assert_allclose(clean["LSE"][b, :, L - 1], causal["LSE"][b, :, L - 1], atol=1e-5, rtol=0)
    assert np.max(np.abs(clean["O"][:, 0] - causal["O"][:, 0])) > 1e-2
    for name in ("q", "k", "v", "do"):
        x = getattr(inp, name)
        for b, L in enumerate(inp.seqlens.tolist()):
            x[b, L:] = float("nan")
    dirty = run_gpu(inp, causal=False)
    for key in clean:
        np.testing.assert_array_equal(clean[key], dirty[key], err_msg=key)
