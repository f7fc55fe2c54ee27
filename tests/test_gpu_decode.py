"""GPU parity of decode attention (attn_decode) against oracle.decode.

Split-KV partials plus their log-sum-exp merge, compared element by element
with the oracle's fp64 definition (pinned in test_oracle_decode.py) on seeded
inputs: cache lengths that are full, ragged, zero or shorter than the number
of new queries, one to 32 query rows per kv head, both head sizes, caches long
enough for many splits, and the serving-batch workload at its full size.
Tolerances are those of the training path: O relative Frobenius error <= 1e-2
and max |err| <= 5e-2; LSE identical -inf pattern and max |err| <= 1e-3.
"""
import numpy as np
import pytest
import torch

import causal_attention_fwd_amd as attn
from attn_workloads import DECODE_WORKLOADS, decode_workload_inputs, make_decode_inputs
from parity import TOL_LSE, TOL_MAX_ABS, TOL_REL_FRO, metrics, say

import oracle
from oracle import rope as oracle_rope

pytestmark = pytest.mark.gpu


def run_decode(inp, rope_base=0.0):
    dev = torch.device("cuda")
    q = inp.q.to(dev).contiguous()
    k = inp.k_cache.to(dev).contiguous()
    v = inp.v_cache.to(dev).contiguous()
    lens = inp.cache_lens.to(dev) if inp.cache_lens is not None else None
    o, lse = attn.decode(q, k, v, inp.scale, lens, rope_base)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.float().cpu().numpy()


def ref_decode(inp, rope_base=0.0):
    lens = inp.cache_lens.numpy() if inp.cache_lens is not None else None
    args = (inp.q.float().numpy(), inp.k_cache.float().numpy(), inp.v_cache.float().numpy(), inp.scale, lens)
    if rope_base:
        # the rotated queries are bf16 tensors in the pipeline
        return oracle_rope.decode(*args, base=rope_base, bf16_storage=True)
    return oracle.decode(*args)


def check(got, ref, label):
    o, lse = got
    ro, rl = ref
    assert np.all(np.isfinite(o)), f"{label}: non-finite O"
    rel, mx = metrics(o, ro)
    assert rel <= TOL_REL_FRO and mx <= TOL_MAX_ABS, f"{label} O: rel_fro={rel:.3e} max_abs={mx:.3e}"
    rl = np.asarray(rl, dtype=np.float64)
    assert not np.any(np.isnan(lse)) and not np.any(np.isposinf(lse)), f"{label}: bad LSE"
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl)), f"{label}: LSE -inf pattern differs"
    fin = np.isfinite(rl)
    lmx = float(np.max(np.abs(lse[fin] - rl[fin]))) if np.any(fin) else 0.0
    assert lmx <= TOL_LSE, f"{label} LSE: max_abs={lmx:.3e}"
    # rows that see no key: O exactly zero
    for b, h, t in zip(*np.nonzero(np.isneginf(rl))):
        assert np.all(o[b, t, h] == 0.0)
    say(f"  {label}: O rel={rel:.2e} max={mx:.2e}  LSE max={lmx:.2e}")


CASES = [
    # B, Sq, Smax, Hq, Hkv, d, cache-length range or None (full)
    (1, 1, 1, 1, 1, 64, None),
    (2, 1, 100, 8, 2, 64, None),
    (3, 1, 1000, 32, 8, 64, (0, 1000)),
    (2, 4, 300, 16, 4, 128, (1, 300)),
    (4, 8, 513, 8, 2, 64, (0, 12)),
    (2, 3, 777, 10, 2, 64, (2, 777)),
    (1, 32, 200, 1, 1, 64, None),
    (2, 2, 4096, 4, 4, 128, None),
    (3, 1, 5000, 12, 4, 128, (64, 5000)),
    (5, 16, 129, 4, 2, 128, (10, 129)),
    # one unit shared by every wave (over a thousand partials to merge)
    (1, 1, 131072, 8, 1, 64, None),
    (2, 1, 70000, 16, 2, 128, (30000, 70000)),
    # more than 32 query rows per kv head: several 32-row blocks per head
    (2, 33, 300, 1, 1, 64, (20, 300)),
    (3, 8, 700, 32, 4, 64, (0, 700)),
    (2, 16, 1000, 8, 1, 128, (5, 1000)),
    (1, 100, 257, 4, 2, 64, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Sq{}_S{}_H{}-{}_d{}_{}".format(
    *c[:6], "ragged" if c[6] else "full"))
def test_decode_every_element(case):
    B, Sq, Smax, Hq, Hkv, d, rng = case
    seed = 7000 + B * 3 + Sq * 5 + Smax * 7 + Hq * 11 + d
    say(f"decode case B={B} Sq={Sq} Smax={Smax} Hq={Hq} Hkv={Hkv} d={d} lens={rng} seed={seed}")
    inp = make_decode_inputs(B, Sq, Smax, Hq, Hkv, d, seed, rng)
    check(run_decode(inp), ref_decode(inp), f"decode{case}")


def test_decode_zero_lengths_and_garbage_beyond_length():
    say("decode contract: zero-length caches, NaN-filled cache beyond the length")
    B, Sq, Smax, Hq, Hkv, d = 4, 2, 700, 8, 2, 64
    inp = make_decode_inputs(B, Sq, Smax, Hq, Hkv, d, 71, (0, 700))
    inp.cache_lens[:] = torch.tensor([0, 1, 333, 700], dtype=torch.int32)
    clean = run_decode(inp)
    check(clean, ref_decode(inp), "decode-lens[0,1,333,700]")
    assert np.all(np.isneginf(clean[1][0])) and np.all(clean[0][0] == 0.0)
    for b, L in enumerate(inp.cache_lens.tolist()):
        inp.k_cache[b, L:] = float("nan")
        inp.v_cache[b, L:] = float("nan")
    dirty = run_decode(inp)
    np.testing.assert_array_equal(clean[0], dirty[0])
    np.testing.assert_array_equal(clean[1], dirty[1])


def test_decode_lengths_out_of_range_are_clamped():
    say("decode contract: cache lengths below 0 and above Smax are clamped")
    inp = make_decode_inputs(3, 1, 256, 4, 1, 64, 73, (0, 256))
    inp.cache_lens[:] = torch.tensor([-5, 999, 100], dtype=torch.int32)
    got = run_decode(inp)
    check(got, ref_decode(inp), "decode-clamped")
    assert np.all(np.isneginf(got[1][0]))


def test_decode_matches_full_cache_when_lengths_are_none():
    inp = make_decode_inputs(2, 1, 300, 4, 2, 64, 79, None)
    a = run_decode(inp)
    inp.cache_lens = torch.full((2,), 300, dtype=torch.int32)
    b = run_decode(inp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.timeout(600)
def test_decode_serving_workload_full_size():
    w = DECODE_WORKLOADS["decode_llama1b"]
    say(f"decode workload {w.describe()}")
    inp = decode_workload_inputs(w)
    check(run_decode(inp), ref_decode(inp), w.name)


def test_decode_deterministic_and_workspace_reuse():
    inp = make_decode_inputs(3, 4, 2000, 16, 4, 64, 83, (100, 2000))
    a = run_decode(inp)
    b = run_decode(inp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    # a second, smaller call into the same (dirty) workspace
    dev = torch.device("cuda")
    ws = torch.empty(attn.attn_decode_workspace_bytes(3, 4, 2000, 16, 4, 64), dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)
    outs = []
    for B, Smax in ((3, 2000), (1, 500)):
        small = make_decode_inputs(B, 4, Smax, 16, 4, 64, 89 + B, (1, Smax))
        q, k, v = (x.to(dev).contiguous() for x in (small.q, small.k_cache, small.v_cache))
        o = torch.empty_like(q)
        lse = torch.empty((B, 16, 4), dtype=torch.float32, device=dev)
        attn.attn_decode(q, k, v, o, lse, small.scale, small.cache_lens.to(dev), ws)
        torch.cuda.synchronize()
        check((o.float().cpu().numpy(), lse.cpu().numpy()), ref_decode(small), f"decode-reuse B={B}")


ROPE_CASES = [
    (2, 1, 500, 8, 2, 64, (1, 500)),
    (3, 4, 300, 16, 4, 128, (0, 300)),
    (2, 2, 70000, 16, 8, 64, (60000, 70000)),
    (1, 40, 128, 4, 1, 64, None),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: "B{}_Sq{}_S{}_H{}-{}_d{}".format(*c[:6]))
def test_decode_with_rope_every_element(case):
    B, Sq, Smax, Hq, Hkv, d, rng = case
    seed = 7700 + B + Sq + Smax + d
    say(f"decode rope case B={B} Sq={Sq} Smax={Smax} Hq={Hq} Hkv={Hkv} d={d} lens={rng} seed={seed}")
    inp = make_decode_inputs(B, Sq, Smax, Hq, Hkv, d, seed, rng)
    check(run_decode(inp, 10000.0), ref_decode(inp, 10000.0), f"decode-rope{case}")


def test_decode_rope_matches_rotated_queries_without_rope():
    # the kernel's own rotation equals rotating the queries (attn_rope at the
    # same positions) and decoding without it: here every sequence is full,
    # so query t sits at position Smax - Sq + t
    B, Sq, Smax, Hq, Hkv, d = 2, 3, 200, 8, 2, 64
    inp = make_decode_inputs(B, Sq, Smax, Hq, Hkv, d, 7799, None)
    dev = torch.device("cuda")
    q = inp.q.to(dev)
    padded = torch.zeros(B, Smax, Hq, d, dtype=torch.bfloat16, device=dev)
    padded[:, Smax - Sq:] = q
    kdummy = torch.zeros(B, Smax, Hkv, d, dtype=torch.bfloat16, device=dev)
    q_rot, _ = attn.rope(padded, kdummy, 10000.0)
    inp_rot = make_decode_inputs(B, Sq, Smax, Hq, Hkv, d, 7799, None)
    inp_rot.q = q_rot[:, Smax - Sq:].contiguous().cpu()
    a = run_decode(inp, 10000.0)
    b = run_decode(inp_rot, 0.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_decode_head_major_cache_and_views(rope_base):
    # caches stored head-major ([B, Hkv, Smax, d], a permuted view here), q a
    # view into a wider buffer: bitwise equal to the dense layout
    B, Sq, Smax, Hq, Hkv, d = 3, 2, 900, 16, 4, 64
    inp = make_decode_inputs(B, Sq, Smax, Hq, Hkv, d, 7900, (1, Smax))
    dev = torch.device("cuda")
    kh = inp.k_cache.to(dev).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    vh = inp.v_cache.to(dev).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert kh.stride() == (Hkv * Smax * d, d, Smax * d, 1)
    wide = torch.zeros(B, Sq, Hq + 5, d, dtype=torch.bfloat16, device=dev)
    wide[:, :, :Hq] = inp.q.to(dev)
    q = wide[:, :, :Hq]
    lens = inp.cache_lens.to(dev)
    o, lse = attn.decode(q, kh, vh, inp.scale, lens, rope_base)
    od, lsed = attn.decode(inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev), inp.scale, lens, rope_base)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), od.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lsed.view(torch.int32))
    check((o.float().cpu().numpy(), lse.cpu().numpy()), ref_decode(inp, rope_base), "decode-head-major")
