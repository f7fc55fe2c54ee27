"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small shapes are compared element by element over every output; the five
named workloads run at their full sizes, in the launch configuration the
benchmark times (and with the backward's other launch order, preprocess then
attn_bwd), and are compared on whole (sequence, kv head) units sampled
from the batch (all of llama1b's and longseq's), plus properties that
hold at any size over every unit (padding zeros, no NaN/Inf, D from the GPU's
O, O within the range of its visible V rows, the gradient sum identities).
"""
import numpy as np
import pytest
import torch

import causal_attention_fwd_amd as attn
from attn_workloads import WORKLOADS, make_inputs, workload_inputs

from parity import compare, host_inputs, oracle_unit, run_gpu, say, slice_unit, to_gpu, whole_output_identities
from attn_workloads import dkdv_split_parts as dealt_parts

import oracle

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ small shapes, every element

FUZZ = [
    # B, S, Hq, Hkv, d, padded-length range or None
    (1, 1, 1, 1, 64, None),
    (1, 17, 2, 1, 64, None),
    (2, 63, 4, 2, 64, None),
    (1, 64, 3, 1, 64, None),
    (1, 65, 2, 2, 128, None),
    (3, 127, 8, 1, 64, None),
    (1, 128, 4, 4, 128, None),
    (2, 129, 6, 2, 64, None),
    (1, 200, 8, 2, 128, None),
    (3, 300, 4, 1, 64, (0, 300)),
    (3, 257, 2, 2, 128, (1, 257)),
    (2, 1000, 6, 3, 64, (500, 1000)),
    (1, 520, 16, 2, 128, None),
    (2, 384, 5, 5, 64, (383, 384)),
    # enough (block, head) pairs that the forward and dQ run their large-grid
    # blocks (256 and 128 rows) and dK/dV needs no split, with sequence
    # lengths that are no multiple of a block
    (2, 1000, 64, 16, 64, None),
    (2, 1000, 64, 16, 64, (500, 1000)),
    (1, 1000, 64, 16, 128, (700, 1000)),
    (1, 777, 128, 32, 64, None),
]


@pytest.mark.parametrize("case", FUZZ, ids=lambda c: "B{}_S{}_H{}-{}_d{}_{}".format(*c[:5], "pad" if c[5] else "dense"))
def test_fuzz_every_element(case):
    B, S, Hq, Hkv, d, rng = case
    seed = 1000 + B * 7 + S * 13 + Hq * 17 + d
    say(f"fuzz case B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} pad={rng} seed={seed}: attn_fwd/preprocess/attn_bwd")
    inp = make_inputs(B, S, Hq, Hkv, d, seed, padded=rng is not None, seqlen_range=rng)
    gpu = run_gpu(inp)
    q, k, v, do, sl = host_inputs(inp)
    ref = oracle.backward(q, k, v, do, inp.scale, sl)
    compare(gpu, ref, f"fuzz{case}")
    # the benchmark's launch order: attn_bwd_dq_delta (D formed in the dQ pass), then attn_bwd_dkdv
    say(f"fuzz case B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} pad={rng} seed={seed}: attn_bwd_dq_delta/attn_bwd_dkdv")
    compare(run_gpu(inp, bench_order=True), ref, f"fuzz{case} (dq_delta, dkdv)")


# The split dK/dV pass deals each (sequence, kv head)'s workgroups to its key
# blocks by their work; at S = 1281 the rounding gives the second block more
# parts than the first (4, 5, 4, 4, ...) and the second-to-last fewer than the
# last: the workspace must hold the largest count, the reduce pass each row's.
UNEVEN = [(2, 1281, 12, 4, 64, None, True), (2, 1281, 12, 4, 64, (640, 1281), True),
          (2, 1281, 12, 4, 128, None, True), (2, 1281, 12, 4, 64, None, False)]


@pytest.mark.parametrize("case", UNEVEN, ids=["causal", "causal_padded", "causal_d128", "bidirectional"])
def test_uneven_split_every_element(case):
    B, S, Hq, Hkv, d, rng, causal = case
    parts = dealt_parts(B, S, Hq, Hkv, causal)
    if causal:
        assert max(parts) > parts[0] and sum(parts) > len(parts), parts
    seed = 4200 + S + d + 7 * int(causal)
    say(f"uneven split B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} pad={rng} causal={causal} parts={parts} seed={seed}")
    inp = make_inputs(B, S, Hq, Hkv, d, seed, padded=rng is not None, seqlen_range=rng)
    gpu = run_gpu(inp, causal=causal)
    q, k, v, do, sl = host_inputs(inp)
    ref = oracle.backward(q, k, v, do, inp.scale, sl, causal=causal)
    compare(gpu, ref, f"uneven{case}")


def test_zero_length_sequences():
    say("edge: every sequence has valid length 0")
    B, S, Hq, Hkv, d = 2, 96, 4, 2, 64
    inp = make_inputs(B, S, Hq, Hkv, d, 7, padded=True, seqlen_range=(0, 0))
    gpu = run_gpu(inp)
    for key in ("O", "dQ", "dK", "dV", "D"):
        assert np.all(gpu[key] == 0.0), key
    assert np.all(np.isneginf(gpu["LSE"]))


# ------------------------------------------------------------------ the five workloads at full size

def _units(w, inp):
    """(b, kv head) units compared against the oracle for a workload (every
    unit also meets the identities of whole_output_identities)."""
    if w.name in ("tiny", "gqa124m"):
        return None  # every unit
    if w.name == "llama1b":
        # every (sequence, kv head) unit
        return [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    if w.name == "padded":
        L = inp.seqlens.tolist()
        return sorted({(int(np.argmin(L)), 0), (int(np.argmax(L)), 15)} | {(b, (5 * b + 3) % w.Hkv) for b in range(w.B)})
    if w.name == "longseq":
        # every one of its eight kv groups
        return [(0, g) for g in range(w.Hkv)]
    raise KeyError(w.name)


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.timeout(600)
def test_workload_parity(name):
    w = WORKLOADS[name]
    say(f"workload {name}: {w.describe()} seed={w.seed}")
    inp = workload_inputs(w)
    # the backward both ways: preprocess + attn_bwd, and the benchmark's
    # launch sequence (attn_bwd_dq_delta forming D, then attn_bwd_dkdv)
    runs = {"separate": run_gpu(inp)}
    say(f"workload {name}: separate preprocess done; benchmark launch order")
    runs["bench"] = run_gpu(inp, bench_order=True)
    say(f"workload {name}: GPU done, oracle running")
    units = _units(w, inp)
    if units is None:
        q, k, v, do, sl = host_inputs(inp)
        ref = oracle.backward(q, k, v, do, inp.scale, sl)
        for how, gpu in runs.items():
            compare(gpu, ref, f"{name} ({how})")
    else:
        dtype = np.float32 if name == "longseq" else np.float64
        G = w.Hq // w.Hkv
        for b, hkv in units:
            say(f"workload {name}: unit b={b} kv_head={hkv}")
            ref = oracle_unit(inp, b, hkv, dtype)
            for how, gpu in runs.items():
                compare(slice_unit(gpu, b, hkv, G), ref, f"{name}[b={b},g={hkv}] ({how})")
    # properties over the whole output
    for how, gpu in runs.items():
        for key in ("O", "dQ", "dK", "dV", "D"):
            assert np.all(np.isfinite(gpu[key])), (how, key)
        whole_output_identities(inp, gpu, label=f"{name} ({how})")
        if inp.seqlens is not None:
            for b, L in enumerate(inp.seqlens.tolist()):
                for key in ("O", "dQ", "dK", "dV"):
                    assert np.all(gpu[key][b, L:] == 0.0), (how, key, b)
                assert np.all(np.isneginf(gpu["LSE"][b, :, L:]))
                assert np.all(np.isfinite(gpu["LSE"][b, :, :L]))
        else:
            assert np.all(np.isfinite(gpu["LSE"]))
    # D from the dQ pass and from the preprocess: fp32 sums of the same d
    # products of bf16 values in two orders, so they differ by at most
    # 2 * d * 2^-24 * sum |dO * O| (the same forward ran twice: O is identical)
    np.testing.assert_array_equal(runs["bench"]["O"], runs["separate"]["O"])
    _, _, _, do, _ = host_inputs(inp)
    abs_sum = np.einsum("bshc->bhs", np.abs(do.astype(np.float64) * runs["bench"]["O"].astype(np.float64)))
    bound = 2 * w.d * 2.0 ** -24 * abs_sum + 1e-30
    assert np.all(np.abs(runs["bench"]["D"].astype(np.float64) - runs["separate"]["D"]) <= bound)


# ------------------------------------------------------------------ contracts

def test_nan_in_padding_does_not_leak():
    say("contract: NaN-filled padded positions")
    B, S, Hq, Hkv, d = 3, 333, 4, 2, 128
    inp = make_inputs(B, S, Hq, Hkv, d, 31, padded=True, seqlen_range=(100, 300))
    clean = run_gpu(inp)
    for name in ("q", "k", "v", "do"):
        x = getattr(inp, name)
        for b, L in enumerate(inp.seqlens.tolist()):
            x[b, L:] = float("nan")
    dirty = run_gpu(inp)
    for key in clean:
        np.testing.assert_array_equal(clean[key], dirty[key], err_msg=key)


def test_deterministic_and_stream_ordered():
    say("contract: bitwise repeatability and a non-default stream")
    inp = make_inputs(2, 700, 8, 2, 64, 41)
    first = run_gpu(inp)
    second = run_gpu(inp)
    for key in first:
        np.testing.assert_array_equal(first[key], second[key], err_msg=key)
    s = torch.cuda.Stream()
    t = to_gpu(inp)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        third = run_gpu(inp, t)
    for key in first:
        np.testing.assert_array_equal(first[key], third[key], err_msg=key)


def test_library_allocates_nothing():
    say("contract: no device allocation inside the library")
    inp = make_inputs(1, 512, 4, 2, 64, 5)
    t = to_gpu(inp)
    B, S, Hq, d = inp.q.shape
    o = torch.empty_like(t["q"])
    lse = torch.empty(B, Hq, S, device="cuda")
    delta = torch.empty(B, Hq, S, device="cuda")
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        attn.attn_fwd(t["q"], t["k"], t["v"], o, lse, inp.scale)
        attn.attn_bwd_preprocess(o, t["do"], delta)
        attn.attn_bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, dq, dk, dv, inp.scale)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free0 == free1


def test_preprocess_alone_tight():
    say("preprocess on independent random O/dO")
    inp = make_inputs(2, 300, 6, 6, 128, 77, padded=True, seqlen_range=(150, 300))
    t = to_gpu(inp)
    delta = torch.empty(2, 6, 300, device="cuda")
    attn.attn_bwd_preprocess(t["q"], t["do"], delta, t["seqlens"])   # q stands in for an O tensor
    torch.cuda.synchronize()
    q, _, _, do, sl = host_inputs(inp)
    ref = oracle.preprocess(q, do, sl)
    got = delta.cpu().numpy()
    # fp32 accumulation of 128 exact bf16 products: |err| <= 128 * 2^-24 * sum|q*do|
    bound = 128 * 2.0 ** -24 * np.einsum("bshc->bhs", np.abs(q * do)) + 1e-30
    assert np.all(np.abs(got - ref) <= bound)


def test_invalid_call_raises_without_launch():
    t = to_gpu(make_inputs(1, 64, 2, 1, 64, 3))
    o = torch.empty_like(t["q"])
    lse = torch.empty(1, 2, 64, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.attn_fwd(t["q"], t["k"], t["v"], o, lse, float("nan"))
    assert e.value.code == 1
