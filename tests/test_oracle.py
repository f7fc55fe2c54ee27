"""Pins for the CPU oracle (CPU only).

The oracle is pinned to things other than itself: hand-worked examples
(tests/golden), central differences of f = sum(O * dO) (the check the "Axis"
Rust/cuTile page names for its causal attention program, "Training building
blocks"), closed forms, invariants, and PyTorch's own CPU attention routine in
fp64 (the "Conformance with PyTorch" practice on that page).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def _value(tok: str) -> float:
    if tok == "nan":
        return float("nan")
    if tok in ("inf", "+inf"):
        return float("inf")
    if tok == "-inf":
        return float("-inf")
    ns = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln6": math.log(6.0), "__builtins__": {}}
    if not set(tok) <= set("0123456789./*+-ln"):
        raise ValueError(tok)
    return float(eval(tok, ns))  # restricted: digits, fractions and ln2/ln3/ln6 only


def load_golden(name):
    fields = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            fields[key] = val
    meta = dict(kv.split("=") for kv in fields.pop("meta").split())
    B, S, Hq, Hkv, d = (int(meta[k]) for k in ("B", "S", "Hq", "Hkv", "d"))
    scale = _value(meta["scale"])
    seqlens = None if meta["seqlens"] == "none" else [int(x) for x in meta["seqlens"].split(",")]
    causal = meta.get("causal", "1") == "1"
    shapes = {"Q": (B, S, Hq, d), "K": (B, S, Hkv, d), "V": (B, S, Hkv, d), "dO": (B, S, Hq, d),
              "O": (B, S, Hq, d), "dQ": (B, S, Hq, d), "dK": (B, S, Hkv, d), "dV": (B, S, Hkv, d),
              "LSE": (B, Hq, S), "D": (B, Hq, S)}
    arrays = {k: np.array([_value(t) for t in v.split()], dtype=np.float64).reshape(shapes[k])
              for k, v in fields.items()}
    return arrays, scale, seqlens, causal


def rand_inputs(B, S, Hq, Hkv, d, seed, q_scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, d)) * q_scale
    k = rng.standard_normal((B, S, Hkv, d))
    v = rng.standard_normal((B, S, Hkv, d))
    do = rng.standard_normal((B, S, Hq, d))
    return q, k, v, do


def objective(q, k, v, do, scale, seqlens=None, orc=oracle):
    O, _ = orc.forward(q, k, v, scale, seqlens)
    return float(np.sum(O * do))


# ----------------------------------------------------------------- golden

@pytest.mark.parametrize("name", ["hand_s3_d2.txt", "hand_gqa_padded.txt", "hand_noncausal_s3_d2.txt"])
def test_hand_worked_examples(name, orc=oracle):
    g, scale, seqlens, causal = load_golden(name)
    out = orc.backward(g["Q"], g["K"], g["V"], g["dO"], scale, seqlens, causal=causal)
    for key in ("O", "LSE", "D", "dQ", "dK", "dV"):
        exp, got = g[key], out[key]
        assert np.array_equal(np.isinf(exp), np.isinf(got)), key
        fin = np.isfinite(exp)
        assert np.all(np.isfinite(got[fin])), key
        np.testing.assert_allclose(got[fin], exp[fin], rtol=0, atol=1e-12, err_msg=key)
    O, LSE = orc.forward(g["Q"], g["K"], g["V"], scale, seqlens, causal=causal)
    np.testing.assert_array_equal(O, out["O"])
    np.testing.assert_array_equal(LSE, out["LSE"])
    D = orc.preprocess(out["O"], g["dO"], seqlens)
    np.testing.assert_allclose(D, g["D"], rtol=0, atol=1e-12)


# ----------------------------------------------------------------- central differences

@pytest.mark.parametrize("B,S,Hq,Hkv,d,seqlens", [
    (1, 6, 2, 1, 4, None),
    (2, 6, 4, 2, 3, [4, 6]),
    (1, 5, 3, 3, 2, [0]),
])
def test_central_differences(B, S, Hq, Hkv, d, seqlens, orc=oracle):
    scale = 0.37
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=11 + S + Hq)
    out = orc.backward(q, k, v, do, scale, seqlens)
    h = 1e-6
    for name, arr, grad in (("dQ", q, out["dQ"]), ("dK", k, out["dK"]), ("dV", v, out["dV"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = arr[idx]
            arr[idx] = keep + h
            fp = objective(q, k, v, do, scale, seqlens, orc)
            arr[idx] = keep - h
            fm = objective(q, k, v, do, scale, seqlens, orc)
            arr[idx] = keep
            num[idx] = (fp - fm) / (2 * h)
        err = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-30)
        if np.linalg.norm(grad) == 0:
            assert np.max(np.abs(num)) < 1e-8, name
        else:
            assert err < 1e-6, (name, err)


# ----------------------------------------------------------------- softmax structure

@pytest.mark.parametrize("dtype,tol", [(np.float64, 1e-12), (np.float32, 1e-5)])
def test_rows_sum_to_one_and_causal_zeros(dtype, tol):
    q, k, _, _ = rand_inputs(1, 50, 1, 1, 16, seed=3)
    P, lse = oracle.probabilities(q[0, :, 0], k[0, :, 0], 0.25, dtype)
    assert P.dtype == dtype
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=tol, rtol=0)
    assert np.all(P[np.triu_indices(50, 1)] == 0.0)
    assert np.all(P[np.tril_indices(50)] > 0.0)
    assert np.all(np.isfinite(lse))


def test_padded_rows_and_columns_are_zero():
    B, S, Hq, Hkv, d = 2, 9, 2, 1, 4
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=5)
    seqlens = [5, 9]
    out = oracle.backward(q, k, v, do, 0.5, seqlens)
    for key in ("O", "dQ"):
        assert np.all(out[key][0, 5:] == 0.0)
    for key in ("dK", "dV"):
        assert np.all(out[key][0, 5:] == 0.0)
    assert np.all(np.isneginf(out["LSE"][0, :, 5:]))
    assert np.all(out["D"][0, :, 5:] == 0.0)
    assert np.all(np.isfinite(out["LSE"][1]))


def test_row0_closed_form():
    q, k, v, _ = rand_inputs(2, 7, 4, 2, 8, seed=9)
    scale = 0.3
    O, LSE = oracle.forward(q, k, v, scale)
    for b in range(2):
        for h in range(4):
            g = h // 2
            np.testing.assert_array_equal(O[b, 0, h], v[b, 0, g])
            s00 = scale * sum(q[b, 0, h, c] * k[b, 0, g, c] for c in range(8))
            assert abs(LSE[b, h, 0] - s00) < 1e-12


def test_uniform_scores_prefix_mean():
    # Q = 0 makes every score 0: row i averages v_0..v_i (the prefix-mean task of
    # the attention program on the "Axis" Rust/cuTile page).
    B, S, Hq, Hkv, d = 1, 12, 2, 1, 5
    _, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=21)
    q = np.zeros((B, S, Hq, d))
    out = oracle.backward(q, k, v, do, 0.125)
    for h in range(Hq):
        for i in range(S):
            mean = sum(v[0, j, 0] for j in range(i + 1)) / (i + 1)
            np.testing.assert_allclose(out["O"][0, i, h], mean, atol=1e-13, rtol=0)
            assert abs(out["LSE"][0, h, i] - math.log(i + 1)) < 1e-13
    for j in range(S):
        expect = sum(do[0, i, h] / (i + 1) for i in range(j, S) for h in range(Hq))
        np.testing.assert_allclose(out["dV"][0, j, 0], expect, atol=1e-12, rtol=0)
    assert np.max(np.abs(out["dK"])) == 0.0


def test_constant_values():
    B, S, Hq, Hkv, d = 1, 10, 2, 2, 4
    q, k, _, do = rand_inputs(B, S, Hq, Hkv, d, seed=4)
    c = np.array([0.5, -1.25, 2.0, 3.0])
    v = np.broadcast_to(c, (B, S, Hkv, d)).copy()
    out = oracle.backward(q, k, v, do, 0.4)
    np.testing.assert_allclose(out["O"], np.broadcast_to(c, out["O"].shape), atol=1e-13, rtol=0)
    assert np.max(np.abs(out["dQ"])) < 1e-12
    assert np.max(np.abs(out["dK"])) < 1e-12


# ----------------------------------------------------------------- structural invariants

def test_gqa_equals_explicit_repeat(orc=oracle):
    B, S, Hq, Hkv, d = 2, 11, 6, 2, 4
    G = Hq // Hkv
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=8)
    seqlens = [11, 7]
    grouped = orc.backward(q, k, v, do, 0.3, seqlens)
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)   # kv head g serves q heads gG..gG+G-1
    full = orc.backward(q, kr, vr, do, 0.3, seqlens)
    for key in ("O", "LSE", "D", "dQ"):
        np.testing.assert_allclose(grouped[key], full[key], atol=1e-13, rtol=0)
    for key in ("dK", "dV"):
        summed = full[key].reshape(B, S, Hkv, G, d).sum(axis=3)
        np.testing.assert_allclose(grouped[key], summed, atol=1e-12, rtol=0)


def test_padding_equals_prefix_slice_and_ignores_nan(orc=oracle):
    B, S, Hq, Hkv, d = 3, 13, 2, 1, 4
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=12)
    seqlens = [13, 6, 1]
    for arr in (q, k, v, do):
        for b, L in enumerate(seqlens):
            arr[b, L:] = np.nan
    out = orc.backward(q, k, v, do, 0.5, seqlens)
    for key in ("O", "LSE", "D", "dQ", "dK", "dV"):
        assert not np.any(np.isnan(out[key])), key
    for b, L in enumerate(seqlens):
        ref = orc.backward(q[b:b + 1, :L], k[b:b + 1, :L], v[b:b + 1, :L], do[b:b + 1, :L], 0.5)
        for key in ("O", "dQ", "dK", "dV"):
            np.testing.assert_array_equal(out[key][b, :L], ref[key][0])
            assert np.all(out[key][b, L:] == 0)
        for key in ("LSE", "D"):
            np.testing.assert_array_equal(out[key][b, :, :L], ref[key][0])


def test_causal_prefix_invariance():
    B, S, Hq, Hkv, d = 1, 16, 2, 1, 4
    q, k, v, _ = rand_inputs(B, S, Hq, Hkv, d, seed=13)
    O, LSE = oracle.forward(q, k, v, 0.5)
    i = 6
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    rng = np.random.default_rng(0)
    for arr in (q2, k2, v2):
        arr[:, i + 1:] += rng.standard_normal(arr[:, i + 1:].shape) * 10
    O2, LSE2 = oracle.forward(q2, k2, v2, 0.5)
    np.testing.assert_array_equal(O[:, :i + 1], O2[:, :i + 1])
    np.testing.assert_array_equal(LSE[:, :, :i + 1], LSE2[:, :, :i + 1])
    assert not np.allclose(O[:, i + 1:], O2[:, i + 1:])


def test_large_scores_are_stable_and_one_hot():
    B, S, Hq, Hkv, d = 1, 40, 1, 1, 16
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=14, q_scale=100.0)
    out = oracle.backward(q, k, v, do, 0.25)
    for key in ("O", "LSE", "D", "dQ", "dK", "dV"):
        assert np.all(np.isfinite(out[key])), key
    P, _ = oracle.probabilities(q[0, :, 0], k[0, :, 0], 0.25)
    s = 0.25 * (q[0, :, 0] @ k[0, :, 0].T)
    for i in range(S):
        row = s[i, :i + 1]
        top = np.argmax(row)
        gap = np.sort(row)[-1] - np.sort(row)[-2] if i > 0 else np.inf
        if gap > 40:   # exp(-40) ~ 4e-18: the row is one-hot in fp64
            assert P[i, top] == pytest.approx(1.0, abs=1e-15)
            np.testing.assert_allclose(out["O"][0, i, 0], v[0, top, 0], atol=1e-12)


# ----------------------------------------------------------------- library routine

def _torch_reference(q, k, v, do, scale):
    """PyTorch CPU fp64 attention (library routine) + autograd, GQA by repeat_interleave."""
    G = q.shape[2] // k.shape[2]
    tq = torch.tensor(q, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.tensor(k, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.tensor(v, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), is_causal=True, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64).permute(0, 2, 1, 3))
    tr = lambda t: t.detach().permute(0, 2, 1, 3).numpy()  # noqa: E731
    return tr(o), tr(tq.grad), tr(tk.grad), tr(tv.grad)


@pytest.mark.parametrize("B,S,Hq,Hkv,d", [(1, 33, 2, 2, 8), (2, 64, 6, 2, 16), (1, 130, 4, 1, 32)])
def test_matches_torch_sdpa_fp64(B, S, Hq, Hkv, d, orc=oracle):
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=B * 100 + S)
    scale = 1.0 / math.sqrt(d)
    out = orc.backward(q, k, v, do, scale)
    o, dq, dk, dv = _torch_reference(q, k, v, do, scale)
    for key, ref in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        np.testing.assert_allclose(out[key], ref, atol=1e-10, rtol=0, err_msg=key)


def test_lse_matches_torch_logsumexp_routine(orc=oracle):
    # torch.logsumexp over the causal row (a library routine for the normaliser)
    B, S, Hq, Hkv, d = 1, 40, 2, 1, 8
    q, k, v, _ = rand_inputs(B, S, Hq, Hkv, d, seed=77)
    _, LSE = orc.forward(q, k, v, 0.2)
    tq = torch.tensor(q[0], dtype=torch.float64)
    tk = torch.tensor(k[0], dtype=torch.float64)
    for h in range(Hq):
        s = torch.einsum("ic,jc->ij", tq[:, h], tk[:, 0]) * 0.2
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(LSE[0, h], torch.logsumexp(s, dim=1).numpy(), atol=1e-12, rtol=0)


# ----------------------------------------------------------------- fp32 vs fp64

def test_fp32_oracle_close_to_fp64():
    from attn_workloads import make_inputs
    inp = make_inputs(1, 128, 2, 2, 64, seed=20260001)
    q, k, v, do = (t.float().numpy() for t in (inp.q, inp.k, inp.v, inp.do))
    r64 = oracle.backward(q, k, v, do, inp.scale, dtype=np.float64)
    r32 = oracle.backward(q, k, v, do, inp.scale, dtype=np.float32)
    for key in ("O", "dQ", "dK", "dV", "LSE", "D"):
        assert r32[key].dtype == np.float32
        assert np.max(np.abs(r32[key] - r64[key])) < 1e-4, key
