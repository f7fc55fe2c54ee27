"""Pins for the oracle's bidirectional (non-causal) path (CPU only).

The "Axis" Rust/cuTile page, "Sudoku as an acceptance test", runs a transformer
with bidirectional multi-head attention: the same softmax attention with no
causal restriction. These tests pin the oracle's ``causal=False`` path to
things other than itself: PyTorch's CPU attention routine in fp64 (with a key
padding mask), central differences, closed forms, permutation equivariance
(which only the bidirectional form has) and agreement with the causal form on
the one row where the two coincide. The hand-worked fixture
tests/golden/hand_noncausal_s3_d2.txt is checked by test_oracle.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from test_oracle import rand_inputs


def _torch_noncausal(q, k, v, do, scale, seqlens):
    """PyTorch CPU fp64 attention with a key padding mask, + autograd; GQA by
    repeat_interleave. Rows at or past L are not compared by the callers."""
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    tq = torch.tensor(q, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.tensor(k, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.tensor(v, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    lens = [S] * B if seqlens is None else list(seqlens)
    keep = torch.zeros(B, 1, S, S, dtype=torch.bool)
    rows = torch.zeros(B, 1, S, 1, dtype=torch.float64)
    for b, L in enumerate(lens):
        keep[b, 0, :, :L] = True
        rows[b, 0, :L] = 1.0
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), attn_mask=keep, scale=scale)
    o = o * rows  # padded query rows are zero by definition
    o.backward(torch.tensor(do, dtype=torch.float64).permute(0, 2, 1, 3) * rows)
    tr = lambda t: t.detach().permute(0, 2, 1, 3).numpy()  # noqa: E731
    return tr(o), tr(tq.grad), tr(tk.grad), tr(tv.grad)


@pytest.mark.parametrize("B,S,Hq,Hkv,d,seqlens", [
    (1, 33, 2, 2, 8, None), (2, 64, 6, 2, 16, [64, 41]), (1, 70, 4, 1, 32, [57]),
])
def test_matches_torch_sdpa_fp64(B, S, Hq, Hkv, d, seqlens, orc=oracle):
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=B * 1000 + S)
    scale = 1.0 / math.sqrt(d)
    out = orc.backward(q, k, v, do, scale, seqlens, causal=False)
    o, dq, dk, dv = _torch_noncausal(q, k, v, do, scale, seqlens)
    lens = [S] * B if seqlens is None else seqlens
    for b, L in enumerate(lens):
        for key, ref in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
            np.testing.assert_allclose(out[key][b, :L], ref[b, :L], atol=1e-10, rtol=0, err_msg=key)
        for key in ("O", "dQ", "dK", "dV"):
            assert np.all(out[key][b, L:] == 0), key
        assert np.all(np.isneginf(out["LSE"][b, :, L:]))


@pytest.mark.parametrize("B,S,Hq,Hkv,d,seqlens", [(1, 5, 2, 1, 3, None), (2, 5, 2, 2, 2, [3, 5])])
def test_central_differences(B, S, Hq, Hkv, d, seqlens, orc=oracle):
    scale = 0.41
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=7 + S + Hq)
    out = orc.backward(q, k, v, do, scale, seqlens, causal=False)

    def f():
        O, _ = orc.forward(q, k, v, scale, seqlens, causal=False)
        return float(np.sum(O * do))

    h = 1e-6
    for name, arr, grad in (("dQ", q, out["dQ"]), ("dK", k, out["dK"]), ("dV", v, out["dV"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = arr[idx]
            arr[idx] = keep + h
            fp = f()
            arr[idx] = keep - h
            fm = f()
            arr[idx] = keep
            num[idx] = (fp - fm) / (2 * h)
        err = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-30)
        assert err < 1e-6, (name, err)


def test_uniform_scores_full_mean(orc=oracle):
    # Q = 0: every score is 0, so every valid row averages all L values, LSE = ln L
    B, S, Hq, Hkv, d, L = 1, 12, 2, 1, 5, 9
    _, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=31)
    q = np.zeros((B, S, Hq, d))
    out = orc.backward(q, k, v, do, 0.125, [L], causal=False)
    mean = v[0, :L, 0].mean(axis=0)
    for h in range(Hq):
        np.testing.assert_allclose(out["O"][0, :L, h], np.broadcast_to(mean, (L, d)), atol=1e-13, rtol=0)
        np.testing.assert_allclose(out["LSE"][0, h, :L], math.log(L), atol=1e-13, rtol=0)
    # dV_j = sum over heads and valid rows of dO_i / L, the same for every valid key
    expect = do[0, :L].sum(axis=(0, 1)) / L
    np.testing.assert_allclose(out["dV"][0, :L, 0], np.broadcast_to(expect, (L, d)), atol=1e-12, rtol=0)
    assert np.max(np.abs(out["dK"])) == 0.0


def test_permutation_equivariance(orc=oracle):
    # bidirectional attention: permuting the keys and values together changes
    # nothing; permuting the queries permutes O, LSE, D and dQ the same way
    B, S, Hq, Hkv, d = 1, 10, 2, 1, 4
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=5)
    base = orc.backward(q, k, v, do, 0.3, causal=False)
    perm = np.random.default_rng(9).permutation(S)
    kv = orc.backward(q, k[:, perm], v[:, perm], do, 0.3, causal=False)
    for key in ("O", "LSE", "D", "dQ"):
        np.testing.assert_allclose(kv[key], base[key], atol=1e-12, rtol=0, err_msg=key)
    np.testing.assert_allclose(kv["dK"], base["dK"][:, perm], atol=1e-12, rtol=0)
    np.testing.assert_allclose(kv["dV"], base["dV"][:, perm], atol=1e-12, rtol=0)
    qp = orc.backward(q[:, perm], k, v, do[:, perm], 0.3, causal=False)
    for key in ("O", "dQ"):
        np.testing.assert_allclose(qp[key], base[key][:, perm], atol=1e-12, rtol=0, err_msg=key)
    np.testing.assert_allclose(qp["LSE"], base["LSE"][:, :, perm], atol=1e-12, rtol=0)
    np.testing.assert_allclose(qp["dK"], base["dK"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(qp["dV"], base["dV"], atol=1e-12, rtol=0)


def test_last_row_agrees_with_causal(orc=oracle):
    # row L-1 sees every key of the prefix in both forms
    B, S, Hq, Hkv, d = 2, 16, 2, 1, 8
    q, k, v, _ = rand_inputs(B, S, Hq, Hkv, d, seed=13)
    seqlens = [16, 11]
    Oc, Lc = orc.forward(q, k, v, 0.25, seqlens)
    On, Ln = orc.forward(q, k, v, 0.25, seqlens, causal=False)
    for b, L in enumerate(seqlens):
        np.testing.assert_allclose(On[b, L - 1], Oc[b, L - 1], atol=1e-13, rtol=0)
        np.testing.assert_allclose(Ln[b, :, L - 1], Lc[b, :, L - 1], atol=1e-13, rtol=0)
    # and differs elsewhere (row 0 of the causal form is v_0)
    assert np.max(np.abs(On[0, 0] - Oc[0, 0])) > 1e-3


def test_rows_are_full_distributions(orc=oracle):
    q, k, _, _ = rand_inputs(1, 40, 1, 1, 16, seed=4)
    P, lse = orc.probabilities(q[0, :, 0], k[0, :, 0], 0.25, causal=False)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert np.all(P > 0)  # no structural zeros above the diagonal
    np.testing.assert_allclose(
        lse, torch.logsumexp(torch.tensor(q[0, :, 0] @ k[0, :, 0].T * 0.25), dim=1).numpy(), atol=1e-12, rtol=0)
