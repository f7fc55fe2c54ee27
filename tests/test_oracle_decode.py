"""Pins for the oracle's decode attention (CPU only).

oracle.decode (new queries against a key/value cache) is pinned to things
other than itself: the pinned causal forward of the full sequence (its last Sq
rows are the decode outputs), PyTorch's CPU attention routine in fp64 with an
explicit mask, closed forms (Q = 0 gives the mean of the visible values), the
hand-worked numbers of tests/golden/hand_s3_d2.txt, and the empty cases.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from test_oracle import load_golden


def _case(B, Sq, Smax, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, Hq, d))
    k = rng.standard_normal((B, Smax, Hkv, d))
    v = rng.standard_normal((B, Smax, Hkv, d))
    return q, k, v


@pytest.mark.parametrize("B,Sq,Smax,Hq,Hkv,d,lens", [
    (2, 1, 40, 4, 2, 8, [40, 17]),
    (3, 4, 33, 6, 2, 16, [33, 4, 9]),
    (1, 7, 20, 2, 1, 4, [20]),
])
def test_equals_last_rows_of_causal_forward(B, Sq, Smax, Hq, Hkv, d, lens, orc=oracle):
    q, k, v = _case(B, Sq, Smax, Hq, Hkv, d, seed=B * 100 + Sq)
    O, LSE = orc.decode(q, k, v, 0.3, lens)
    rng = np.random.default_rng(1)
    for b, L in enumerate(lens):
        # the full sequence: anything at positions < L - Sq, the new queries after
        qf = rng.standard_normal((1, Smax, Hq, d))
        qf[0, L - Sq:L] = q[b]
        Of, LSEf = oracle.forward(qf, k[b:b + 1], v[b:b + 1], 0.3, [L])
        np.testing.assert_allclose(O[b], Of[0, L - Sq:L], atol=1e-12, rtol=0)
        np.testing.assert_allclose(LSE[b], LSEf[0, :, L - Sq:L], atol=1e-12, rtol=0)


def test_matches_torch_sdpa_with_mask(orc=oracle):
    B, Sq, Smax, Hq, Hkv, d = 2, 3, 50, 8, 2, 16
    lens = [50, 23]
    q, k, v = _case(B, Sq, Smax, Hq, Hkv, d, seed=5)
    O, LSE = orc.decode(q, k, v, 0.25, lens)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        tq = torch.tensor(q[b]).permute(1, 0, 2)                       # [Hq, Sq, d]
        tk = torch.tensor(k[b, :L]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        tv = torch.tensor(v[b, :L]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        pos = torch.arange(Sq) + (L - Sq)
        mask = torch.arange(L)[None, :] <= pos[:, None]                # [Sq, L]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.25)
        np.testing.assert_allclose(O[b], ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
        s = (tq @ tk.transpose(1, 2)) * 0.25
        lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
        np.testing.assert_allclose(LSE[b], lse.numpy(), atol=1e-12, rtol=0)


def test_zero_query_is_the_mean_of_the_visible_values(orc=oracle):
    B, Sq, Smax, Hq, Hkv, d = 1, 2, 30, 4, 1, 6
    _, k, v = _case(B, Sq, Smax, Hq, Hkv, d, seed=8)
    q = np.zeros((B, Sq, Hq, d))
    L = 25
    O, LSE = orc.decode(q, k, v, 0.5, [L])
    for t in range(Sq):
        p = L - Sq + t
        for h in range(Hq):
            np.testing.assert_allclose(O[0, t, h], v[0, :p + 1, 0].mean(axis=0), atol=1e-13, rtol=0)
            assert abs(LSE[0, h, t] - math.log(p + 1)) < 1e-13


def test_queries_without_keys(orc=oracle):
    B, Sq, Smax, Hq, Hkv, d = 3, 4, 10, 2, 2, 4
    q, k, v = _case(B, Sq, Smax, Hq, Hkv, d, seed=9)
    O, LSE = orc.decode(q, k, v, 0.5, [0, 2, 10])
    assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))
    # L = 2 < Sq = 4: queries 0 and 1 sit at positions -2, -1 and see nothing
    assert np.all(O[1, :2] == 0) and np.all(np.isneginf(LSE[1, :, :2]))
    assert np.all(np.isfinite(LSE[1, :, 2:])) and np.all(np.isfinite(LSE[2]))


def test_hand_worked_values(orc=oracle):
    # rows 1 and 2 of the hand-worked causal example are two new queries
    # against its three cached positions
    g, scale, _, _ = load_golden("hand_s3_d2.txt")
    O, LSE = orc.decode(g["Q"][:, 1:], g["K"], g["V"], scale, [3])
    np.testing.assert_allclose(O, g["O"][:, 1:], atol=1e-12, rtol=0)
    np.testing.assert_allclose(LSE, g["LSE"][:, :, 1:], atol=1e-12, rtol=0)
    # one query against the first two positions only (row 1 of the example)
    O1, LSE1 = orc.decode(g["Q"][:, 1:2], g["K"], g["V"], scale, [2])
    np.testing.assert_allclose(O1[0, 0, 0], [2.0, 4.0], atol=1e-12, rtol=0)
    assert abs(LSE1[0, 0, 0] - math.log(3.0)) < 1e-12


def test_gqa_equals_explicit_repeat(orc=oracle):
    B, Sq, Smax, Hq, Hkv, d = 2, 2, 24, 6, 2, 8
    q, k, v = _case(B, Sq, Smax, Hq, Hkv, d, seed=12)
    O, LSE = orc.decode(q, k, v, 0.4, [24, 11])
    O2, LSE2 = orc.decode(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 0.4, [24, 11])
    np.testing.assert_allclose(O, O2, atol=0, rtol=0)
    np.testing.assert_allclose(LSE, LSE2, atol=0, rtol=0)
