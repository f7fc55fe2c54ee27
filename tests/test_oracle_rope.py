"""Pins for the oracle's rotary position embedding (CPU only).

oracle/rope.py follows "AxiomLM" (PyPI page), "8. Standalone Modern
Architectural Modules" (frequencies precomputed for a head size, applied to q
and k before attention) under the reading stated in its header (interleaved
pairs, theta_i = 10000^(-2i/d), angle = position * theta_i). These tests pin it
to things other than itself: the plane rotation by the position itself when
d = 2, exact powers of ten for d = 8, complex multiplication by exp(i a) (the
form the pages' freqs_cis table implies), orthogonality, the relative-position
property that motivates the method, central differences through rope and
attention, and PyTorch's complex routines with SDPA and autograd in fp64.
"""
import math

import numpy as np
import pytest
import torch

from oracle import rope as oracle_rope
from test_oracle import rand_inputs


def test_position_zero_is_identity(rp=oracle_rope):
    x = np.random.default_rng(0).standard_normal((2, 1, 3, 16))
    np.testing.assert_array_equal(rp.rotate(x), x)


def test_head_size_two_is_plane_rotation_by_the_position(rp=oracle_rope):
    # d = 2: one pair, theta_0 = 1, so token p is rotated by p radians
    S = 7
    x = np.zeros((1, S, 1, 2))
    x[..., 0] = 1.0
    y = rp.rotate(x)
    for p in range(S):
        np.testing.assert_allclose(y[0, p, 0], [math.cos(p), math.sin(p)], atol=1e-15, rtol=0)
    x2 = np.zeros((1, S, 1, 2))
    x2[..., 1] = 1.0
    y2 = rp.rotate(x2)
    for p in range(S):
        np.testing.assert_allclose(y2[0, p, 0], [-math.sin(p), math.cos(p)], atol=1e-15, rtol=0)


def test_frequencies_are_powers_of_ten_for_head_size_eight(rp=oracle_rope):
    # 10000^(-2i/8) = 10^(-i)
    np.testing.assert_allclose(rp.frequencies(8), [1.0, 0.1, 0.01, 0.001], rtol=1e-15, atol=0)
    x = np.random.default_rng(1).standard_normal((1, 40, 2, 8))
    y = rp.rotate(x)
    for p in (0, 1, 13, 39):
        for i in range(4):
            a = p * 10.0 ** (-i)
            c, s = math.cos(a), math.sin(a)
            x0, x1 = x[0, p, :, 2 * i], x[0, p, :, 2 * i + 1]
            np.testing.assert_allclose(y[0, p, :, 2 * i], x0 * c - x1 * s, atol=1e-14, rtol=0)
            np.testing.assert_allclose(y[0, p, :, 2 * i + 1], x0 * s + x1 * c, atol=1e-14, rtol=0)


def test_matches_complex_multiplication(rp=oracle_rope):
    B, S, H, d = 2, 300, 3, 64
    x = np.random.default_rng(2).standard_normal((B, S, H, d))
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = 10000.0 ** (-np.arange(0, d, 2) / d)
    zr = z * np.exp(1j * np.arange(S)[:, None] * theta[None, :])[None, :, None, :]
    y = rp.rotate(x)
    np.testing.assert_allclose(y[..., 0::2], zr.real, atol=1e-12, rtol=0)
    np.testing.assert_allclose(y[..., 1::2], zr.imag, atol=1e-12, rtol=0)


def test_orthogonal_and_inverse(rp=oracle_rope):
    x = np.random.default_rng(3).standard_normal((2, 100, 4, 32))
    y = rp.rotate(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(rp.rotate(y, inverse=True), x, atol=1e-13, rtol=0)
    # the adjoint: <R x, w> = <x, R^T w>
    w = np.random.default_rng(4).standard_normal(x.shape)
    np.testing.assert_allclose(np.sum(y * w), np.sum(x * rp.rotate(w, inverse=True)), rtol=1e-12)


def test_scores_depend_only_on_relative_position(rp=oracle_rope):
    rng = np.random.default_rng(5)
    S, d = 24, 16
    q = rng.standard_normal((1, S, 1, d))
    k = rng.standard_normal((1, S, 1, d))
    pos = np.arange(S)

    def scores(shift):
        qr = rp.rotate(q, positions=pos + shift)[0, :, 0]
        kr = rp.rotate(k, positions=pos + shift)[0, :, 0]
        return qr @ kr.T

    base = scores(0)
    for shift in (1, 17, 1000):
        np.testing.assert_allclose(scores(shift), base, atol=1e-10, rtol=0)
    # and they do depend on the positions: unrotated scores differ
    assert np.max(np.abs(base - q[0, :, 0] @ k[0, :, 0].T)) > 1e-2


@pytest.mark.parametrize("B,S,Hq,Hkv,d,seqlens,causal", [
    (1, 5, 2, 1, 4, None, True),
    (2, 5, 2, 2, 6, [3, 5], True),
    (1, 4, 2, 1, 4, None, False),
])
def test_central_differences_through_rope(B, S, Hq, Hkv, d, seqlens, causal, rp=oracle_rope):
    scale = 0.41
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=31 + S + d)
    out = rp.backward(q, k, v, do, scale, seqlens, causal=causal)

    def f():
        O, _ = rp.forward(q, k, v, scale, seqlens, causal=causal)
        return float(np.sum(O * do))

    h = 1e-6
    for name, arr in (("dQ", q), ("dK", k), ("dV", v)):
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
        err = np.linalg.norm(num - out[name]) / max(np.linalg.norm(out[name]), 1e-30)
        assert err < 1e-6, (name, err)


def _torch_rope_attention(q, k, v, do, scale, causal=True):
    """fp64 PyTorch: rope through torch.polar and complex products, SDPA, autograd."""
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    inv = 1.0 / (10000.0 ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    ang = torch.outer(torch.arange(S, dtype=torch.float64), inv)
    cis = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

    def rot(x):
        xc = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
        return torch.view_as_real(xc * cis).reshape(x.shape)

    qr = rot(tq).permute(0, 2, 1, 3)
    kr = rot(tk).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vr = tv.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qr, kr, vr, is_causal=causal, scale=scale)
    o = o.permute(0, 2, 1, 3)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_complex_rope_and_sdpa(causal, rp=oracle_rope):
    B, S, Hq, Hkv, d = 2, 48, 4, 2, 16
    q, k, v, do = rand_inputs(B, S, Hq, Hkv, d, seed=77)
    scale = 1.0 / math.sqrt(d)
    out = rp.backward(q, k, v, do, scale, causal=causal)
    o, dq, dk, dv = _torch_rope_attention(q, k, v, do, scale, causal)
    for key, ref in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        np.testing.assert_allclose(out[key], ref, atol=1e-10, rtol=0, err_msg=key)


def test_bf16_rounding_matches_torch_conversion(rp=oracle_rope):
    # values exactly representable in fp32, so torch's fp32 -> bf16 conversion
    # (round to nearest, ties to even) rounds the same number once
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.0 * (1 + 2.0 ** -8)], np.float32)
    x = np.concatenate([x, ties])
    want = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = rp.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(rp.round_bf16(np.array([1.0 + 2.0 ** -8])), [1.0])       # tie to even
    np.testing.assert_array_equal(rp.round_bf16(np.array([1.0 + 3 * 2.0 ** -8])), [1.0 + 2.0 ** -6])


def test_bf16_storage_rounds_only_the_rotated_inputs(rp=oracle_rope):
    q, k, v, do = rand_inputs(1, 20, 2, 1, 8, seed=12)
    exact = rp.backward(q, k, v, do, 0.3)
    stored = rp.backward(q, k, v, do, 0.3, bf16_storage=True)
    np.testing.assert_array_equal(stored["Qrot"], rp.round_bf16(exact["Qrot"]))
    np.testing.assert_array_equal(stored["Krot"], rp.round_bf16(exact["Krot"]))
    assert 0 < np.max(np.abs(stored["O"] - exact["O"])) < 1e-2


@pytest.mark.parametrize("B,Sq,S,Hq,Hkv,d,lens", [
    (2, 1, 40, 4, 2, 8, [40, 17]),
    (3, 4, 33, 6, 2, 16, [33, 4, 9]),
    (1, 3, 70, 2, 1, 32, [70]),
])
def test_decode_equals_last_rows_of_rope_forward(B, Sq, S, Hq, Hkv, d, lens, rp=oracle_rope):
    # a cache holding keys rotated at their positions, queried by the last Sq
    # queries of each sequence, gives the last Sq rows of the causal rope
    # forward over the whole valid prefix
    q, k, v, _ = rand_inputs(B, S, Hq, Hkv, d, seed=S + Sq)
    scale = 1.0 / math.sqrt(d)
    cache = rp.rotate(k)
    qn = np.zeros((B, Sq, Hq, d))
    for b, L in enumerate(lens):
        for t in range(Sq):
            if L - Sq + t >= 0:
                qn[b, t] = q[b, L - Sq + t]
    O, LSE = rp.decode(qn, cache, v, scale, lens)
    for b, L in enumerate(lens):
        Of, LSEf = rp.forward(q[b:b + 1, :L], k[b:b + 1, :L], v[b:b + 1, :L], scale)
        for t in range(Sq):
            p = L - Sq + t
            if p < 0:
                assert np.all(O[b, t] == 0) and np.all(np.isneginf(LSE[b, :, t]))
                continue
            np.testing.assert_allclose(O[b, t], Of[0, p], atol=1e-12, rtol=0)
            np.testing.assert_allclose(LSE[b, :, t], LSEf[0, :, p], atol=1e-12, rtol=0)


def test_decode_at_position_zero_is_plain_decode(rp=oracle_rope):
    import oracle
    q, k, v, _ = rand_inputs(3, 1, 4, 2, 16, seed=5)
    kc = np.random.default_rng(6).standard_normal((3, 9, 2, 16))
    vc = np.random.default_rng(7).standard_normal((3, 9, 2, 16))
    O, LSE = rp.decode(q, kc, vc, 0.25, [1, 1, 1])
    O2, LSE2 = oracle.decode(q, kc, vc, 0.25, [1, 1, 1])
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, LSE2)
