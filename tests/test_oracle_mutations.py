"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a private copy of the oracle's source (a
dropped term, a wrong sign, index or scale, a transposed operand, a wrong
normaliser) and checks that at least one pin from test_oracle.py fails on the
mutant. The real oracle is never modified.
"""
import os
import types

import pytest

import test_oracle as pins
import test_oracle_noncausal as ncpins
import test_oracle_decode as dpins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTATIONS = {
    "drop_D_term": ("dS = P * (dP - Dh[:, None])", "dS = P * dP"),
    "flip_dS_sign": ("dS = P * (dP - Dh[:, None])", "dS = P * (Dh[:, None] - dP)"),
    "gqa_modulo_mapping": ("g = h // G", "g = h % Hkv"),
    "dK_without_scale": ("dK[b, :L, g, :] += sc * (dS.T @ qh)", "dK[b, :L, g, :] += (dS.T @ qh)"),
    "dQ_transposed_dS": ("dQ[b, :L, h, :] = sc * (dS @ kh)", "dQ[b, :L, h, :] = sc * (dS.T @ kh)"),
    "dV_untransposed_P": ("dV[b, :L, g, :] += P.T @ doh", "dV[b, :L, g, :] += P @ doh"),
    "lse_base2": ("lse = m + np.log(denom)", "lse = m + np.log2(denom)"),
    "mask_off_by_one": ("np.tril(np.ones((L, L), dtype=bool))", "np.tril(np.ones((L, L), dtype=bool), 1)"),
    "scores_unscaled": ("s = (qh @ kh.T) * dtype(scale)", "s = (qh @ kh.T)"),
    "D_without_O": ("Dh = np.sum(doh * oh, axis=1)", "Dh = np.sum(doh, axis=1)"),
    "padding_ignored": ("L = lens[b]\n        for h in range(Hq):\n            g = h // G\n            qh",
                        "L = S\n        for h in range(Hq):\n            g = h // G\n            qh"),
    # the bidirectional path
    "noncausal_still_causal": ("if causal else np.ones((L, L), dtype=bool)",
                               "if True else np.ones((L, L), dtype=bool)"),
    "noncausal_upper_triangle": ("if causal else np.ones((L, L), dtype=bool)",
                                 "if causal else np.triu(np.ones((L, L), dtype=bool))"),
    "backward_ignores_causal_flag": ("P, lse = probabilities(qh, kh, scale, dtype, causal)",
                                     "P, lse = probabilities(qh, kh, scale, dtype)"),
    # decode
    "decode_position_off_by_one": ("p = L - Sq + t\n", "p = L - Sq + t - 1\n"),
    "decode_new_queries_see_everything": ("p = L - Sq + t\n", "p = L - 1\n"),
    "decode_gqa_modulo": ("            g = h // G\n            for t in range(Sq):", "            g = h % Hkv\n            for t in range(Sq):"),
    "decode_unscaled": ("s_ = (kk @ np.asarray(q[b, t, h, :], dtype=dtype)) * sc", "s_ = (kk @ np.asarray(q[b, t, h, :], dtype=dtype))"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert old in src, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins(orc):
    yield lambda: pins.test_hand_worked_examples("hand_s3_d2.txt", orc)
    yield lambda: pins.test_hand_worked_examples("hand_gqa_padded.txt", orc)
    yield lambda: pins.test_central_differences(1, 6, 2, 1, 4, None, orc)
    yield lambda: pins.test_central_differences(2, 6, 4, 2, 3, [4, 6], orc)
    yield lambda: pins.test_matches_torch_sdpa_fp64(2, 64, 6, 2, 16, orc)
    yield lambda: pins.test_gqa_equals_explicit_repeat(orc)
    yield lambda: pins.test_padding_equals_prefix_slice_and_ignores_nan(orc)
    yield lambda: pins.test_lse_matches_torch_logsumexp_routine(orc)
    yield lambda: pins.test_hand_worked_examples("hand_noncausal_s3_d2.txt", orc)
    yield lambda: ncpins.test_matches_torch_sdpa_fp64(2, 64, 6, 2, 16, [64, 41], orc)
    yield lambda: ncpins.test_uniform_scores_full_mean(orc)
    yield lambda: ncpins.test_permutation_equivariance(orc)
    yield lambda: dpins.test_equals_last_rows_of_causal_forward(3, 4, 33, 6, 2, 16, [33, 4, 9], orc)
    yield lambda: dpins.test_matches_torch_sdpa_with_mask(orc)
    yield lambda: dpins.test_hand_worked_values(orc)


def test_unmutated_copy_passes_every_pin():
    src = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), mod.__dict__)
    for pin in _pins(mod):
        pin()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    old, new = MUTATIONS[name]
    mod = _mutant(old, new)
    caught = 0
    for pin in _pins(mod):
        try:
            pin()
        except Exception:  # assertion failures, and crashes caused by the mutant
            caught += 1
    assert caught > 0, f"no pin caught mutation {name}"


# ------------------------------------------------------------------ rotary position embedding

import test_oracle_rope as rpins  # noqa: E402

ROPE_SRC = os.path.join(os.path.dirname(SRC), "rope.py")

ROPE_MUTATIONS = {
    "rope_sin_sign": ("out[..., 0::2] = even * c - odd * s", "out[..., 0::2] = even * c + odd * s"),
    "rope_exponent_without_two": ("-2.0 * i / d", "-1.0 * i / d"),
    "rope_positions_from_one": ("np.arange(S, dtype=np.float64) if positions", "np.arange(1, S + 1, dtype=np.float64) if positions"),
    "rope_half_split_pairs": ("even, odd = x[..., 0::2], x[..., 1::2]", "even, odd = x[..., :d // 2], x[..., d // 2:]"),
    "rope_backward_rotates_forward": ('ref["dQ"] = rotate(ref["dQ"], base, inverse=True', 'ref["dQ"] = rotate(ref["dQ"], base, inverse=False'),
    "rope_dK_not_taken_back": ('    ref["dK"] = rotate(ref["dK"], base, inverse=True, dtype=dtype)\n', ""),
    "rope_decode_position_off_by_one": ("pos = lens[b] - Sq + np.arange(Sq)", "pos = lens[b] - Sq + 1 + np.arange(Sq)"),
    "rope_values_rotated": ("ref = attention.backward(qr, kr, v,", "ref = attention.backward(qr, kr, rotate(v, base),"),
}


def _rope_module(src):
    mod = types.ModuleType("oracle_rope_copy")
    exec(compile(src.replace("from . import attention", "from oracle import attention"), "oracle_rope_copy", "exec"),
         mod.__dict__)
    return mod


def _rope_pins(rp):
    yield lambda: rpins.test_position_zero_is_identity(rp)
    yield lambda: rpins.test_head_size_two_is_plane_rotation_by_the_position(rp)
    yield lambda: rpins.test_frequencies_are_powers_of_ten_for_head_size_eight(rp)
    yield lambda: rpins.test_matches_complex_multiplication(rp)
    yield lambda: rpins.test_orthogonal_and_inverse(rp)
    yield lambda: rpins.test_scores_depend_only_on_relative_position(rp)
    yield lambda: rpins.test_central_differences_through_rope(1, 5, 2, 1, 4, None, True, rp)
    yield lambda: rpins.test_matches_torch_complex_rope_and_sdpa(True, rp)
    yield lambda: rpins.test_decode_equals_last_rows_of_rope_forward(3, 4, 33, 6, 2, 16, [33, 4, 9], rp)


def test_unmutated_rope_copy_passes_every_pin():
    mod = _rope_module(open(ROPE_SRC).read())
    for pin in _rope_pins(mod):
        pin()


@pytest.mark.parametrize("name", sorted(ROPE_MUTATIONS))
def test_rope_pins_catch_mutation(name):
    old, new = ROPE_MUTATIONS[name]
    src = open(ROPE_SRC).read()
    assert old in src, old
    mod = _rope_module(src.replace(old, new))
    caught = 0
    for pin in _rope_pins(mod):
        try:
            pin()
        except Exception:
            caught += 1
    assert caught > 0, f"no pin caught mutation {name}"
