"""Planted mistakes in the oracle (on the CPU only): each plausible slip in
its arithmetic must make at least one pin fail.  The mutations are applied
with monkeypatch and undone after each test."""
import math

import numpy as np
import pytest

from oracle import kvq_oracle as O
from tests import test_oracle_attention as TA
from tests import test_oracle_codebook as TC
from tests import test_oracle_codec as TK
from tests import test_oracle_rotation as TR


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_hadamard_wrong_sign_is_caught(monkeypatch):
    good = O.hadamard

    def bad(d):
        H = good(d).copy()
        H[1] *= -1
        return H
    monkeypatch.setattr(O, "hadamard", bad)
    _fails(TR.test_hadamard_matches_library_and_is_orthogonal, 8)


def test_sign_flip_after_transform_is_caught(monkeypatch):
    def bad(x, signs):
        d = x.shape[-1]
        return (np.asarray(x, np.float64) @ O.hadamard(d).astype(np.float64)) * signs / math.sqrt(d)
    monkeypatch.setattr(O, "rotate", bad)
    _fails(TR.test_rotation_orthonormal_and_inverse, 128)


def test_dropped_term_in_conditional_mean_is_caught(monkeypatch):
    monkeypatch.setattr(O, "gaussian_conditional_mean", lambda a, b: O._phi(a) / O._cell_mass(a, b))
    O._gaussian_levels.cache_clear()
    try:
        _fails(TC.test_fixed_point_conditions_by_quadrature, 8)
    finally:
        O._gaussian_levels.cache_clear()


def test_msb_first_packing_is_caught(monkeypatch):
    good = O.pack
    monkeypatch.setattr(O, "pack", lambda c, b: np.packbits(
        ((np.asarray(c, np.uint8)[..., None] >> np.arange(b - 1, -1, -1, dtype=np.uint8)) & 1)
        .reshape(*np.shape(c)[:-1], -1), axis=-1, bitorder="big"))
    _fails(TK.test_packing_page_example)
    monkeypatch.setattr(O, "pack", good)


def test_ties_to_lower_cell_is_caught(monkeypatch):
    from fractions import Fraction

    def strict(z, m, dS):
        M = Fraction(m)
        if M >= 0:
            return z > 0 and Fraction(z) ** 2 > M * M * dS
        return z >= 0 or Fraction(z) ** 2 < M * M * dS
    monkeypatch.setattr(O, "_z_ge_m_sqrt", strict)
    _fails(TK.test_codes_exact_tie_goes_up)


def test_missing_softmax_scale_is_caught(monkeypatch):
    good = O.rotate
    monkeypatch.setattr(O, "rotate", lambda x, s: good(x, s) * math.sqrt(x.shape[-1]) ** 0.5)
    _fails(TA.test_identity_codec_equals_library_sdpa)


def test_merge_without_rescale_is_caught(monkeypatch):
    def bad(m, l, o):
        W = l.sum()
        return (l[:, None] * o).sum(axis=0) / W, float(np.max(m))
    monkeypatch.setattr(O, "merge_partials", bad)
    _fails(TA.test_split_merge_invariance, 7, 1)


def test_gqa_head_map_mod_instead_of_div_is_caught(monkeypatch):
    good = np.repeat

    def tile(a, G, axis=None):
        return np.tile(a, (1, G) + (1,) * (a.ndim - 2)) if axis == 1 else good(a, G, axis=axis)
    monkeypatch.setattr(O.np, "repeat", tile)
    _fails(TA.test_gqa_head_map_and_mha_reduction)


def test_qjl_constant_pi_over_2_is_caught(monkeypatch):
    from tests import test_oracle_qjl as TQ
    good = O.qjl_estimate
    monkeypatch.setattr(O, "qjl_estimate",
                        lambda q, rn, z, S: good(q, rn, z, S) * math.sqrt(math.pi / 2))   # pi/2 in place of sqrt(pi/2)
    _fails(TQ.test_estimator_is_unbiased_with_closed_form_variance)


def test_qjl_residual_sign_is_caught(monkeypatch):
    from tests import test_oracle_qjl as TQ
    good = O.qjl_residual

    def bad(x, signs, bits):
        r, c, n, w = good(x, signs, bits)
        return -r, c, n, w
    monkeypatch.setattr(O, "qjl_residual", bad)
    _fails(TQ.test_corrected_scores_have_unit_slope)


def test_qjl_sign_of_zero_is_caught(monkeypatch):
    from tests import test_oracle_qjl as TQ
    good = O.qjl_sketch_bits

    def bad(r, S):
        z, w = good(r, S)
        dots = np.einsum("...md,...d->...m", np.asarray(S, np.float64), np.asarray(r, np.float64))
        return np.where(dots == 0.0, 0, z).astype(np.uint8), w
    monkeypatch.setattr(O, "qjl_sketch_bits", bad)
    _fails(TQ.test_identity_projection_by_hand)


def test_window_hundred_times_too_wide_is_caught(monkeypatch):
    from tests import test_oracle_window as TW
    monkeypatch.setattr(O, "WINDOW", 100 * O.WINDOW)
    _fails(TW.test_lm_window_width_and_scale, 128, 4)
    _fails(TW.test_fp8_window_width_and_scale, 128)


def test_window_ten_times_too_narrow_is_caught(monkeypatch):
    from tests import test_oracle_window as TW
    monkeypatch.setattr(O, "WINDOW", O.WINDOW / 10)
    _fails(TW.test_lm_window_width_and_scale, 64, 2)
    _fails(TW.test_fp8_window_width_and_scale, 256)


def test_window_on_the_unit_scale_is_caught(monkeypatch):
    """A window measured on u = z / (sqrt(d) ||x||) (the N(0, 1/d) scale)
    instead of the coordinate's sigma is sqrt(d) times too wide."""
    from tests import test_oracle_window as TW
    monkeypatch.setattr(O, "WINDOW", O.WINDOW * (128 ** 0.5))
    _fails(TW.test_lm_window_width_and_scale, 128, 3)
