"""Pins of the oracle's QJL residual sketch (VeloxQuant-MLX, "Stage 3: QJL
Residual Correction"; "Memory Layout: What Actually Gets Stored").

The page prints the estimator in a form that cannot be unbiased; the oracle
takes the form fixed by the page's stored quantities (the signs of S r, the
norm of r) and its stated property (unbiased over the random projection).
These pins check that property and its closed-form variance by Monte Carlo,
a hand case with the identity projection, the residual against the codec,
and the whole path (codes, residual, sketch, estimate) by the slope of the
corrected scores against the exact ones."""
import math

import numpy as np

from oracle import kvq_oracle as O


def test_estimator_is_unbiased_with_closed_form_variance():
    """Over Gaussian projections S (m rows), the estimate of q . r has mean
    q . r and variance ((pi/2) |r|^2 |q|^2 - (q . r)^2) / m: one row gives
    sqrt(pi/2) |r| (S_i . q) sign(S_i . r), whose mean is q . r because
    E[g sign(h)] = sqrt(2/pi) cov(g, h) / sd(h) for jointly Gaussian g, h, and
    whose second moment is (pi/2) |r|^2 |q|^2."""
    rng = np.random.default_rng(5)
    d = m = 16
    q = rng.standard_normal(d)
    r = 0.3 * rng.standard_normal(d)
    N = 40000
    S = rng.standard_normal((N, m, d))
    z, _ = O.qjl_sketch_bits(r, S)
    est = O.qjl_estimate(q, np.linalg.norm(r), z, S)
    true = float(q @ r)
    var = (math.pi / 2 * (r @ r) * (q @ q) - true ** 2) / m
    se = math.sqrt(var / N)
    assert abs(est.mean() - true) < 5 * se, (est.mean(), true, se)
    assert 0.95 < est.var() / var < 1.05, est.var() / var
    # the printed form (query side reduced to signs too) misses the product
    sq = np.einsum("nmd,d->nm", S, q)
    printed = np.linalg.norm(r) * (math.pi / 2 / m) * ((2.0 * z - 1.0) * np.sign(sq)).sum(axis=-1)
    assert abs(printed.mean() - true) > 20 * se


def test_identity_projection_by_hand():
    """With S = I the sketch is the sign pattern of r itself (sign(0) = +1),
    packed LSB-first, and the estimate is |r| sqrt(pi/2)/m sum_j sign(r_j) q_j."""
    r = np.array([0.5, -0.25, 0.0, -1.0, 2.0, -0.0, 1e-30, -3.0])
    S = np.eye(8)
    z, win = O.qjl_sketch_bits(r, S)
    assert z.tolist() == [1, 0, 1, 0, 1, 1, 1, 0]
    assert O.pack(z, 1).tolist() == [0b01110101]
    assert not win[[0, 1, 3, 4, 7]].any() and win[2] and win[5]       # exact zeros sit on the boundary
    q = np.arange(1.0, 9.0)
    # sum_j (2 z_j - 1) q_j = 1 - 2 + 3 - 4 + 5 + 6 + 7 - 8 = 8
    norm = math.sqrt(0.25 + 0.0625 + 1.0 + 4.0 + 1e-60 + 9.0)
    assert math.isclose(O.qjl_estimate(q, norm, z, S), norm * math.sqrt(math.pi / 2) / 8 * 8.0, rel_tol=1e-15)


def test_residual_closes_the_codec():
    """khat + r is the rotated key; the stored residual norm is numpy's
    correctly rounded fp16 of |r|; |r|^2 / |y|^2 is the codec's distortion
    (Max's Gaussian values 0.034548 at 3 bits, 0.009501 at 4 bits, within 3%
    at d = 128)."""
    rng = np.random.default_rng(3)
    s = O.rademacher_signs(42, 128)
    x = rng.standard_normal((4000, 128)).astype(np.float16)
    y = O.rotate(x, s)
    for bits, D in ((3, 0.034548), (4, 0.009501)):
        r, codes, norms, _ = O.qjl_residual(x, s, bits)
        assert np.allclose(O.dequantize_lm(codes, norms, bits) + r, y, rtol=0, atol=1e-15)
        rn, near = O.qjl_norm_bits(r)
        assert not near.any()
        assert np.array_equal(rn, np.linalg.norm(r, axis=-1).astype(np.float16).view(np.uint16))
        ratio = (r * r).sum() / (y * y).sum()
        assert abs(ratio / D - 1) < 0.03, (bits, ratio)


def test_corrected_scores_have_unit_slope():
    """Whole path on fp16 Gaussian keys (3-bit codes, fresh S per key): the
    corrected score regresses on the exact score q~ . R k with slope 1 (the
    estimate is unbiased given each key); the codec alone shrinks it by about
    its distortion, and a correction with its sign flipped shrinks it twice
    as much."""
    rng = np.random.default_rng(11)
    d, bits, N = 32, 3, 20000
    s = O.rademacher_signs(42, d)
    x = rng.standard_normal((N, d)).astype(np.float16)
    q = rng.standard_normal(d)
    S = rng.standard_normal((N, d, d))
    enc = O.qjl_encode(x[:, None, :], s, bits, S[0])          # the per-key S below; shapes only
    assert enc["sketch"].shape == (N, 1, d // 8)
    r, codes, norms, _ = O.qjl_residual(x, s, bits)
    z, _ = O.qjl_sketch_bits(r, S)
    rn, _ = O.qjl_norm_bits(r)
    exact = O.rotate(x, s) @ q
    codec = O.dequantize_lm(codes, norms, bits) @ q
    est = O.qjl_estimate(q, O.fp16_bits_to_f64(rn), z, S)

    def slope(a):
        c = exact - exact.mean()
        return float(c @ (a - a.mean()) / (c @ c))
    assert abs(slope(codec + est) - 1) < 0.006, slope(codec + est)
    assert slope(codec) < 0.985
    assert slope(codec - est) < 0.955


def test_attention_forms_agree_and_reduce():
    """QJL attention equals plain attention over the effective keys
    khat + |r| sqrt(pi/2)/m S^T (2z - 1); with zero residual norms it is plain
    attention over the codec; with one token it returns that token's value."""
    rng = np.random.default_rng(9)
    B, Hkv, G, T, d = 2, 2, 2, 7, 16
    s = O.rademacher_signs(42, d)
    q = rng.standard_normal((B, Hkv * G, d))
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    S = rng.standard_normal((d, d)).astype(np.float32)
    enc = O.qjl_encode(k, s, 3, S)
    kh = O.dequantize_lm(enc["codes"], enc["norms"], 3)
    vc, vn, _ = O.quantize_lm(v, s, 3)
    vh = O.dequantize_lm(vc, vn, 3)
    z = enc["sketch_bits"]
    got = O.qjl_attention(q, kh, vh, enc["rnorm"], z, S, s)
    eff = O.qjl_effective_keys(kh, enc["rnorm"], z, S)
    assert np.allclose(got, O.attention(q, eff, vh, s), rtol=0, atol=1e-12)
    zero = np.zeros_like(enc["rnorm"])
    assert np.allclose(O.qjl_attention(q, kh, vh, zero, z, S, s), O.attention(q, kh, vh, s), rtol=0, atol=1e-12)
    one = O.qjl_attention(q, kh[:, :, :1], vh[:, :, :1], enc["rnorm"][:, :, :1], z[:, :, :1], S, s)
    want = np.repeat(O.rotate_inverse(vh[:, :, 0], s), G, axis=1)
    assert np.allclose(one, want, rtol=0, atol=1e-12)


def test_zero_key_has_empty_sketch():
    """A zero key: codes at 2^(b-1), zero norm, zero residual, every sketch
    bit set (sign(0) = +1), zero residual norm, nothing in a window."""
    s = O.rademacher_signs(42, 64)
    S = np.random.default_rng(1).standard_normal((64, 64)).astype(np.float32)
    enc = O.qjl_encode(np.zeros((1, 64), np.float16), s, 2, S)
    assert (enc["codes"] == 2).all() and enc["norms"][0] == 0
    assert (enc["sketch"] == 0xFF).all() and enc["rnorm"][0] == 0
    assert not enc["sketch_window"].any() and not enc["rnorm_window"].any()
