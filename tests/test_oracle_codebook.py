"""Pins for the oracle's Lloyd-Max codebook (CPU)."""
import math

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import kvq_oracle as O
from tests.conftest import read_golden


def _max_table():
    out = {}
    for ln in read_golden("max1960_gaussian_levels.txt"):
        lv, rest = ln.split(":")
        levels, mse = rest.split("|")
        out[int(lv)] = ([float(v) for v in levels.split()], float(mse))
    return out


@pytest.mark.parametrize("L", [2, 4, 8, 16])
def test_textbook_levels_and_distortion(L):
    want, mse = _max_table()[L]
    g, _ = O.lloyd_max_gaussian(L)
    pos = g[L // 2:]
    # each printed value to its printed precision (last printed digit +- 1)
    for got, w in zip(pos, want):
        digits = len(repr(w).split(".")[1])
        assert abs(got - w) <= 1.01 * 10 ** -digits, (got, w)
    assert abs(_distortion(g) - mse) <= 2e-4 * max(1.0, mse * 100)


def _distortion(g):
    b = np.concatenate([[-np.inf], 0.5 * (g[:-1] + g[1:]), [np.inf]])
    tot = 0.0
    for i, c in enumerate(g):
        v, _ = integrate.quad(lambda x: (x - c) ** 2 * stats.norm.pdf(x), b[i], b[i + 1], epsabs=1e-14)
        tot += v
    return tot


def test_one_bit_closed_form():
    g, b = O.lloyd_max_gaussian(2)
    assert g[1] == pytest.approx(math.sqrt(2 / math.pi), abs=1e-15)
    assert b[0] == 0.0


@pytest.mark.parametrize("L", [4, 8, 16])
def test_fixed_point_conditions_by_quadrature(L):
    """Centroid = conditional mean of its cell, computed by numerical
    integration (independent of the closed form the solver iterates)."""
    g, b = O.lloyd_max_gaussian(L)
    assert np.array_equal(b, 0.5 * (g[:-1] + g[1:]))
    edges = np.concatenate([[-np.inf], b, [np.inf]])
    for i in range(L):
        num, _ = integrate.quad(lambda x: x * stats.norm.pdf(x), edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-13)
        den, _ = integrate.quad(stats.norm.pdf, edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-13)
        assert abs(num / den - g[i]) < 1e-10
    # exact antisymmetry and strict order
    assert np.array_equal(g, -g[::-1])
    assert np.all(np.diff(g) > 0)


@pytest.mark.parametrize("L", [4, 8, 16])
def test_closed_form_residual_tiny(L):
    g, b = O.lloyd_max_gaussian(L)
    edges = np.concatenate([[-np.inf], b, [np.inf]])
    res = max(abs(O.gaussian_conditional_mean(edges[i], edges[i + 1]) - g[i]) for i in range(L))
    assert res < 1e-12


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_float32_table_and_midpoints(bits, d):
    c, m = O.codebook(bits, d)
    assert c.dtype == np.float32 and len(c) == 2 ** bits
    assert np.array_equal(c, -c[::-1])
    g, _ = O.lloyd_max_gaussian(2 ** bits)
    assert np.allclose(c, g / math.sqrt(d), rtol=6e-8, atol=0)
    c64 = c.astype(np.float64)
    assert np.array_equal(m, (c64[:-1] + c64[1:]) / 2)
    assert m[len(m) // 2] == 0.0


@pytest.mark.parametrize("bits,dist", [(2, 0.117482), (3, 0.034548), (4, 0.009501)])
def test_quantizer_mse_on_gaussian_vectors(bits, dist):
    """Relative MSE of the whole codec on N(0,1) vectors stays near the
    codebook's Gaussian distortion (rotation of an isotropic vector is
    isotropic; the unit-norm coordinates are close to N(0,1/d))."""
    d = 128
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3000, d)).astype(np.float16)
    s = O.rademacher_signs(42, d)
    codes, norms, _ = O.quantize_lm(x, s, bits)
    xr = O.rotate(x.astype(np.float64), s)
    xh = O.dequantize_lm(codes, norms, bits)
    rel = np.sum((xr - xh) ** 2, axis=-1) / np.sum(xr ** 2, axis=-1)
    assert abs(rel.mean() / dist - 1.0) < 0.03
