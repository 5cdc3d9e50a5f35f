"""Pins for the width and the scale of the oracle's boundary window (CPU).

The parity bar excuses a code mismatch only where a rotated coordinate lies
within 1e-6 of a decision boundary, measured on the coordinate's own scale
sigma = ||x|| / sqrt(d) (the reading of north_star's "1e-6 relative" that keeps
the boundary at 0 usable).  For Lloyd-Max codes that is
|z_j / ||x|| - m_i sqrt(d)| <= 1e-6 with z = H (s * x); for the fp8 far-tier
keys |y_j - mid| <= 1e-6 sigma with y = R x and mid an E4M3 rounding midpoint.

Each case builds an fp32 vector whose coordinate 0 sits a KNOWN distance delta
(in sigma units) from a chosen boundary: x is nonzero on coordinates 0..n
only, x_0 = A s_0 and x_k = s_k for 1 <= k <= n, so that
z_0 = A + n and ||x||^2 = A^2 + n follow from the construction alone (row 0
of a Sylvester Hadamard matrix is all ones).  A is solved for in 60-digit
decimal arithmetic and rounded to fp32; the offset that rounding leaves is
checked to stay within 1e-7 of delta.  The flag must be set for |delta| in
{0.5e-6, 0.8e-6} and clear for |delta| in {1.25e-6, 2e-6}, and the code
must fall on the side of the boundary that delta's sign gives (ties go to
the upper cell, never reached here).  A window ten times too wide or too
narrow, or one measured on the N(0, 1/d) scale instead of sigma (off by
sqrt(d)), fails these cases.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import kvq_oracle as O

getcontext().prec = 60

INSIDE = (0.5e-6, 0.8e-6)
OUTSIDE = (1.25e-6, 2e-6)
N_ONES = 15          # coordinates 1..15 carry s_k, so z_0 / ||x|| reaches sqrt(16) = 4


def _signs(d):
    return O.rademacher_signs(42, d)


def _solve(f, lo, hi):
    """Root of an increasing function on [lo, hi] (Decimal bisection)."""
    lo, hi = Decimal(lo), Decimal(hi)
    for _ in range(200):
        mid = (lo + hi) / 2
        if f(mid) < 0:
            lo = mid
        else:
            hi = mid
    return (lo + hi) / 2


def _fp32_candidates(a: Decimal):
    f = np.float32(float(a))
    return [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]


def _vector(d, a32, neg):
    """The construction: x_0 = A s_0, x_k = s_k (1 <= k <= n), optionally negated."""
    s = _signs(d).astype(np.float32)
    x = np.zeros(d, dtype=np.float32)
    x[0] = a32 * s[0]
    x[1:1 + N_ONES] = s[1:1 + N_ONES]
    return -x if neg else x


def _lm_offset(a, target_abs):
    """(z_0 / ||x|| - |T|) of the construction, for the unnegated vector."""
    a = Decimal(a) if not isinstance(a, Decimal) else a
    return (a + N_ONES) / (a * a + N_ONES).sqrt() - target_abs


def _lm_case(d, bits, i, delta):
    """Vector whose coordinate 0 sits delta (sigma units) from midpoint i."""
    _, mids = O.codebook(bits, d)
    T = Decimal(float(mids[i])) * Decimal(d).sqrt() + Decimal(delta)
    neg = T < 0
    # z_0 / ||x|| = (A + n) / sqrt(A^2 + n) increases on A < 1 from -1 to sqrt(n + 1)
    root = _solve(lambda a: _lm_offset(a, abs(T)), -1e6, 1)
    best = min(_fp32_candidates(root), key=lambda c: abs(_lm_offset(Decimal(float(c)), abs(T))))
    achieved = _lm_offset(Decimal(float(best)), abs(T))          # error of |T| after rounding A
    achieved = float(-achieved if neg else achieved) + delta       # offset from the midpoint, signed
    assert abs(achieved - delta) <= 1e-7, (d, bits, i, delta, achieved)
    return _vector(d, best, neg), i


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lm_window_width_and_scale(d, bits):
    L = 1 << bits
    s = _signs(d)
    for i in sorted({0, L // 2 - 1, L - 2}):          # lowest, central (the boundary at 0) and highest midpoint
        for mag in INSIDE + OUTSIDE:
            for delta in (mag, -mag):
                x, i_mid = _lm_case(d, bits, i, delta)
                codes, _, window = O.quantize_lm(x[None], s, bits)
                want_flag = mag in INSIDE
                assert bool(window[0, 0]) == want_flag, (d, bits, i, delta)
                assert int(codes[0, 0]) == (i_mid + 1 if delta > 0 else i_mid), (d, bits, i, delta)


def _fp8_offset(a, c):
    """((z_0 - c) / ||x||) of the construction, c = sqrt(d) * mid."""
    return (a + N_ONES - c) / (a * a + N_ONES).sqrt()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_window_width_and_scale(d):
    s = _signs(d)
    grid = O.e4m3_decode(np.arange(0x7F))
    for k in (40, 56, 70):                             # midpoints between grid values 0.25.., 1.0.., 4.0..
        lo_v, hi_v = float(grid[k]), float(grid[k + 1])
        c = Decimal(0.5 * (lo_v + hi_v)) * Decimal(d).sqrt()
        for mag in INSIDE + OUTSIDE:
            for delta in (mag, -mag):
                root = _solve(lambda a: _fp8_offset(a, c) - Decimal(delta), -1e4, 1e4)
                best = min(_fp32_candidates(root),
                           key=lambda v: abs(_fp8_offset(Decimal(float(v)), c) - Decimal(delta)))
                achieved = float(_fp8_offset(Decimal(float(best)), c))
                assert abs(achieved - delta) <= 1e-7, (d, k, delta, achieved)
                x = _vector(d, best, False)
                codes, window = O.quantize_fp8(x[None], s)
                assert bool(window[0, 0]) == (mag in INSIDE), (d, k, delta)
                assert int(codes[0, 0]) == (k + 1 if delta > 0 else k), (d, k, delta)
