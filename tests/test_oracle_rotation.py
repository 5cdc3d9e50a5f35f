"""Pins for the oracle's signs and Hadamard rotation (CPU)."""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import kvq_oracle as O
from tests.conftest import read_golden


def test_splitmix64_published_vectors():
    lines = read_golden("splitmix64_seed0.txt")
    seed = int(lines[0].split()[1])
    want = [int(v, 16) for v in lines[1:]]
    assert O.splitmix64(seed, len(want)) == want


def test_signs_are_top_bits_and_balanced():
    s = O.rademacher_signs(42, 4096)
    raw = O.splitmix64(42, 4096)
    assert set(np.unique(s)) == {-1, 1}
    assert all((v >> 63 == 0) == (x == 1) for v, x in zip(raw, s))
    assert abs(int(s.sum())) < 4 * math.sqrt(4096)


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_hadamard_matches_library_and_is_orthogonal(d):
    H = O.hadamard(d)
    assert np.array_equal(H, scipy.linalg.hadamard(d))
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, d * np.eye(d, dtype=np.int64))


@pytest.mark.parametrize("d", [8, 128, 256])
def test_fwht_butterflies_equal_matrix(d):
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1000, size=(5, d))
    assert np.array_equal(O.fwht(x), x @ O.hadamard(d))


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_orthonormal_and_inverse(d):
    rng = np.random.default_rng(1)
    s = O.rademacher_signs(42, d)
    x = rng.standard_normal((7, d))
    y = O.rotate(x, s)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    assert np.allclose(O.rotate_inverse(y, s), x, atol=1e-14)
    # sign flip happens before the transform: R e_j = s_j * H[:, j] / sqrt(d)
    e = np.zeros(d); e[3] = 1.0
    assert np.allclose(O.rotate(e, s), s[3] * O.hadamard(d)[:, 3] / math.sqrt(d))


def test_rotation_spreads_an_outlier():
    # one huge channel becomes d equal-magnitude coordinates
    d = 128
    s = O.rademacher_signs(42, d)
    x = np.zeros(d); x[17] = 20.0
    y = O.rotate(x, s)
    assert np.allclose(np.abs(y), 20.0 / math.sqrt(d))
