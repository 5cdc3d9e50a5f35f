"""Pins for the oracle's packing, norms, codes and fp8 codec (CPU)."""
import math

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
from tests.conftest import read_golden


def _kv(lines):
    return {ln.split()[0]: ln.split()[1:] for ln in lines}


def test_packing_page_example():
    g = _kv(read_golden("packing_3bit_example.txt"))
    bits = int(g["bits"][0])
    codes = np.array([[int(v) for v in g["codes"]]], dtype=np.uint8)
    want = [int(v, 16) for v in g["bytes"]]
    # the page's example is 5 codes = 15 bits; pad the stream to 8 codes (3 bytes)
    padded = np.zeros((1, 8), dtype=np.uint8)
    padded[0, :5] = codes
    got = O.pack(padded, bits)[0]
    assert list(got[:2]) == want
    assert O.unpack(got[None], bits, 8)[0, :5].tolist() == codes[0].tolist()


def test_packing_2bit_shifts_and_4bit_nibbles():
    shifts = [int(v) for v in _kv(read_golden("packing_2bit_shifts.txt"))["shifts"]]
    rng = np.random.default_rng(0)
    c2 = rng.integers(0, 4, size=(3, 128), dtype=np.uint8)
    p2 = O.pack(c2, 2)
    assert p2.shape == (3, 32)
    for i, sh in enumerate(shifts):
        assert np.array_equal((p2 >> sh) & 3, c2[:, i::4])
    c4 = rng.integers(0, 16, size=(3, 128), dtype=np.uint8)
    p4 = O.pack(c4, 4)
    assert np.array_equal(p4 & 15, c4[:, 0::2]) and np.array_equal(p4 >> 4, c4[:, 1::2])


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256])
def test_pack_roundtrip(bits, d):
    rng = np.random.default_rng(bits * d)
    c = rng.integers(0, 2 ** bits, size=(9, d), dtype=np.uint8)
    p = O.pack(c, bits)
    assert p.shape == (9, d * bits // 8)
    assert np.array_equal(O.unpack(p, bits, d), c)
    # brute force: stream bit b*j+k is bit k of code j
    for r in range(9):
        stream = sum(int(v) << (bits * j) for j, v in enumerate(c[r]))
        assert bytes(p[r]) == stream.to_bytes(d * bits // 8, "little")


def _norm_value(bits):
    return float(np.array(bits, dtype=np.uint16).view(np.float16))


def test_norm_integer_vectors():
    d = 128
    s = O.rademacher_signs(42, d)
    x = np.zeros((3, d), dtype=np.float16)
    x[0, :2] = [3, 4]                     # 5
    x[1, :4] = [1, 1, 1, 1]               # 2
    x[2, 0] = 0.0                         # zero vector
    _, n, _ = O.quantize_lm(x, s, 4)
    assert [_norm_value(v) for v in n] == [5.0, 2.0, 0.0]


def test_norm_matches_numpy_rounding_away_from_midpoints():
    d = 256
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((400, d)) * rng.lognormal(0, 2, size=(400, 1))).astype(np.float16)
    s = O.rademacher_signs(42, d)
    _, n, _ = O.quantize_lm(x, s, 3)
    ref = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1))      # error ~1e-16
    assert np.array_equal(n, ref.astype(np.float16).view(np.uint16))


def test_norm_exact_midpoint_ties_and_overflow():
    # ||x|| exactly halfway between fp16 1.0 and 1.0009765625 -> even (1.0)
    S = (1 + 2 ** -11) ** 2
    assert O.rne_fp16_sqrt(__import__("fractions").Fraction(S)) == 0x3C00
    # just above the midpoint -> 1.0009765625
    from fractions import Fraction
    assert O.rne_fp16_sqrt(Fraction(S) + Fraction(1, 2 ** 60)) == 0x3C01
    assert O.rne_fp16_sqrt(Fraction(65520) ** 2) == 0x7C00       # overflow -> inf
    assert O.rne_fp16_sqrt(Fraction(65519) ** 2) == 0x7BFF


def test_codes_unit_vector_closed_form():
    """x = e_k: z = s_k * H[:, k], so every coordinate of the unit vector is
    +-1/sqrt(d); +1 lands in the 4-bit cell (0.7996, 1.0993] of N(0,1) = index 11,
    -1 in index 4."""
    d = 128
    s = O.rademacher_signs(42, d)
    H = O.hadamard(d)
    x = np.zeros((1, d), dtype=np.float16); x[0, 5] = 1.0
    codes, n, win = O.quantize_lm(x, s, 4)
    want = np.where(s[5] * H[:, 5] > 0, 11, 4)
    assert np.array_equal(codes[0], want) and not win.any()
    assert _norm_value(n[0]) == 1.0


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_codes_are_nearest_centroid(bits, dtype):
    """Interval search against midpoints == nearest centroid of the unit-norm
    rotated coordinate ([Velox] Stage 2: 'find nearest centroid')."""
    d = 128
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, d)).astype(dtype)
    x[:, 7] *= 20
    s = O.rademacher_signs(42, d)
    codes, _, win = O.quantize_lm(x, s, bits)
    c, _ = O.codebook(bits, d)
    y = O.rotate(x.astype(np.float64), s)
    u = y / np.linalg.norm(x.astype(np.float64), axis=-1, keepdims=True)
    nearest = np.argmin(np.abs(u[..., None] - c.astype(np.float64)), axis=-1)
    assert np.array_equal(codes[~win], nearest[~win])


def test_codes_exact_tie_goes_up():
    """A coordinate exactly on the midpoint 0 (z_j = 0) takes the upper cell."""
    d = 8
    s = np.ones(d, dtype=np.int8)
    x = np.array([[1, 1, 0, 0, 0, 0, 0, 0]], dtype=np.float16)   # z = (2,0,2,0,2,0,2,0)
    codes, _, _ = O.quantize_lm(x, s, 2)
    assert codes[0, 1] == 2 and codes[0, 3] == 2          # 0 -> upper cell (index L/2)
    assert np.all(codes[0, ::2] >= 2)


def test_zero_vector_codes():
    s = O.rademacher_signs(42, 128)
    codes, n, _ = O.quantize_lm(np.zeros((2, 128), np.float16), s, 3)
    assert np.all(codes == 4) and np.all(n == 0)


def test_e4m3_table_values():
    for ln in read_golden("e4m3fn_values.txt"):
        val, code = float(ln.split()[0]), int(ln.split()[1], 16)
        got = _e4m3_of_value(val)
        assert got == code, (val, hex(got), hex(code))
        on_grid = abs(val) <= 448 and val in set(O.e4m3_decode(np.arange(0x7F)).tolist()) | {-1.0}
        if on_grid:
            assert O.e4m3_decode(np.array([code]))[0] == val


def _e4m3_of_value(val):
    """Drive quantize_fp8 with a vector whose rotation has `val` in coordinate 0.
    With s = +1 and x = val/sqrt(d) * H[:, 0] ... simpler: d = 256 so that
    y = H x / 16; x = (16 val / 256) * ones gives y_0 = val exactly."""
    d = 256
    x = np.full((1, d), val / 16.0, dtype=np.float32)
    codes, _ = O.quantize_fp8(x, np.ones(d, np.int8))
    return int(codes[0, 0])


def test_e4m3_matches_torch_after_clamp():
    rng = np.random.default_rng(5)
    d = 128
    x = (rng.standard_normal((200, d)) * rng.lognormal(0, 2.5, size=(200, 1))).astype(np.float16)
    s = O.rademacher_signs(42, d)
    codes, win = O.quantize_fp8(x, s)
    y = O.rotate(x.astype(np.float64), s)
    ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[~win], ref[~win])
    assert win.mean() < 1e-3
    assert np.allclose(O.e4m3_decode(np.arange(256)[np.arange(256) & 0x7F != 0x7F]),
                       torch.from_numpy(np.arange(256, dtype=np.uint8)[np.arange(256) & 0x7F != 0x7F])
                       .view(torch.float8_e4m3fn).to(torch.float64).numpy())
