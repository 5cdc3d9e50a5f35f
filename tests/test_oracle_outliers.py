"""Pins of the oracle's outlier two-stream key cache ([Velox] "Outlier
Two-Stream Cache"): calibration finds planted high-variance channels,
the int8 stream rounds as written out by hand, and the two score parts
add up to the full key's score."""
import math

import numpy as np

from oracle import kvq_oracle as O


def test_calibration_finds_planted_channels_and_breaks_ties_low():
    rng = np.random.default_rng(3)
    B, H, N, d = 2, 3, 64, 128
    x = rng.standard_normal((B, H, N, d))
    planted = np.zeros((B, H, 8), np.int64)
    for b in range(B):
        for h in range(H):
            ch = np.sort(rng.choice(d, 8, replace=False))
            x[b, h][:, ch] *= 20.0
            planted[b, h] = ch
    assert np.array_equal(O.calibrate_outliers(x), planted)
    # equal variances everywhere: the lowest channels
    assert np.array_equal(O.calibrate_outliers(np.ones((1, 1, 5, 16))), np.arange(8)[None, None])
    # two channels tie for the 8th place: the lower one wins
    y = np.zeros((1, 1, 4, 16))
    y[0, 0, :, [1, 2, 3, 4, 5, 6, 7]] = np.array([[0, 9, 0, 9]] * 7)
    y[0, 0, :, [10, 12]] = np.array([[0, 1, 0, 1]] * 2)
    assert np.array_equal(O.calibrate_outliers(y)[0, 0], [1, 2, 3, 4, 5, 6, 7, 10])


def test_int8_stream_rounding_by_hand():
    xo = np.array([127, -63.5, 0.5, 1.5, 2.5, -127, 0, 3], np.float32)
    codes, scale = O.quantize_outliers(xo)
    assert scale == np.float32(1.0)
    assert codes.tolist() == [127, -64, 0, 2, 2, -127, 0, 3]          # nearest, ties to even
    z, sz = O.quantize_outliers(np.zeros(8, np.float32))
    assert sz == 0 and not z.any()
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((1000, 8)) * 30).astype(np.float16)
    c, s = O.quantize_outliers(x)
    err = np.abs(O.dequantize_outliers(c, s) - x.astype(np.float64))
    assert np.all(err <= s.astype(np.float64)[:, None] * 0.5 * (1 + 1e-6))
    assert np.all(np.abs(c).max(axis=1) == 127)
    assert np.array_equal(s, (np.abs(x.astype(np.float32)).max(axis=1) / np.float32(127)).astype(np.float32))


def test_split_and_two_stream_scores_add_up():
    """With the codec part left unquantised (the exact rotation of the key
    with its outlier channels zeroed) and outlier values the int8 grid holds
    exactly, two-stream attention is plain attention on the full keys."""
    rng = np.random.default_rng(5)
    B, Hkv, G, T, d = 1, 2, 2, 40, 64
    s = O.rademacher_signs(42, d)
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    idx = np.sort(np.stack([rng.choice(d, 8, replace=False) for _ in range(B * Hkv)]).reshape(B, Hkv, 8), axis=-1)
    grid = rng.integers(-127, 128, (B, Hkv, T, 8)).astype(np.float64)
    grid[..., 0] = 127                                   # max |code| = 127, so the scale is exactly 0.5
    sel = np.broadcast_to(idx[:, :, None, :], (B, Hkv, T, 8))
    np.put_along_axis(k, sel, grid * 0.5, axis=3)
    ki, ko = O.split_outliers(k, idx)
    assert np.all(np.take_along_axis(ki, sel, axis=3) == 0) and np.array_equal(ko, grid * 0.5)
    codes, scale = O.quantize_outliers(ko.astype(np.float32))
    assert np.all(scale == np.float32(0.5)) and np.array_equal(codes, grid.astype(np.int8))
    q = rng.standard_normal((B, Hkv * G, d))
    got = O.two_stream_attention(q, O.rotate(ki, s), O.rotate(v, s), idx, codes, scale, s)
    want = O.attention_original_domain(q, O.rotate(k, s), O.rotate(v, s), s)
    assert np.allclose(got, want, atol=1e-12)
    # no outlier energy: the plain rotated-domain attention
    k0 = k.copy()
    np.put_along_axis(k0, sel, 0.0, axis=3)
    z, zs = O.quantize_outliers(np.zeros((B, Hkv, T, 8), np.float32))
    assert np.allclose(O.two_stream_attention(q, O.rotate(k0, s), O.rotate(v, s), idx, z, zs, s),
                       O.attention(q, O.rotate(k0, s), O.rotate(v, s), s), atol=1e-12)
