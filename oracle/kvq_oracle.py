"""Plain CPU oracle for rotation-based KV-cache quantization and decode attention
computed on the compressed cache.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP library: it is written from the method's description alone, in numpy
float64, with exact integer / rational arithmetic wherever a floating-point
value decides an integer (a code, a rounding direction).

Sources (page titles as published; sections named in each docstring):
  [AdapTQ]   "Shrinking the LLM KV Cache by 8x on CPU: The Engineering Behind
             AdapTQ" -- sections "The Math Fix", "Engineering the Hot Path".
  [Foveated] "FoveatedKV" -- sections "The VR headset thing", "Making it fast".
  [Velox]    "I Ported a Google Research Paper to Apple Silicon" (VeloxQuant-MLX)
             -- sections "The Core Idea", "Stage 1: Random Rotation",
             "Stage 2: Lloyd-Max Scalar Quantization", "Stage 3: QJL Residual
             Correction", "The Bit-Packing Problem", "Outlier Two-Stream Cache".

Readings taken where the pages are silent (each also listed in the design
notes): signs from SplitMix64 (top bit), Sylvester-ordered Hadamard with
orthonormal 1/sqrt(d) scaling, sign flip applied before the transform,
2^b Lloyd-Max levels for N(0,1) scaled by 1/sqrt(d) and rounded to float32,
decision boundaries at the exact midpoints of that float32 table, codes decided
against the exact norm, ties to the upper cell, zero vector -> norm 0 and code
2^(b-1), dequantization with the stored fp16 norm.

Every function here is pinned by tests against something other than itself
(see tests/test_oracle_*.py); none is "parity unpinned".
"""
from __future__ import annotations

import functools
import math
from fractions import Fraction

import numpy as np

MASK64 = (1 << 64) - 1

# ----------------------------------------------------------------------------
# Seeded Rademacher signs  ([Velox] "Stage 1": r is a random +-1 vector;
# the seed parameter is the builder's with_seed).
# ----------------------------------------------------------------------------


def splitmix64(seed: int, n: int) -> list[int]:
    """SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): state += golden gamma,
    output = variant-13 mix of the state.  Returns n 64-bit outputs."""
    state = seed & MASK64
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        out.append(z ^ (z >> 31))
    return out


def rademacher_signs(seed: int, d: int) -> np.ndarray:
    """s_j = +1 if the top bit of the j-th SplitMix64 output is 0, else -1."""
    return np.array([1 if (v >> 63) == 0 else -1 for v in splitmix64(seed, d)], dtype=np.int8)


# ----------------------------------------------------------------------------
# Walsh-Hadamard rotation  ([AdapTQ] "The Math Fix"; [Velox] "Stage 1")
# ----------------------------------------------------------------------------


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix, H[i, j] = (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d, dtype=np.int64)
    parity = np.zeros((d, d), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while np.any(a):
        parity ^= a & 1
        a = a >> 1
    return np.where(parity == 0, 1, -1).astype(np.int64)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis,
    Sylvester order (butterflies a+b, a-b at strides 1, 2, 4, ...)."""
    x = np.array(x, copy=True)
    d = x.shape[-1]
    h = 1
    while h < d:
        y = x.reshape(*x.shape[:-1], d // (2 * h), 2, h)
        a, b = y[..., 0, :], y[..., 1, :]
        x = np.stack([a + b, a - b], axis=-2).reshape(x.shape)
        h *= 2
    return x


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R x = H (s * x) / sqrt(d) in float64 (R orthonormal)."""
    d = x.shape[-1]
    H = hadamard(d).astype(np.float64)
    return (np.asarray(x, np.float64) * signs.astype(np.float64)) @ H / math.sqrt(d)


def rotate_inverse(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R^T y = s * (H y) / sqrt(d) in float64."""
    d = y.shape[-1]
    H = hadamard(d).astype(np.float64)
    return (np.asarray(y, np.float64) @ H) * signs.astype(np.float64) / math.sqrt(d)


# ----------------------------------------------------------------------------
# Lloyd-Max codebook for a Gaussian  ([Velox] "The Core Idea": boundaries at
# centroid midpoints, centroid = conditional mean of its cell; "Stage 2":
# computed once, reused for every token)
# ----------------------------------------------------------------------------

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi(x: float) -> float:
    return 0.0 if math.isinf(x) else _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _cell_mass(a: float, b: float) -> float:
    """Phi(b) - Phi(a) without cancellation (complementary form on each side)."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / _SQRT2) - math.erfc(b / _SQRT2))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / _SQRT2) - math.erfc(-a / _SQRT2))
    return 1.0 - 0.5 * math.erfc(-a / _SQRT2) - 0.5 * math.erfc(b / _SQRT2)


def gaussian_conditional_mean(a: float, b: float) -> float:
    """E[X | a < X < b] for X ~ N(0,1): (phi(a) - phi(b)) / (Phi(b) - Phi(a))."""
    return (_phi(a) - _phi(b)) / _cell_mass(a, b)


def lloyd_max_gaussian(levels: int, tol: float = 1e-15, max_iter: int = 1_000_000):
    """Fixed point of the two Lloyd-Max conditions for N(0,1) with `levels`
    reconstruction points.  Returns (centroids, boundaries) in float64,
    ascending, exactly antisymmetric.  Iterates the plain Lloyd map from the
    Gaussian quantiles until the largest change is below `tol`."""
    if levels < 2:
        raise ValueError("need at least two levels")
    c = np.array([_inv_norm_cdf((i + 0.5) / levels) for i in range(levels)])
    c = 0.5 * (c - c[::-1])
    for _ in range(max_iter):
        b = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate([[-math.inf], b, [math.inf]])
        new = np.array([gaussian_conditional_mean(edges[i], edges[i + 1]) for i in range(levels)])
        new = 0.5 * (new - new[::-1])
        delta = float(np.max(np.abs(new - c)))
        c = new
        if delta < tol:
            break
    return c, 0.5 * (c[:-1] + c[1:])


def _inv_norm_cdf(p: float) -> float:
    """Gaussian quantile by bisection on erfc (initialisation only)."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / _SQRT2) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


@functools.lru_cache(maxsize=None)
def _gaussian_levels(levels: int):
    return lloyd_max_gaussian(levels)[0]


def codebook(bits: int, d: int):
    """Centroid table for N(0, 1/d): c_i = RN_float32(gamma_i / sqrt(d)),
    ascending; decision midpoints m_i = (c_i + c_{i+1}) / 2 (exact in float64)."""
    gamma = _gaussian_levels(1 << bits)
    c = (gamma / math.sqrt(d)).astype(np.float32)
    c64 = c.astype(np.float64)
    return c, 0.5 * (c64[:-1] + c64[1:])


# ----------------------------------------------------------------------------
# Exact helpers
# ----------------------------------------------------------------------------


def _to_int_grid(x: np.ndarray):
    """Exact integer representation x = X * 2^-E of an fp16 / fp32 array."""
    if x.dtype == np.float16:
        E = 24
        X = (x.astype(np.float64) * 2.0 ** E).astype(np.int64)   # |X| < 2^40, exact
        return X, E, False
    if x.dtype == np.float32:
        E = 149
        flat = [int(Fraction(float(v)) * (1 << E)) for v in x.reshape(-1)]
        return np.array(flat, dtype=object).reshape(x.shape), E, True
    raise TypeError("inputs are fp16 or fp32")


def _sum_squares_exact(X: np.ndarray, big: bool) -> list[int]:
    """Exact sum over the last axis of X^2 (Python ints, one per row)."""
    rows = X.reshape(-1, X.shape[-1])
    if big:
        return [sum(int(v) * int(v) for v in r) for r in rows]
    A = np.abs(rows)
    hi, lo = A >> 20, A & ((1 << 20) - 1)          # each < 2^20
    s_hh = (hi * hi).sum(axis=1)                    # < 2^49 for d <= 512
    s_hl = (hi * lo).sum(axis=1)
    s_ll = (lo * lo).sum(axis=1)
    return [(int(a) << 40) + (int(b) << 21) + int(c) for a, b, c in zip(s_hh, s_hl, s_ll)]


def _rotate_exact(X: np.ndarray, signs: np.ndarray, big: bool) -> np.ndarray:
    """Exact integers Z = H (s * X) along the last axis."""
    d = X.shape[-1]
    H = hadamard(d)
    if big:
        Xs = X * signs.astype(object)
        return Xs.dot(H.astype(object))
    # |partial sums| < d * 2^40 < 2^49: exact in float64 whatever the order.
    Z = (X.astype(np.float64) * signs.astype(np.float64)) @ H.astype(np.float64)
    return Z.astype(np.int64)


def _fp16_grid(bits: int) -> Fraction:
    return Fraction(int(np.array(bits, dtype=np.uint16).view(np.float16).astype(np.float64) * 2**24), 2**24)


def rne_fp16_sqrt(S: Fraction) -> np.uint16:
    """Bits of RNE_fp16(sqrt(S)) for an exact non-negative rational S,
    decided by comparing S with squared fp16 midpoints (IEEE overflow -> inf)."""
    if S == 0:
        return np.uint16(0)
    guess = np.float16(min(math.sqrt(float(S)), 65519.0))
    p = int(np.array(guess).view(np.uint16))
    p = max(1, min(p, 0x7BFF))

    def val(bits):  # value of a positive fp16 pattern; 0x7C00 treated as 2^16
        return Fraction(65536) if bits == 0x7C00 else _fp16_grid(bits)

    while True:
        lo_mid = (val(p - 1) + val(p)) / 2 if p > 0 else Fraction(0)
        hi_mid = (val(p) + val(p + 1)) / 2
        if p > 0 and S < lo_mid * lo_mid:
            p -= 1
            continue
        if p > 0 and S == lo_mid * lo_mid and (p & 1):
            p -= 1
            continue
        if S > hi_mid * hi_mid or (S == hi_mid * hi_mid and (p & 1)):
            if p + 1 >= 0x7C00:
                return np.uint16(0x7C00)
            p += 1
            continue
        return np.uint16(p)


# ----------------------------------------------------------------------------
# Quantize-on-append: rotation, norm split, Lloyd-Max codes
# ([AdapTQ] "The Math Fix"; [Velox] "Stage 1", "Stage 2")
# ----------------------------------------------------------------------------

WINDOW = 1e-6
_CHUNK = 4096


def fp16_norm_bits(S_list: list[int], E: int) -> np.ndarray:
    """RNE_fp16(sqrt(S)) for exact integers S (value S * 2^-2E), one per row.
    A float64 estimate decides rows far from every fp16 midpoint; the rest are
    decided exactly by rne_fp16_sqrt."""
    out = np.empty(len(S_list), dtype=np.uint16)
    for r, Sr in enumerate(S_list):
        est = math.sqrt(float(Sr)) * 2.0 ** -E
        h = np.float16(est) if est < 65504.0 else None
        if h is not None and est > 2.0 ** -14:
            p = int(np.array(h).view(np.uint16))
            lo = (float(_fp16_grid(p - 1)) + float(h)) / 2
            hi = (float(h) + (65536.0 if p + 1 == 0x7C00 else float(_fp16_grid(p + 1)))) / 2
            if min(est - lo, hi - est) > 1e-9 * est:
                out[r] = p
                continue
        out[r] = rne_fp16_sqrt(Fraction(Sr, 1 << (2 * E)))
    return out


def _nearest_mid_distance(u: np.ndarray, mids: np.ndarray) -> np.ndarray:
    k = np.searchsorted(mids, u)
    below = np.abs(u - mids[np.clip(k - 1, 0, len(mids) - 1)])
    above = np.abs(u - mids[np.clip(k, 0, len(mids) - 1)])
    return np.minimum(below, above)


def quantize_lm(x: np.ndarray, signs: np.ndarray, bits: int):
    """Quantize vectors x[..., d] (fp16 or fp32) with the rotated Lloyd-Max codec.

    Returns (codes uint8[..., d], norms_fp16_bits uint16[...], window bool[..., d]):
      z = H (s * x)                    (unnormalised rotation, exact)
      norm = RNE_fp16(||x||)           (exact decision)
      code_j = #{i : z_j >= m_i * sqrt(d) * ||x||}   (ties to the upper cell)
      a zero vector gets norm 0 and code 2^(b-1) everywhere.
    window marks coordinates whose z_j / (sqrt(d)||x||) lies within
    WINDOW / sqrt(d) of a decision midpoint (the boundary window)."""
    d = x.shape[-1]
    L = 1 << bits
    _, mids = codebook(bits, d)
    lead = x.shape[:-1]
    x2 = np.ascontiguousarray(x).reshape(-1, d)
    n = x2.shape[0]
    codes = np.empty((n, d), dtype=np.uint8)
    window = np.zeros((n, d), dtype=bool)
    norms = np.empty(n, dtype=np.uint16)
    for r0 in range(0, n, _CHUNK):
        X, E, big = _to_int_grid(x2[r0:r0 + _CHUNK])
        Z = _rotate_exact(X, signs, big)
        S = _sum_squares_exact(X, big)
        norms[r0:r0 + len(S)] = fp16_norm_bits(S, E)
        Sf = np.array([float(s) for s in S])
        Zf = np.vectorize(float, otypes=[np.float64])(Z) if big else Z.astype(np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            u = Zf / np.sqrt(d * Sf)[:, None]
        zero = Sf == 0
        u[zero] = 0.0
        code = np.searchsorted(mids, u, side="right")
        dist = _nearest_mid_distance(u, mids)
        for i, j in zip(*np.nonzero((dist <= 1e-12) & ~zero[:, None])):
            code[i, j] = sum(1 for m in mids if _z_ge_m_sqrt(int(Z[i, j]), float(m), d * S[i]))
        code[zero] = L // 2
        codes[r0:r0 + len(S)] = code
        window[r0:r0 + len(S)] = (dist * math.sqrt(d) <= WINDOW) & ~zero[:, None]
    return codes.reshape(*lead, d), norms.reshape(lead), window.reshape(*lead, d)


def _z_ge_m_sqrt(z: int, m: float, dS: int) -> bool:
    """Exact test z >= m * sqrt(dS) for integer z, dyadic m, integer dS >= 0."""
    M = Fraction(m)
    if M >= 0:
        return z >= 0 and Fraction(z) ** 2 >= M * M * dS
    if z >= 0:
        return True
    return Fraction(z) ** 2 <= M * M * dS


# ----------------------------------------------------------------------------
# fp8 E4M3 (OCP "FN" variant) keys of the far tier
# ([Foveated] "The VR headset thing": far-tier keys in fp8 E4M3)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
    is subnormal (m * 2^-9); 0x7F / 0xFF are NaN."""
    code = np.asarray(code, dtype=np.int64)
    s = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


_E4M3_POS = e4m3_decode(np.arange(0x7F))  # all finite non-negative values, ascending


def quantize_fp8(x: np.ndarray, signs: np.ndarray):
    """Far-tier key codec: y = R x, each y_j rounded to E4M3FN, nearest-even,
    saturating at +-448, no scale.  Returns (codes uint8[..., d], window).
    A coordinate rounding to zero keeps its sign (0x80 for negative y_j);
    an exactly zero y_j is +0 (0x00)."""
    d = x.shape[-1]
    lead = x.shape[:-1]
    x2 = np.ascontiguousarray(x).reshape(-1, d)
    n = x2.shape[0]
    codes = np.empty((n, d), dtype=np.uint8)
    window = np.zeros((n, d), dtype=bool)
    grid = _E4M3_POS
    mids = 0.5 * (grid[:-1] + grid[1:])
    for r0 in range(0, n, _CHUNK):
        X, E, big = _to_int_grid(x2[r0:r0 + _CHUNK])
        Z = _rotate_exact(X, signs, big)
        S = _sum_squares_exact(X, big)
        Zf = np.vectorize(float, otypes=[np.float64])(Z) if big else Z.astype(np.float64)
        y = Zf / (2.0 ** E * math.sqrt(d))
        a = np.abs(y)
        k = np.searchsorted(mids, a, side="left")
        kc = np.minimum(k, len(mids) - 1)
        tie = (k < len(mids)) & (a == mids[kc])
        k = np.where(tie & (k % 2 == 1), k + 1, k)
        dist = _nearest_mid_distance(a, mids)
        for i, j in zip(*np.nonzero(dist <= 1e-12 * np.maximum(a, 2.0 ** -9))):
            k[i, j] = _e4m3_exact_index(abs(int(Z[i, j])), E, d)
        k = np.minimum(k, 0x7E)
        codes[r0:r0 + len(S)] = (k + np.where(Zf < 0, 0x80, 0)).astype(np.uint8)
        sigma = np.sqrt(np.array([float(s) for s in S])) / 2.0 ** E / math.sqrt(d)
        window[r0:r0 + len(S)] = dist <= WINDOW * sigma[:, None]
    return codes.reshape(*lead, d), window.reshape(*lead, d)


def _e4m3_exact_index(zabs: int, E: int, d: int) -> int:
    """RNE index into the non-negative E4M3 grid of y = zabs * 2^-E / sqrt(d)."""
    y2 = Fraction(zabs * zabs, (1 << (2 * E)) * d)   # y^2, exact
    grid = [Fraction(float(g)) for g in _E4M3_POS]
    for k in range(len(grid) - 1):
        mid = (grid[k] + grid[k + 1]) / 2
        if y2 < mid * mid:
            return k
        if y2 == mid * mid:
            return k if k % 2 == 0 else k + 1
    return len(grid) - 1


# ----------------------------------------------------------------------------
# Bit packing  ([Velox] "The Bit-Packing Problem": b-bit indices packed into a
# byte stream, least significant bit first)
# ----------------------------------------------------------------------------


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Code j occupies stream bits [bits*j, bits*j + bits), LSB first; the row
    is d*bits/8 bytes."""
    codes = np.asarray(codes, dtype=np.uint8)
    d = codes.shape[-1]
    if (d * bits) % 8:
        raise ValueError("row must be whole bytes")
    bitplanes = (codes[..., None] >> np.arange(bits, dtype=np.uint8)) & 1
    stream = bitplanes.reshape(*codes.shape[:-1], d * bits)
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack(packed: np.ndarray, bits: int, d: int) -> np.ndarray:
    stream = np.unpackbits(np.asarray(packed, np.uint8), axis=-1, bitorder="little")
    stream = stream[..., : d * bits].reshape(*packed.shape[:-1], d, bits)
    return (stream.astype(np.uint8) << np.arange(bits, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)


def row_bytes(bits: int, d: int) -> int:
    return d * bits // 8


# ----------------------------------------------------------------------------
# Dequantization and attention  ([AdapTQ] "Engineering the Hot Path": rotate
# the query once, score keys from their codes; [Foveated] "Making it fast":
# query pre-scaled by 1/sqrt(D), online softmax, split-K)
# ----------------------------------------------------------------------------


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def dequantize_lm(codes: np.ndarray, norm_bits: np.ndarray, bits: int) -> np.ndarray:
    """Rotated-domain reconstruction: norm_fp16 * c[code] (exact in float64)."""
    d = codes.shape[-1]
    c, _ = codebook(bits, d)
    return fp16_bits_to_f64(norm_bits)[..., None] * c.astype(np.float64)[codes]


def attention(q: np.ndarray, k_rot: np.ndarray, v_rot: np.ndarray, signs: np.ndarray,
              lse: bool = False):
    """Decode attention over a rotated-domain cache, by definition, in float64.

    q: [B, Hq, d] (original domain); k_rot, v_rot: [B, Hkv, T, d] rotated-domain
    reconstructions.  KV head of query head h is floor(h / G).
      q~ = R q;  s_t = q~ . k_t / sqrt(d);  p = softmax(s);  o~ = sum p_t v_t;
      o = R^T o~.   Returns o [B, Hq, d] (and the log-sum-exp of s if asked)."""
    B, Hq, d = q.shape
    Hkv = k_rot.shape[1]
    G = Hq // Hkv
    qr = rotate(q, signs)
    kk = np.repeat(np.asarray(k_rot, np.float64), G, axis=1)
    vv = np.repeat(np.asarray(v_rot, np.float64), G, axis=1)
    s = np.einsum("bhd,bhtd->bht", qr, kk) / math.sqrt(d)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    o_rot = np.einsum("bht,bhtd->bhd", e / l, vv)
    o = rotate_inverse(o_rot, signs)
    if lse:
        return o, (m + np.log(l))[..., 0]
    return o


def attention_original_domain(q, k_rot, v_rot, signs):
    """Same attention computed in the original domain (keys and values mapped
    back with R^T first); agrees with attention() because R is orthonormal."""
    B, Hq, d = q.shape
    G = Hq // k_rot.shape[1]
    k = np.repeat(rotate_inverse(k_rot, signs), G, axis=1)
    v = np.repeat(rotate_inverse(v_rot, signs), G, axis=1)
    s = np.einsum("bhd,bhtd->bht", np.asarray(q, np.float64), k) / math.sqrt(d)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("bht,bhtd->bhd", p, v)


def split_bounds(T: int, S: int, align: int = 1):
    """Contiguous chunks of ceil(T/S) tokens, that size rounded up to a multiple
    of `align`; trailing chunks may be empty."""
    step = -(-T // S) if S else 0
    step = -(-step // align) * align
    return [(min(T, i * step), min(T, (i + 1) * step)) for i in range(S)]


def attention_partials(q_rot_scaled: np.ndarray, k: np.ndarray, v: np.ndarray, S: int, align: int = 1):
    """Split-K partial softmax states for one (query head, KV stream).

    q_rot_scaled: [d] query already in the domain of k and divided by sqrt(d);
    k, v: [T, d].  Returns (m [S], l [S], o [S, d]) with o the chunk's
    normalised output (sum p v / l); an empty chunk gives m=-inf, l=0, o=0."""
    T, d = k.shape
    ms, ls, os_ = [], [], []
    for a, b in split_bounds(T, S, align):
        if a == b:
            ms.append(-math.inf); ls.append(0.0); os_.append(np.zeros(d))
            continue
        s = k[a:b] @ q_rot_scaled
        m = s.max()
        e = np.exp(s - m)
        ms.append(m); ls.append(e.sum()); os_.append(e @ v[a:b] / e.sum())
    return np.array(ms), np.array(ls), np.array(os_)


def merge_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray):
    """Combine split states: M = max m_s, w_s = l_s e^(m_s - M),
    o = sum w_s o_s / sum w_s; also returns the log-sum-exp M + log sum w_s."""
    M = np.max(m)
    w = np.where(l > 0, l * np.exp(np.where(np.isfinite(m), m - M, -np.inf)), 0.0)
    W = w.sum()
    return (w[:, None] * o).sum(axis=0) / W, M + math.log(W)


def two_tier_attention(q, near_k, near_v, far_k_rot, far_v_rot, signs, lse: bool = False):
    """One softmax over both tiers ([Foveated] "The VR headset thing": every
    token still contributes; near tier exact fp16 in the original domain, far
    tier rotated).  near_k/near_v: [B, H, Tn, d] original domain;
    far_k_rot/far_v_rot: [B, H, Tf, d] rotated-domain reconstructions."""
    B, Hq, d = q.shape
    G = Hq // near_k.shape[1]
    q64 = np.asarray(q, np.float64)
    qr = rotate(q, signs)
    nk = np.repeat(np.asarray(near_k, np.float64), G, axis=1)
    nv = np.repeat(np.asarray(near_v, np.float64), G, axis=1)
    fk = np.repeat(np.asarray(far_k_rot, np.float64), G, axis=1)
    fv = np.repeat(np.asarray(far_v_rot, np.float64), G, axis=1)
    sn = np.einsum("bhd,bhtd->bht", q64, nk) / math.sqrt(d)
    sf = np.einsum("bhd,bhtd->bht", qr, fk) / math.sqrt(d)
    m = np.maximum(sn.max(axis=-1, initial=-np.inf), sf.max(axis=-1, initial=-np.inf))[..., None]
    en, ef = np.exp(sn - m), np.exp(sf - m)
    l = en.sum(axis=-1, keepdims=True) + ef.sum(axis=-1, keepdims=True)
    o = np.einsum("bht,bhtd->bhd", en, nv) + rotate_inverse(np.einsum("bht,bhtd->bhd", ef, fv), signs)
    o = o / l
    if lse:
        return o, (m + np.log(l))[..., 0]
    return o


# Score gate and spike flags ([Foveated] "Making it fast": value loading is
# skipped for a token whose score falls below exp(-16), i.e. whose weight is
# below e^-16 of the reference; a far-tier token scoring above the near tier
# is flagged for promotion).  Reading: the reference is given per (b, query
# head) in natural-log score units (a previous step's log-sum-exp, say); a
# gated token keeps its weight in the softmax sum and only its value is left
# out; flags mark far tokens whose score exceeds a given threshold.
GATE_LOG = 16.0


def far_scores(q, far_k_rot, signs):
    """s[b, h, t] = (R q_h) . khat_t / sqrt(d) for the far tier, natural-log units."""
    B, Hq, d = q.shape
    G = Hq // far_k_rot.shape[1]
    fk = np.repeat(np.asarray(far_k_rot, np.float64), G, axis=1)
    return np.einsum("bhd,bhtd->bht", rotate(q, signs), fk) / math.sqrt(d)


def gated_two_tier_attention(q, near_k, near_v, far_k_rot, far_v_rot, signs, gate_ref, lse: bool = False):
    """two_tier_attention with the score gate on the far tier: far token t's
    value is left out of head h's sum when s[b,h,t] < gate_ref[b,h] - 16,
    its weight still counting in the normaliser.  gate_ref: [B, Hq]."""
    B, Hq, d = q.shape
    G = Hq // far_k_rot.shape[1]
    sf = far_scores(q, far_k_rot, signs)
    keep = sf >= np.asarray(gate_ref, np.float64)[..., None] - GATE_LOG
    q64 = np.asarray(q, np.float64)
    nk = np.repeat(np.asarray(near_k, np.float64), G, axis=1)
    nv = np.repeat(np.asarray(near_v, np.float64), G, axis=1)
    fv = np.repeat(np.asarray(far_v_rot, np.float64), G, axis=1)
    sn = np.einsum("bhd,bhtd->bht", q64, nk) / math.sqrt(d)
    m = np.maximum(sn.max(axis=-1, initial=-np.inf), sf.max(axis=-1, initial=-np.inf))[..., None]
    en, ef = np.exp(sn - m), np.exp(sf - m)
    l = en.sum(axis=-1, keepdims=True) + ef.sum(axis=-1, keepdims=True)
    o = np.einsum("bht,bhtd->bhd", en, nv) + rotate_inverse(np.einsum("bht,bhtd->bhd", ef * keep, fv), signs)
    o = o / l
    if lse:
        return o, (m + np.log(l))[..., 0]
    return o


def spike_flags(q, far_k_rot, signs, spike_ref):
    """bool [B, Hq, Tf]: far token t of head h scores above spike_ref[b, h]."""
    return far_scores(q, far_k_rot, signs) > np.asarray(spike_ref, np.float64)[..., None]


def pack_flags(flags):
    """bool [..., T] -> uint32 [..., ceil(T/32)], token t at bit t % 32 of word t // 32."""
    T = flags.shape[-1]
    W = -(-T // 32)
    pad = np.zeros(flags.shape[:-1] + (W * 32,), dtype=np.uint64)
    pad[..., :T] = flags
    bits = pad.reshape(flags.shape[:-1] + (W, 32)) << np.arange(32, dtype=np.uint64)
    return bits.sum(axis=-1).astype(np.uint32)


# Outlier two-stream key cache ([Velox] "Outlier Two-Stream Cache"): a
# calibration over the first tokens picks, per (b, KV head), the channels of
# largest variance; those channels of every key are kept as int8 with a
# per-token scale and zeroed in the vector that goes through the rotation
# codec; a score adds the codec part and the int8 part.  Readings: 8
# channels (the page's benchmark), population variance over the calibration
# tokens with ties to the lower channel, indices ascending; scale =
# RN_fp32(max |x_o| / 127) in float32 arithmetic (fp32: the page fixes no
# precision), code = RNE(x_o / scale) clamped to +-127, zero scale -> zero
# codes.
OUTLIER_COUNT = 8


def calibrate_outliers(k_calib: np.ndarray, count: int = OUTLIER_COUNT) -> np.ndarray:
    """[B, H, N, d] calibration keys -> int64 [B, H, count]: the channels of
    largest variance over the N tokens, ascending."""
    x = np.asarray(k_calib, np.float64)
    var = x.var(axis=2)
    order = np.argsort(-var, axis=-1, kind="stable")[..., :count]
    return np.sort(order, axis=-1)


def split_outliers(x: np.ndarray, idx: np.ndarray):
    """x [B, H, T, d], idx [B, H, K] -> (x with those channels zeroed, the
    channels' values [B, H, T, K]); both in x's dtype."""
    sel = np.broadcast_to(idx[:, :, None, :], x.shape[:3] + (idx.shape[-1],))
    xo = np.take_along_axis(x, sel, axis=3)
    xi = x.copy()
    np.put_along_axis(xi, sel, np.zeros((), x.dtype), axis=3)
    return xi, xo


def quantize_outliers(xo: np.ndarray):
    """[..., K] outlier values -> (codes int8 [..., K], scale float32 [...])."""
    a = np.abs(np.asarray(xo, np.float32)).max(axis=-1)
    scale = (a / np.float32(127.0)).astype(np.float32)          # one float32 rounding
    s64 = scale.astype(np.float64)[..., None]
    x64 = np.asarray(xo, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s64 > 0, x64 / s64, 0.0)
    code = np.rint(u)
    # quotients within 1e-9 of a half-integer: decide the rounding exactly
    frac = np.abs(u - np.floor(u) - 0.5)
    for i in zip(*np.nonzero((frac < 1e-9) & (s64 > 0))):
        q = Fraction(float(x64[i])) / Fraction(float(s64[i[:-1] + (0,)]))
        fl = q.numerator // q.denominator
        r = q - fl
        code[i] = fl + (1 if (r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1)) else 0)
    return np.clip(code, -127, 127).astype(np.int8), scale


def dequantize_outliers(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return codes.astype(np.float64) * np.asarray(scale, np.float64)[..., None]


def two_stream_attention(q, k_rot, v_rot, idx, out_codes, out_scale, signs, lse: bool = False):
    """Decode attention over a two-stream key cache, by definition, float64:
    s_t = (R q) . khat_t / sqrt(d) + q[idx] . xhat_o,t / sqrt(d), with
    khat the codec reconstruction of the key whose outlier channels were
    zeroed and xhat_o the int8 reconstruction; values as in attention().
    idx [B, Hkv, K]; out_codes [B, Hkv, T, K]; out_scale [B, Hkv, T]."""
    B, Hq, d = q.shape
    Hkv = k_rot.shape[1]
    G = Hq // Hkv
    qr = rotate(q, signs)
    kk = np.repeat(np.asarray(k_rot, np.float64), G, axis=1)
    vv = np.repeat(np.asarray(v_rot, np.float64), G, axis=1)
    xo = np.repeat(dequantize_outliers(out_codes, out_scale), G, axis=1)          # [B, Hq, T, K]
    qo = np.take_along_axis(np.asarray(q, np.float64), np.repeat(idx, G, axis=1), axis=2)   # [B, Hq, K]
    s = (np.einsum("bhd,bhtd->bht", qr, kk) + np.einsum("bhk,bhtk->bht", qo, xo)) / math.sqrt(d)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    o = rotate_inverse(np.einsum("bht,bhtd->bhd", e / l, vv), signs)
    if lse:
        return o, (m + np.log(l))[..., 0]
    return o


# ----------------------------------------------------------------------------
# QJL residual sketch  ([Velox] "Stage 3: QJL Residual Correction" and "Memory
# Layout: What Actually Gets Stored"): the key codec's residual is not stored;
# its sign sketch under a random Gaussian projection S (m x d) is, one bit per
# row of S, beside the residual's fp16 norm.  A score adds an estimate of the
# query's product with the residual.
#
# Readings (the page's estimator is garbled: with the query side reduced to
# signs as printed, the expectation is a function of the angle, not of the
# product, so it could not be unbiased as the page states it is):
#   * residual in the rotated domain, r = R k - n16 * c[code] (R is orthonormal
#     and S Gaussian, so S R is again Gaussian: the same sketch law as on the
#     original-domain residual);
#   * z_i = 1 if S_i . r >= 0 else 0 (sign(0) = +1), packed LSB-first;
#   * the estimate of q~ . r is ||r||_16 * sqrt(pi/2) / m * sum_i (2 z_i - 1)
#     (S_i . q~): for jointly Gaussian (S_i . q~, S_i . r),
#     E[(S_i . q~) sign(S_i . r)] = sqrt(2/pi) (q~ . r) / ||r||, so this is the
#     estimator linear in the stored bits that is unbiased over S;
#   * m = d (the page's layout: 128 sketch bits at d = 128);
#   * sign decisions in float64; a product within QJL_WINDOW * ||S_i|| ||r|| of
#     zero is a boundary case (counted, like a code on a decision midpoint).
QJL_WINDOW = 1e-12


def qjl_residual(x: np.ndarray, signs: np.ndarray, bits: int):
    """Rotated-domain residual of the Lloyd-Max codec for keys x[..., d]:
    returns (r float64 [..., d], codes, norm bits, code window), where
    r = R x - n16 * c[code] (rotation in float64, reconstruction exact)."""
    codes, norms, window = quantize_lm(x, signs, bits)
    r = rotate(x, signs) - dequantize_lm(codes, norms, bits)
    return r, codes, norms, window


def qjl_sketch_bits(r: np.ndarray, S: np.ndarray):
    """Sign bits of S r for residuals r[..., d] and S [..., m, d] (broadcast
    over the leading axes): (bits uint8 0/1 [..., m], window bool [..., m])."""
    S64 = np.asarray(S, np.float64)
    dots = np.einsum("...md,...d->...m", S64, np.asarray(r, np.float64))
    bits = (dots >= 0.0).astype(np.uint8)
    scale = np.linalg.norm(S64, axis=-1) * np.linalg.norm(r, axis=-1)[..., None]
    window = (np.abs(dots) <= QJL_WINDOW * scale) & (scale > 0)
    return bits, window


def qjl_norm_bits(r: np.ndarray):
    """fp16 bits of ||r|| (round to nearest even from the float64 norm) and a
    flag for norms within 1e-12 (relative) of an fp16 rounding midpoint."""
    n = np.sqrt(np.einsum("...d,...d->...", np.asarray(r, np.float64), np.asarray(r, np.float64)))
    h = n.astype(np.float16)
    bits = h.view(np.uint16)
    hv = h.astype(np.float64)
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(0)).astype(np.float64)
    near = np.minimum(np.abs(n - (hv + up) / 2), np.abs(n - (hv + dn) / 2)) <= 1e-12 * n
    return bits, near & (n > 0)


def qjl_encode(x: np.ndarray, signs: np.ndarray, bits: int, S: np.ndarray):
    """Key codec plus sketch for keys x[..., d] and S [m, d]: returns a dict
    with codes, norms, the packed sketch (uint8 [..., m/8]), the sketch bits,
    the residual norm bits and the three boundary windows (code, sketch, norm)."""
    r, codes, norms, cwin = qjl_residual(x, signs, bits)
    z, zwin = qjl_sketch_bits(r, S)
    rn, rwin = qjl_norm_bits(r)
    return dict(codes=codes, norms=norms, code_window=cwin, sketch=pack(z, 1), sketch_bits=z,
                sketch_window=zwin, rnorm=rn, rnorm_window=rwin, residual=r)


def qjl_estimate(q_rot: np.ndarray, r_norm, z: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Estimate of q~ . r from the sketch: ||r|| sqrt(pi/2)/m sum_i (2 z_i - 1)
    (S_i . q~).  q_rot [..., d], r_norm [...] (a float norm), z [..., m] bits,
    S [..., m, d]; leading axes broadcast."""
    S64 = np.asarray(S, np.float64)
    m = S64.shape[-2]
    sq = np.einsum("...md,...d->...m", S64, np.asarray(q_rot, np.float64))
    pm = 2.0 * np.asarray(z, np.float64) - 1.0
    return np.asarray(r_norm, np.float64) * math.sqrt(math.pi / 2.0) / m * np.einsum("...m,...m->...", pm, sq)


def qjl_effective_keys(k_rot: np.ndarray, rnorm_bits: np.ndarray, z: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Rotated-domain keys whose plain product with q~ is the corrected score:
    khat + ||r||_16 sqrt(pi/2)/m S^T (2 z - 1)  (the estimate is linear in q~)."""
    S64 = np.asarray(S, np.float64)
    m = S64.shape[0]
    pm = 2.0 * np.asarray(z, np.float64) - 1.0
    corr = pm @ S64                                                          # [..., d]
    rn = fp16_bits_to_f64(rnorm_bits)[..., None]
    return np.asarray(k_rot, np.float64) + rn * math.sqrt(math.pi / 2.0) / m * corr


def qjl_attention(q, k_rot, v_rot, rnorm_bits, z, S, signs, lse: bool = False):
    """Decode attention with QJL-corrected scores, float64, by definition:
    s_t = (q~ . khat_t + ||r_t||_16 sqrt(pi/2)/m sum_i (2 z_ti - 1)(S_i . q~)) / sqrt(d),
    q~ = R q; softmax; values as in attention().  k_rot, v_rot [B, Hkv, T, d];
    rnorm_bits [B, Hkv, T]; z [B, Hkv, T, m]; S [m, d]."""
    B, Hq, d = q.shape
    Hkv = k_rot.shape[1]
    G = Hq // Hkv
    qr = rotate(q, signs)                                                      # [B, Hq, d]
    kk = np.repeat(np.asarray(k_rot, np.float64), G, axis=1)
    vv = np.repeat(np.asarray(v_rot, np.float64), G, axis=1)
    S64 = np.asarray(S, np.float64)
    m = S64.shape[0]
    sq = qr @ S64.T                                                            # [B, Hq, m]
    pm = 2.0 * np.repeat(np.asarray(z, np.float64), G, axis=1) - 1.0           # [B, Hq, T, m]
    rn = np.repeat(fp16_bits_to_f64(rnorm_bits), G, axis=1)                    # [B, Hq, T]
    corr = rn * math.sqrt(math.pi / 2.0) / m * np.einsum("bhtm,bhm->bht", pm, sq)
    s = (np.einsum("bhd,bhtd->bht", qr, kk) + corr) / math.sqrt(d)
    mx = s.max(axis=-1, keepdims=True)
    e = np.exp(s - mx)
    l = e.sum(axis=-1, keepdims=True)
    o = rotate_inverse(np.einsum("bht,bhtd->bhd", e / l, vv), signs)
    if lse:
        return o, (mx + np.log(l))[..., 0]
    return o
