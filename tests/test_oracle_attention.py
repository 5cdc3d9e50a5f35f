"""Pins for the oracle's attention, split-K merge and two-tier attention (CPU)."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O


def _rand_cache(rng, B, Hkv, T, d):
    return rng.standard_normal((B, Hkv, T, d)), rng.standard_normal((B, Hkv, T, d))


def test_identity_codec_equals_library_sdpa():
    """Without quantization (cache = R k, R v) the method is plain attention:
    compare with torch's scaled_dot_product_attention in float64, with GQA
    expressed by repeating KV heads."""
    rng = np.random.default_rng(0)
    B, Hq, Hkv, T, d = 2, 8, 2, 37, 64
    s = O.rademacher_signs(42, d)
    k, v = _rand_cache(rng, B, Hkv, T, d)
    q = rng.standard_normal((B, Hq, d))
    o = O.attention(q, O.rotate(k, s), O.rotate(v, s), s)
    G = Hq // Hkv
    tq = torch.from_numpy(q)[:, :, None, :]
    tk = torch.from_numpy(np.repeat(k, G, axis=1))
    tv = torch.from_numpy(np.repeat(v, G, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, :, 0].numpy()
    assert np.allclose(o, ref, atol=1e-12, rtol=0)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    d = 128
    s = O.rademacher_signs(42, d)
    k, v = _rand_cache(rng, 1, 1, 1, d)
    q = rng.standard_normal((1, 4, d))
    o = O.attention(q, k, v, s)
    assert np.allclose(o, O.rotate_inverse(v[:, 0, 0], s)[:, None, :].repeat(4, 1), atol=1e-13)


def test_equal_keys_give_mean_value():
    rng = np.random.default_rng(2)
    d, T = 64, 9
    s = O.rademacher_signs(42, d)
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), T, axis=2)
    v = rng.standard_normal((1, 1, T, d))
    o = O.attention(rng.standard_normal((1, 1, d)), k, v, s)
    assert np.allclose(o[0, 0], O.rotate_inverse(v[0, 0].mean(axis=0), s), atol=1e-13)


def test_rotated_and_original_domain_agree():
    rng = np.random.default_rng(3)
    d = 128
    s = O.rademacher_signs(42, d)
    k, v = _rand_cache(rng, 2, 2, 50, d)
    q = rng.standard_normal((2, 8, d))
    assert np.allclose(O.attention(q, k, v, s), O.attention_original_domain(q, k, v, s), atol=1e-12)


def test_gqa_head_map_and_mha_reduction():
    """Query head h reads KV head floor(h/G); with G=1 each head is independent."""
    rng = np.random.default_rng(4)
    d = 32
    s = O.rademacher_signs(42, d)
    k, v = _rand_cache(rng, 1, 2, 11, d)
    q = rng.standard_normal((1, 4, d))
    o = O.attention(q, k, v, s)
    for h in range(4):
        oh = O.attention(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1], s)
        assert np.allclose(o[:, h], oh[:, 0], atol=1e-14)


def test_brute_force_tiny_every_code_pattern():
    """d=8, 2-bit codes, T=2: enumerate every code pattern of one key against
    a fixed second key and compare with a scalar-loop softmax."""
    d, bits = 8, 2
    s = O.rademacher_signs(7, d)
    c, _ = O.codebook(bits, d)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, d))
    vrot = rng.standard_normal((1, 1, 2, d))
    qr = O.rotate(q, s)[0, 0]
    for pattern in itertools.product(range(4), repeat=4):
        codes = np.array(pattern * 2, dtype=np.uint8)
        k0 = 1.5 * c.astype(np.float64)[codes]
        k1 = 0.5 * c.astype(np.float64)[codes[::-1]]
        krot = np.stack([k0, k1])[None, None]
        o = O.attention(q, krot, vrot, s)[0, 0]
        sc = [sum(qr[j] * kk[j] for j in range(d)) / math.sqrt(d) for kk in (k0, k1)]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        orot = [(w[0] * vrot[0, 0, 0, j] + w[1] * vrot[0, 0, 1, j]) / (w[0] + w[1]) for j in range(d)]
        ref = [s[i] * sum(O.hadamard(d)[i, j] * orot[j] for j in range(d)) / math.sqrt(d) for i in range(d)]
        assert np.allclose(o, ref, atol=1e-14)


@pytest.mark.parametrize("S,align", [(1, 1), (2, 1), (3, 1), (7, 1), (64, 1), (100, 1), (3, 16), (7, 16), (3, 32), (7, 32)])
def test_split_merge_invariance(S, align):
    rng = np.random.default_rng(6)
    d, T = 64, 97
    k = rng.standard_normal((T, d)) * 3
    v = rng.standard_normal((T, d))
    q = rng.standard_normal(d) / math.sqrt(d)
    s = k @ q
    p = np.exp(s - s.max()); p /= p.sum()
    m, l, o = O.attention_partials(q, k, v, S, align)
    out, lse = O.merge_partials(m, l, o)
    assert np.allclose(out, p @ v, atol=1e-13)
    assert lse == pytest.approx(s.max() + math.log(np.exp(s - s.max()).sum()), abs=1e-12)
    bounds = O.split_bounds(T, S, align)
    assert all((a % align == 0 or a == T) for a, _ in bounds)
    assert bounds[0][0] == 0 and bounds[-1][1] == T
    assert all(b0 == a1 for (_, b0), (a1, _) in zip(bounds, bounds[1:]))


def test_two_tier_limits_and_permutation():
    rng = np.random.default_rng(8)
    B, H, T, d = 1, 2, 30, 64
    s = O.rademacher_signs(42, d)
    k = rng.standard_normal((B, H, T, d)).astype(np.float16).astype(np.float64)
    v = rng.standard_normal((B, H, T, d)).astype(np.float16).astype(np.float64)
    q = rng.standard_normal((B, H, d))
    empty = np.zeros((B, H, 0, d))
    plain = O.attention_original_domain(q, O.rotate(k, s), O.rotate(v, s), s)
    # all tokens near -> exact attention in the original domain
    assert np.allclose(O.two_tier_attention(q, k, v, empty, empty, s), plain, atol=1e-12)
    # no near tokens -> pure rotated far path
    assert np.allclose(O.two_tier_attention(q, empty, empty, O.rotate(k, s), O.rotate(v, s), s), plain, atol=1e-12)
    # any split of the same tokens between tiers gives the same answer
    nk, nv = k[:, :, :7], v[:, :, :7]
    fk, fv = O.rotate(k[:, :, 7:], s), O.rotate(v[:, :, 7:], s)
    both = O.two_tier_attention(q, nk, nv, fk, fv, s)
    assert np.allclose(both, plain, atol=1e-12)
    perm = rng.permutation(T - 7)
    assert np.allclose(O.two_tier_attention(q, nk[:, :, ::-1], nv[:, :, ::-1], fk[:, :, perm], fv[:, :, perm], s),
                       both, atol=1e-12)


def test_end_to_end_quality_report():
    """Sanity (not a pin): 4-bit rotated codes keep attention output close to
    unquantized attention on outlier-heavy keys."""
    rng = np.random.default_rng(9)
    d, T = 128, 512
    s = O.rademacher_signs(42, d)
    k = rng.standard_normal((1, 1, T, d)).astype(np.float16)
    k[..., :4] *= 20
    v = rng.standard_normal((1, 1, T, d)).astype(np.float16)
    q = rng.standard_normal((1, 4, d)).astype(np.float16)
    ck, nk, _ = O.quantize_lm(k, s, 4)
    cv, nv, _ = O.quantize_lm(v, s, 4)
    oq = O.attention(q, O.dequantize_lm(ck, nk, 4), O.dequantize_lm(cv, nv, 4), s)
    oe = O.attention(q, O.rotate(k.astype(np.float64), s), O.rotate(v.astype(np.float64), s), s)
    cos = np.sum(oq * oe, -1) / np.linalg.norm(oq, axis=-1) / np.linalg.norm(oe, axis=-1)
    assert np.all(cos > 0.9)


def _tiny_two_tier(seed, B=1, H=2, Tn=3, Tf=6, d=8, scale=4.0):
    rng = np.random.default_rng(seed)
    s = O.rademacher_signs(42, d)
    nk = rng.standard_normal((B, H, Tn, d)).astype(np.float16).astype(np.float64)
    nv = rng.standard_normal((B, H, Tn, d)).astype(np.float16).astype(np.float64)
    fk = rng.standard_normal((B, H, Tf, d)) * scale
    fv = rng.standard_normal((B, H, Tf, d))
    q = rng.standard_normal((B, H, d)) * scale
    return q, nk, nv, fk, fv, s


def test_score_gate_limits():
    """gate_ref = -inf gates nothing (the ungated pass); +inf gates every far
    value, which equals the ungated pass with the far values zeroed and
    leaves the log-sum-exp unchanged ([Foveated] "Making it fast")."""
    q, nk, nv, fk, fv, s = _tiny_two_tier(21)
    B, H = q.shape[:2]
    ref, ref_lse = O.two_tier_attention(q, nk, nv, fk, fv, s, lse=True)
    lo, lo_lse = O.gated_two_tier_attention(q, nk, nv, fk, fv, s, np.full((B, H), -np.inf), lse=True)
    assert np.allclose(lo, ref, atol=1e-13) and np.allclose(lo_lse, ref_lse, atol=1e-13)
    hi, hi_lse = O.gated_two_tier_attention(q, nk, nv, fk, fv, s, np.full((B, H), np.inf), lse=True)
    zero, zero_lse = O.two_tier_attention(q, nk, nv, fk, np.zeros_like(fv), s, lse=True)
    assert np.allclose(hi, zero, atol=1e-13) and np.allclose(hi_lse, ref_lse, atol=1e-13)


def test_score_gate_brute_force():
    """Tiny two-tier cases, scores spread wide: every head's output summed
    token by token in plain Python loops, the far values of tokens scoring
    below gate_ref - 16 left out of the numerator only."""
    for seed in range(6):
        q, nk, nv, fk, fv, s = _tiny_two_tier(30 + seed, scale=6.0)
        B, H, d = q.shape
        sf = O.far_scores(q, fk, s)
        gate = sf.max(axis=-1) - 3.0 + seed          # a threshold inside the score range
        gated = sf < gate[..., None] - 16.0
        assert gated.any() and (~gated).any()
        got = O.gated_two_tier_attention(q, nk, nv, fk, fv, s, gate)
        H_ = O.hadamard(d)
        for b in range(B):
            for h in range(H):
                qr = [sum(H_[i][j] * s[j] * q[b, h, j] for j in range(d)) / math.sqrt(d) for i in range(d)]
                scores, vals, near = [], [], []
                for t in range(nk.shape[2]):
                    scores.append(sum(q[b, h, j] * nk[b, h, t, j] for j in range(d)) / math.sqrt(d))
                    vals.append(list(nv[b, h, t])); near.append(True)
                for t in range(fk.shape[2]):
                    scores.append(sum(qr[j] * fk[b, h, t, j] for j in range(d)) / math.sqrt(d))
                    vals.append(list(fv[b, h, t])); near.append(False)
                m = max(scores)
                w = [math.exp(x - m) for x in scores]
                L = sum(w)
                num_near = [sum(w[i] * vals[i][j] for i in range(len(w)) if near[i]) for j in range(d)]
                num_far = [sum(w[i] * vals[i][j] for i in range(len(w))
                               if not near[i] and scores[i] >= gate[b, h] - 16.0) for j in range(d)]
                far_orig = [s[i] * sum(H_[i][j] * num_far[j] for j in range(d)) / math.sqrt(d) for i in range(d)]
                want = [(num_near[j] + far_orig[j]) / L for j in range(d)]
                assert np.allclose(got[b, h], want, atol=1e-12)


def test_spike_flags_brute_force_and_packing():
    """Flags equal a per-token comparison written out in loops; the packed
    words put token t at bit t % 32 of word t // 32; with the threshold at the
    k-th largest score exactly k - 1 tokens are flagged (distinct scores)."""
    q, nk, nv, fk, fv, s = _tiny_two_tier(50, Tf=70, scale=3.0)
    B, H, d = q.shape
    sf = O.far_scores(q, fk, s)
    ref = np.sort(sf, axis=-1)[..., -5]                    # the 5th largest
    flags = O.spike_flags(q, fk, s, ref)
    assert np.all(flags.sum(axis=-1) == 4)
    words = O.pack_flags(flags)
    assert words.shape == (B, H, 3) and words.dtype == np.uint32
    for b in range(B):
        for h in range(H):
            for t in range(fk.shape[2]):
                bit = (int(words[b, h, t // 32]) >> (t % 32)) & 1
                assert bit == int(sf[b, h, t] > ref[b, h])
    assert np.array_equal(O.pack_flags(np.array([True] + [False] * 31 + [True, True])), np.array([1, 3], np.uint32))
