"""Pins of the KV-cache codec oracle ([Shimmy] §3.2, TurboShimmy INT4 KV) and of its
two fused-dequant products, against what the page and arithmetic fix: exhaustive
nibble round trips, constructed vectors whose codes are known in closed form, the
half-away-from-zero ties of the listing's f32::round, the |error| <= scale/2 bound,
and exact rational sums on small cases."""
from fractions import Fraction

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.cpu


def _vec_from_ints(k, e):
    """fp32 vector k * 2^-e (exact)."""
    return (np.asarray(k, dtype=np.float64) * 2.0 ** -e).astype(np.float32)


def test_every_nibble_pair_lands_where_the_page_puts_it():
    # 256 vectors with scale 1 (element 0 is 7.5): elements 2 and 3 carry every
    # (lo, hi) pair of codes in [-8, 7]; as little-endian 32-bit words,
    # element k must sit in nibble k % 8 of word k / 8, holding k's integer + 8
    pairs = [(lo, hi) for lo in range(-8, 8) for hi in range(-8, 8)]
    x = np.zeros((256, 16), dtype=np.float32)
    x[:, 0] = 7.5
    x[:, 2:4] = np.array(pairs, dtype=np.float32)
    x[x == -8] = -7.5                                          # -7.5 rounds away to -8
    codes, s = oracle.kv_quantize(x)
    assert np.all(s == 1.0)
    words = codes.view("<u4")                                  # [256][2]
    for r, (lo, hi) in enumerate(pairs):
        got = [int((words[r, k // 8] >> (4 * (k % 8))) & 0xF) - 8 for k in range(16)]
        assert got[:4] == [7, 0, lo, hi]
    assert len(set(codes[:, 1].tolist())) == 256               # every byte value once
    assert np.array_equal(oracle.kv_unpack(codes)[:, 2:4], np.array(pairs))


def test_closed_form_codes():
    # max |v| = 7.5 * 2^-e makes scale exactly 2^-e; every k * 2^-e with |k| <= 7
    # is then code k, +7.5 rounds away to 8 and clamps to 7, -7.5 rounds to -8
    e = 5
    k = np.array(list(range(-7, 8)) + [7.5, -7.5, 0.0] * 3 + [1.0] * 104)
    x = _vec_from_ints(k, e)[None, :]
    assert x.shape == (1, 128)
    codes, s = oracle.kv_quantize(x)
    assert s.dtype == np.float32 and s[0] == np.float32(2.0 ** -e)
    q = oracle.kv_unpack(codes)[0]
    expect = np.array(list(range(-7, 8)) + [7, -8, 0] * 3 + [1] * 104)
    assert np.array_equal(q, expect)
    assert codes.shape == (1, 64)
    assert codes[0, 0] == ((-6 + 8) << 4) | (-7 + 8)       # elements 0 and 1


def test_ties_round_half_away_from_zero():
    # scale 1 (max 7.5): quotients +-0.5, +-1.5, +-2.5, +-3.5 are exact halves;
    # the listing's f32::round sends them away from zero (half-to-even would
    # give 0, 2, 2, 4 for the positive ones)
    vals = [7.5, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 3.5, -3.5, 6.5, -6.5]
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :len(vals)] = vals
    codes, s = oracle.kv_quantize(x)
    assert s[0] == np.float32(1.0)
    q = oracle.kv_unpack(codes)[0, :len(vals)]
    assert q.tolist() == [7, 1, -1, 2, -2, 3, -3, 4, -4, 7, -7]


def test_zero_vector_and_constant_vector():
    codes, s = oracle.kv_quantize(np.zeros((2, 128), dtype=np.float32))
    assert np.all(s == 0) and np.all(codes == 0x88)
    assert np.all(oracle.kv_dequant(codes, s) == 0)
    c = np.full((1, 128), -3.0, dtype=np.float32)         # |v| = max everywhere: -7.5 -> -8
    codes, s = oracle.kv_quantize(c)
    assert s[0] == np.float32(3.0 / 7.5) and np.all(oracle.kv_unpack(codes) == -8)


def test_error_bound_and_code_range_on_random_vectors():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 10, size=(64, 1))).astype(np.float32)
    codes, s = oracle.kv_quantize(x)
    q = oracle.kv_unpack(codes)
    assert q.min() >= -8 and q.max() <= 7
    err = np.abs(x.astype(np.float64) - oracle.kv_dequant(codes, s))
    # |v - s q| <= s / 2, plus the fp32 quotient's rounding (<= 8 * 2^-24 * s)
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0 ** -20))
    # the largest magnitude lands on 7 (positive) or -8 (negative): |q| reaches the top
    assert np.all(np.abs(q).max(axis=1) >= 7)
    # s = max / 7.5 rounded once in fp32
    assert np.array_equal(s, (np.abs(x).max(axis=1) / np.float32(7.5)).astype(np.float32))


def test_scores_and_weighted_sum_exact_on_small_integers():
    rng = np.random.default_rng(5)
    Hq, Hkv, T, D = 4, 2, 5, 8
    kq = rng.integers(-8, 8, size=(Hkv, T, D))
    codes = (((kq[..., 1::2] + 8) << 4) | (kq[..., 0::2] + 8)).astype(np.uint8)
    scale = np.array([[2.0 ** -(1 + (h + t) % 3) for t in range(T)] for h in range(Hkv)], dtype=np.float32)
    qi = rng.integers(-3, 4, size=(Hq, D)).astype(np.float32)
    pi = rng.integers(0, 5, size=(Hq, T)).astype(np.float32)
    y, S = oracle.kv_scores(qi, codes, scale)
    out, So = oracle.kv_weighted_sum(pi, codes, scale)
    for h in range(Hq):
        g = h // (Hq // Hkv)                                # heads 0,1 -> kv 0; 2,3 -> kv 1
        for t in range(T):
            ex = sum(Fraction(int(qi[h, i])) * Fraction(float(scale[g, t])) * int(kq[g, t, i]) for i in range(D))
            assert Fraction(float(y[h, t])) == ex
            assert S[h, t] == sum(abs(float(qi[h, i])) * float(scale[g, t]) * abs(int(kq[g, t, i])) for i in range(D))
        for i in range(D):
            ex = sum(Fraction(int(pi[h, t])) * Fraction(float(scale[g, t])) * int(kq[g, t, i]) for t in range(T))
            assert Fraction(float(out[h, i])) == ex


def test_one_hot_queries_and_weights_read_single_entries():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 6, 128)).astype(np.float32)      # Hkv=3, T=6
    codes, s = oracle.kv_quantize(x)
    Kd = oracle.kv_dequant(codes, s)
    q = np.zeros((3, 128), dtype=np.float32)
    q[:, 17] = 1
    y, _ = oracle.kv_scores(q, codes, s)
    assert np.array_equal(y, Kd[:, :, 17])
    p = np.zeros((3, 6), dtype=np.float32)
    p[:, 4] = 1
    out, _ = oracle.kv_weighted_sum(p, codes, s)
    assert np.array_equal(out, Kd[:, 4, :])


def test_rejects_bad_shapes():
    with pytest.raises(TypeError):
        oracle.kv_quantize(np.zeros((1, 128)))                  # fp64
    with pytest.raises(ValueError):
        oracle.kv_quantize(np.zeros((1, 7), dtype=np.float32))
    codes, s = oracle.kv_quantize(np.ones((2, 1, 8), dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.kv_scores(np.ones((3, 8), dtype=np.float32), codes, s)   # 3 heads over 2 kv heads
