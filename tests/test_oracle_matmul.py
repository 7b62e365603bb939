"""Pins for the oracle's fused-dequant product Y = X · dequant(W)^T (CPU only).

Brute force in exact rationals on 8x64 (affine) and 8x128 (sym) toys with
dyadic weights and small-integer activations, built from the integer codes and
the scales directly (not through the oracle's packing), so a wrong nibble
order, a dropped bias, a wrong sign extension or a transposed operand fails."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import (abs_matmul_f64, bf16_to_f32, dequantize, gemv_reference, matmul_f64, pack,
                    quantize_pack)

pytestmark = pytest.mark.cpu


def _bf16_bits_of_small_ints(v):
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _exact_y(q, s, b, x, g):
    N, K = q.shape
    out = []
    for n in range(N):
        acc = Fraction(0)
        for k in range(K):
            w = Fraction(float(s[n][k // g])) * int(q[n][k])
            if b is not None:
                w += Fraction(float(b[n][k // g]))
            acc += w * int(x[k])
        out.append(acc)
    return out


def test_brute_force_affine_8x64_toy_is_exact():
    rng = np.random.default_rng(11)
    q = rng.integers(0, 16, size=(8, 64))
    s_f = np.array([2.0 ** -(5 + n % 4) for n in range(8)], dtype=np.float32)[:, None]
    b_f = np.array([-(n + 1) * 2.0 ** -6 for n in range(8)], dtype=np.float32)[:, None]
    sb = (s_f.view(np.uint32) >> 16).astype(np.uint16)
    bb = (b_f.view(np.uint32) >> 16).astype(np.uint16)
    x = rng.integers(-4, 5, size=64)
    y = matmul_f64(_bf16_bits_of_small_ints(x)[None, :], dequantize(pack(q, 4), sb, bb, "aff4_g64"))[0]
    exact = _exact_y(q, s_f, b_f, x, 64)
    assert [Fraction(float(v)) for v in y] == exact


def test_brute_force_sym_8x128_toy_is_exact():
    rng = np.random.default_rng(12)
    q = rng.integers(-7, 8, size=(8, 128))
    s = np.array([2.0 ** -(3 + n) for n in range(8)], dtype=np.float32)[:, None]
    x = rng.integers(-3, 4, size=128)
    y = matmul_f64(_bf16_bits_of_small_ints(x)[None, :], dequantize(pack(q, 4), s, None, "sym4_g128"))[0]
    assert [Fraction(float(v)) for v in y] == _exact_y(q, s, None, x, 128)


@pytest.mark.parametrize("scheme", ["sym4_g128", "aff4_g64", "aff8_g64"])
def test_one_hot_activation_returns_a_dequantized_column(scheme):
    W = synth.weights(24, 256, seed=5, name="onehot" + scheme)
    c, s, b = quantize_pack(W, scheme)
    Wd = dequantize(c, s, b, scheme)
    for k in (0, 1, 63, 64, 200, 255):
        x = np.zeros((1, 256), dtype=np.float32)
        x[0, k] = 1.0
        y = matmul_f64(_bf16_bits_of_small_ints(x), Wd)[0]
        assert np.array_equal(y, Wd[:, k])


def test_all_ones_activation_gives_group_sums():
    W = synth.weights(16, 256, seed=6, name="ones")
    c, sb, bb = quantize_pack(W, "aff4_g64")
    x = _bf16_bits_of_small_ints(np.ones((1, 256)))
    y = matmul_f64(x, dequantize(c, sb, bb, "aff4_g64"))[0]
    q = np.zeros((16, 256), dtype=np.int64)
    q[:, 0::2] = c & 0xF
    q[:, 1::2] = c >> 4
    s = bf16_to_f32(sb).astype(np.float64)
    b = bf16_to_f32(bb).astype(np.float64)
    expect = (s * q.reshape(16, 4, 64).sum(axis=2) + 64 * b).sum(axis=1)
    assert np.allclose(y, expect, rtol=0, atol=1e-15)


def test_linearity_and_tolerance_scale():
    W = synth.weights(32, 512, seed=7, name="lin")
    c, s, b = quantize_pack(W, "sym4_g128")
    x = synth.activations_bf16(3, 512, seed=7, name="lin_x")
    y, S = gemv_reference(c, s, b, "sym4_g128", x)
    x2 = (x.astype(np.uint32) + (1 << 7)).astype(np.uint16)      # exponent + 1: exactly 2x (no zeros/denormals here)
    assert np.all(bf16_to_f32(x2) == 2 * bf16_to_f32(x))
    y2, S2 = gemv_reference(c, s, b, "sym4_g128", x2)
    assert np.array_equal(y2, 2 * y) and np.array_equal(S2, 2 * S)
    assert np.all(S >= np.abs(y))
    Wd = dequantize(c, s, b, "sym4_g128")
    assert np.array_equal(abs_matmul_f64(x, Wd), S)
    yr, _ = gemv_reference(c, s, b, "sym4_g128", x, rows=[3, 17])
    assert np.array_equal(yr, y[:, [3, 17]])


def _toy(scheme, seed):
    """Mixed-sign dyadic toy: integer codes, power-of-two scales, dyadic biases
    (affine), signed small-integer activations; every product and partial sum is
    exact in fp64."""
    rng = np.random.default_rng(seed)
    if scheme == "sym4_g128":
        g, K = 128, 256
        q = rng.integers(-7, 8, size=(8, K))
        s = np.array([[2.0 ** -(3 + (n + j) % 4) for j in range(K // g)] for n in range(8)], np.float32)
        return q, s, None, rng.integers(-3, 4, size=(2, K)), g
    g, K = 64, 192
    q = rng.integers(0, 16, size=(8, K))
    s = np.array([[2.0 ** -(4 + (n + j) % 3) for j in range(K // g)] for n in range(8)], np.float32)
    b = np.array([[(n - 3 - j) * 2.0 ** -5 for j in range(K // g)] for n in range(8)], np.float32)
    return q, s, b, rng.integers(-4, 5, size=(2, K)), g


@pytest.mark.parametrize("scheme", ["sym4_g128", "aff4_g64"])
def test_tolerance_scale_is_the_exact_sum_of_absolute_products(scheme):
    """S[m][n] = sum_k |w'[n][k]| |x[m][k]|, computed here in exact rationals from
    the integer codes, scales and biases. A mistaken S such as (sum|x|)(sum|w|),
    sum|w x| without the absolute values, or a transposed product fails."""
    q, s, b, x, g = _toy(scheme, 31)
    if scheme == "sym4_g128":
        codes, sc, bi = pack(q, 4), s, None
    else:
        codes = pack(q, 4)
        sc = (s.view(np.uint32) >> 16).astype(np.uint16)
        bi = (b.view(np.uint32) >> 16).astype(np.uint16)
    xb = _bf16_bits_of_small_ints(x)
    y, S = gemv_reference(codes, sc, bi, scheme, xb)
    for m in range(2):
        for n in range(8):
            exact = Fraction(0)
            for k in range(q.shape[1]):
                w = Fraction(float(s[n][k // g])) * int(q[n][k])
                if b is not None:
                    w += Fraction(float(b[n][k // g]))
                exact += abs(w) * abs(int(x[m][k]))
            assert Fraction(float(S[m, n])) == exact, (m, n)
    # the scale of a product with cancelling terms exceeds |y| strictly
    assert np.any(S > np.abs(y))
