"""Pins for the oracle's quantizers (CPU only).

sym4_g128: airllm article §4.2 group_quantize (bits=4, group 128): s = absmax/7,
clamp_min(1e-8), round, clamp to ±7.  aff4_g64 / aff8_g64: TurboFieldfare
article, section 量化和精度 (affine, 64-weight groups, bf16 scale + bf16 bias),
with the min/max rule as the stated reading."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import (bf16_round, bf16_to_f32, dequantize, packed_nbytes, quantize,
                    quantize_affine, quantize_pack, quantize_sym4)

pytestmark = pytest.mark.cpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_arithmetic.json")


# ------------------------------------------------------------------ bf16 rounding
def _bf16_exact(x: float) -> Fraction:
    """Round-to-nearest-even onto bf16 (8 significant bits), in exact rationals."""
    f = Fraction(x)
    if f == 0:
        return f
    sign = -1 if f < 0 else 1
    a = abs(f)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128            # 8 significant bits -> integer part of scaled
    lo = scaled.numerator // scaled.denominator
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * Fraction(lo, 128) * Fraction(2) ** e


def test_bf16_round_matches_exact_round_half_even():
    vals = [1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 1.0 - 2 ** -10, 3.14159274,
            -2.71828174, 1e-8, 6.5e-3, -0.0421, 0.0999, 255.5, 1.0 + 2 ** -8 + 2 ** -20]
    rng = np.random.default_rng(3)
    vals += list(rng.standard_normal(200).astype(np.float32) * 0.05)
    a = np.array(vals, dtype=np.float32)
    got = bf16_to_f32(bf16_round(a))
    for x, g in zip(a, got):
        assert Fraction(float(g)) == _bf16_exact(float(x)), (x, g)


# ------------------------------------------------------------------ sym4_g128
def test_sym_closed_form_dyadic_group_recovers_codes_and_scale():
    rng = np.random.default_rng(0)
    N, K = 6, 512
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    q[:, ::128] = 7          # every group holds its absmax 7 ...
    q[:, 5::128] = -7        # ... and -7
    e = np.array([3, 5, 7, 9, 11, 13])[:, None]
    W = (q.astype(np.float64) * 2.0 ** (-e)).astype(np.float32)
    qq, s = quantize_sym4(W)
    assert np.array_equal(qq, q)
    assert np.array_equal(s, np.repeat(2.0 ** (-e), 4, axis=1).astype(np.float32))


def test_sym_round_trip_error_within_half_scale():
    W = synth.weights(64, 1024, 0.02, seed=1, name="symrt")
    q, s = quantize_sym4(W)
    err = np.abs(W.astype(np.float64) - (q.astype(np.float64).reshape(64, 8, 128) * s[:, :, None]).reshape(64, 1024))
    bound = (s.astype(np.float64) * (0.5 + 2.0 ** -21))
    assert np.all(err.reshape(64, 8, 128) <= bound[:, :, None])
    assert q.min() >= -7 and q.max() <= 7          # nibble 0x8 (-8) never produced
    assert np.all(np.abs(q).reshape(64, 8, 128).max(axis=2) == 7)


def test_sym_negation_symmetry_and_zero_group():
    W = synth.weights(8, 256, 0.02, seed=2, name="symneg")
    q, s = quantize_sym4(W)
    qn, sn = quantize_sym4(-W)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    Z = np.zeros((2, 128), dtype=np.float32)
    qz, sz = quantize_sym4(Z)
    assert np.all(qz == 0) and np.all(sz == np.float32(1e-8))


def test_sym_ties_round_half_to_even():
    # absmax 7 -> s = 1 exactly; w = 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 0.5 -> 0
    g = np.zeros(128, dtype=np.float32)
    g[:6] = [7.0, 2.5, 3.5, -2.5, 0.5, -1.5]
    q, s = quantize_sym4(g.reshape(1, 128))
    assert s[0, 0] == 1.0
    assert list(q[0, :6]) == [7, 2, 4, -2, 0, -2]


# ------------------------------------------------------------------ affine
@pytest.mark.parametrize("bits", [4, 8])
def test_affine_closed_form_dyadic_group_recovers_codes(bits):
    rng = np.random.default_rng(bits)
    levels = 2 ** bits - 1
    N = 5
    q = rng.integers(0, levels + 1, size=(N, 256)).astype(np.int64)
    q[:, ::64] = 0
    q[:, 1::64] = levels
    s = np.array([2.0 ** -7, 2.0 ** -9, 3 * 2.0 ** -10, 2.0 ** -6, 5 * 2.0 ** -12])[:, None]
    b = np.array([-0.0625, -0.03125, 0.0078125, -1.5, -0.01171875])[:, None]
    W = (q * s + b).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), q * s + b)        # the construction is exact
    qq, sb, bb = quantize_affine(W, bits)
    assert np.array_equal(qq.astype(np.int64), q)
    assert np.array_equal(bf16_to_f32(sb).astype(np.float64), np.repeat(s, 4, axis=1))
    assert np.array_equal(bf16_to_f32(bb).astype(np.float64), np.repeat(b, 4, axis=1))


@pytest.mark.parametrize("bits", [4, 8])
def test_affine_round_trip_error_bound(bits):
    W = synth.weights(64, 1024, 0.02, seed=3, name=f"affrt{bits}")
    q, sb, bb = quantize_affine(W, bits)
    s = bf16_to_f32(sb).astype(np.float64)[:, :, None]
    b = bf16_to_f32(bb).astype(np.float64)[:, :, None]
    G = W.astype(np.float64).reshape(64, 16, 64)
    Q = q.astype(np.float64).reshape(64, 16, 64)
    levels = 2 ** bits - 1
    inside = (G >= b - s / 2) & (G <= b + (levels + 0.5) * s)
    err = np.abs(G - (Q * s + b))
    # inside the coded range: round-to-nearest error, plus the fp32 subtract/divide slack
    assert np.all(err[inside] <= (s * (0.5 + 2.0 ** -19) * np.ones_like(G))[inside])
    # outside it (bf16 rounding of scale/bias can leave the group max past the top
    # code): the code is the clamp boundary
    assert np.all(Q[~inside & (G > b)] == levels) and np.all(Q[~inside & (G < b)] == 0)
    if bits == 4:
        assert inside.all()    # 15 levels: bf16 rounding never leaves the range on N(0, 0.02)
    assert q.min() == 0 and q.max() == levels


def test_affine_zero_range_group_uses_floor_scale():
    W = np.full((1, 64), 0.25, dtype=np.float32)
    q, sb, bb = quantize_affine(W, 4)
    assert bf16_to_f32(bb)[0, 0] == 0.25 and np.all(q == 0)
    assert bf16_to_f32(sb)[0, 0] == bf16_to_f32(bf16_round(np.float32([1e-8])))[0]


def test_group_must_divide_k():
    W = np.zeros((2, 96), dtype=np.float32)
    with pytest.raises(ValueError):
        quantize(W, "sym4_g128")
    with pytest.raises(ValueError):
        quantize(np.zeros((2, 100), np.float32), "aff4_g64")


# ------------------------------------------------------------------ storage accounting
def test_bytes_per_weight_matches_printed_figures():
    gold = json.load(open(GOLDEN))
    ent = gold["int4_plus_f32_scale_per_128_bytes_per_element"]
    c, s, b = packed_nbytes("sym4_g128", 4096, 4096)
    per = (c + s + b) / (4096 * 4096)
    assert per == ent["exact"]
    assert round(per, 2) == ent["printed"]
    c, s, b = packed_nbytes("aff4_g64", 4096, 4096)
    assert (c + s + b) / (4096 * 4096) == 0.5625       # 4 bits + 32 bits per 64 weights
    c, s, b = packed_nbytes("aff8_g64", 128, 2048)
    assert (c + s + b) == 128 * 2048 + 2 * 2 * 128 * 32


def test_selected_expert_fraction_matches_printed_figure():
    gold = json.load(open(GOLDEN))["selected_expert_bytes"]
    mb = gold["experts_total_GB"] * 1000 * gold["selected"] / gold["experts"]
    assert abs(mb - gold["printed_selected_MB"]) / gold["printed_selected_MB"] < 0.05
    t = json.load(open(GOLDEN))["decode_step_breakdown_ms"]
    assert abs(sum(t["rows"].values()) - t["printed_total"]) < 1e-9


def test_storage_form_shapes_and_dtypes():
    W = synth.weights(16, 256, seed=4, name="shapes")
    c, s, b = quantize_pack(W, "sym4_g128")
    assert c.shape == (16, 128) and c.dtype == np.uint8 and s.shape == (16, 2) and s.dtype == np.float32 and b is None
    c, s, b = quantize_pack(W, "aff4_g64")
    assert c.shape == (16, 128) and s.shape == (16, 4) and s.dtype == np.uint16 and b.shape == (16, 4)
    c, s, b = quantize_pack(W, "aff8_g64")
    assert c.shape == (16, 256) and s.shape == (16, 4)
    for scheme in ("sym4_g128", "aff4_g64", "aff8_g64"):
        c, s, b = quantize_pack(W, scheme)
        assert dequantize(c, s, b, scheme).shape == (16, 256)
