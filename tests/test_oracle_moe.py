"""Pins for the oracle's MoE routing and expert FFN (CPU only).

TurboFieldfare article (Gemma 4 26B-A4B section, 量化和精度): 128 routed
experts, 8 chosen per token, an always-on shared expert added without a routing
weight, 8-bit router. Top-k is checked against a full stable sort; the sparse
evaluation against a dense all-experts-masked evaluation; gelu_tanh against an
independent library routine."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import (bf16_to_f32, dequantize, ffn, gelu_tanh, matmul_f64, moe_dense_masked,
                    moe_sparse, quantize_pack, route)

pytestmark = pytest.mark.cpu


def _stack(E, N, K, seed, name, scheme="aff4_g64"):
    cs, ss, bs = [], [], []
    for e in range(E):
        c, s, b = quantize_pack(synth.weights(N, K, 0.02, seed, f"{name}{e}"), scheme)
        cs.append(c), ss.append(s), bs.append(b)
    return np.stack(cs), np.stack(ss), (None if bs[0] is None else np.stack(bs))


def test_top_k_is_the_head_of_a_full_stable_sort():
    E, D = 128, 256
    rc, rs, rb = quantize_pack(synth.weights(E, D, 0.02, 0, "router"), "aff8_g64")
    x = synth.activations_bf16(6, D, 0, "rx")
    logits, ids, p, margin = route(x, rc, rs, rb, top_k=8)
    Wr = dequantize(rc, rs, rb, "aff8_g64")
    for m in range(6):
        l = (bf16_to_f32(x[m]).astype(np.float64) @ Wr.T).astype(np.float32)
        full = sorted(range(E), key=lambda e: (-l[e], e))
        assert list(ids[m]) == full[:8]
        ex = np.exp(logits[m] - logits[m].max())
        assert np.allclose(p[m], (ex / ex.sum())[ids[m]], rtol=1e-15)
        assert np.all(np.diff(p[m]) <= 0) and p[m].sum() < 1.0     # not renormalized
        assert abs((ex / ex.sum()).sum() - 1.0) < 1e-12
        assert margin[m] >= 0


def test_ties_go_to_the_lower_expert_index():
    E, D = 16, 64
    # identical router rows -> identical logits; the lowest indices must win
    W = np.tile(synth.weights(1, D, 0.02, 1, "tie"), (E, 1))
    rc, rs, rb = quantize_pack(W, "aff8_g64")
    x = synth.activations_bf16(1, D, 1, "tx")
    _, ids, p, margin = route(x, rc, rs, rb, top_k=4)
    assert list(ids[0]) == [0, 1, 2, 3] and margin[0] == 0.0
    assert np.allclose(p[0], 1.0 / E)


def test_constructed_router_forces_a_known_expert_set():
    E, D = 32, 64
    # row e of the router is a constant (e mod 7) * 2^-6 plus an exact affine grid; with
    # x = one-hot at column 0 the logit of e is its column-0 weight.
    want = [5, 12, 19, 26, 30, 1, 8, 15]
    W = np.zeros((E, D), dtype=np.float32)
    W[:, 1] = 1.0                                   # every group spans [0, 1]
    for rank, e in enumerate(want):
        W[e, 0] = np.float32(1.0 - rank / 255.0 * 16)   # distinct, descending
    rc, rs, rb = quantize_pack(W, "aff8_g64")
    x = np.zeros((1, D), dtype=np.uint16)
    x[0, 0] = 0x3F80                                # bf16 1.0
    _, ids, _, _ = route(x, rc, rs, rb, top_k=8)
    assert list(ids[0]) == want


def test_gelu_tanh_matches_library_and_special_values():
    g = np.linspace(-8, 8, 1001)
    ref = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy()
    assert np.allclose(gelu_tanh(g), ref, rtol=1e-14, atol=1e-14)
    assert gelu_tanh(0.0) == 0.0
    assert abs(gelu_tanh(10.0) - 10.0) < 1e-12 and abs(gelu_tanh(-10.0)) < 1e-12
    c = math.sqrt(2 / math.pi)
    assert abs(gelu_tanh(1.0) - 0.5 * (1 + math.tanh(c * 1.044715))) < 1e-15


def test_sparse_equals_dense_masked_with_shared_expert():
    E, D, F, Fs, M, k = 16, 128, 64, 128, 3, 4
    gate, up, down = _stack(E, F, D, 2, "g"), _stack(E, F, D, 2, "u"), _stack(E, D, F, 2, "d")
    shared = tuple(quantize_pack(synth.weights(n, kk, 0.02, 2, nm), "aff4_g64")
                   for n, kk, nm in ((Fs, D, "sg"), (Fs, D, "su"), (D, Fs, "sd")))
    rc, rs, rb = quantize_pack(synth.weights(E, D, 0.02, 2, "r"), "aff8_g64")
    x = synth.activations_bf16(M, D, 2, "x")
    _, ids, p, _ = route(x, rc, rs, rb, top_k=k)
    ys, S = moe_sparse(x, ids, p, gate, up, down, shared)
    yd = moe_dense_masked(x, ids, p, gate, up, down, shared)
    assert np.allclose(ys, yd, rtol=1e-12, atol=1e-14)
    assert np.all(S >= np.abs(ys) - 1e-12)


def test_identical_experts_scale_by_total_weight_and_shared_adds_unweighted():
    E, D, F, M = 8, 128, 64, 2
    one = [quantize_pack(synth.weights(n, kk, 0.02, 3, nm), "aff4_g64")
           for n, kk, nm in ((F, D, "g"), (F, D, "u"), (D, F, "d"))]
    stack = [tuple(np.stack([t[i]] * E) for i in range(3)) for t in one]
    x = synth.activations_bf16(M, D, 3, "x")
    ids = np.array([[1, 4, 6], [0, 2, 7]], dtype=np.int32)
    p = np.array([[0.5, 0.25, 0.125], [0.3, 0.2, 0.1]])
    y, _ = moe_sparse(x, ids, p, *stack)
    f, _, _ = ffn(x, *one, "aff4_g64")
    assert np.allclose(y, p.sum(axis=1, keepdims=True) * f, rtol=1e-13, atol=1e-15)
    # with every weight zero only the shared expert remains, equal to a plain FFN
    y0, _ = moe_sparse(x, ids, np.zeros_like(p), *stack, shared=tuple(one))
    assert np.array_equal(y0, f)


def test_ffn_h_is_bf16_of_gelu_gate_times_up():
    D, F = 128, 64
    trip = [quantize_pack(synth.weights(n, kk, 0.02, 4, nm), "aff4_g64")
            for n, kk, nm in ((F, D, "g"), (F, D, "u"), (D, F, "d"))]
    x = synth.activations_bf16(2, D, 4, "x")
    y, S, h = ffn(x, *trip, "aff4_g64")
    g = matmul_f64(x, dequantize(*trip[0], "aff4_g64"))
    u = matmul_f64(x, dequantize(*trip[1], "aff4_g64"))
    hv = bf16_to_f32(h).astype(np.float64)
    exact = gelu_tanh(g) * u
    assert np.all(np.abs(hv - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-30)
    assert np.allclose(y, matmul_f64(h, dequantize(*trip[2], "aff4_g64")), rtol=0, atol=0)


def test_moe_tolerance_scale_is_the_weighted_sum_of_each_down_product():
    """moe_sparse's S[m][n] = sum_j p[m][j] sum_f |W_down[e_j][n][f]| |h_j[f]| plus the
    shared expert's sum_f |W_sd[n][f]| |hs[f]|, recomputed here in exact rationals
    from the dequantized down matrices and the bf16 h of each (token, expert).
    Fixed ids and dyadic p; an expert id outside [0, E) adds nothing."""
    from fractions import Fraction
    E, D, F, Fs, M = 3, 64, 64, 64, 2
    gate, up, down = _stack(E, F, D, 5, "sg"), _stack(E, F, D, 5, "su"), _stack(E, D, F, 5, "sd")
    shared = tuple(quantize_pack(synth.weights(n, kk, 0.02, 5, nm), "aff4_g64")
                   for n, kk, nm in ((Fs, D, "ssg"), (Fs, D, "ssu"), (D, Fs, "ssd")))
    x = synth.activations_bf16(M, D, 5, "sx")
    ids = np.array([[2, 0, -1], [1, 2, 5]], dtype=np.int32)
    p = np.array([[0.5, 0.25, 0.125], [0.375, 0.0625, 0.5]])
    y, S = moe_sparse(x, ids, p, gate, up, down, shared)
    for m in range(M):
        terms = []                      # (weight, dequantized down matrix, h row)
        for j in range(3):
            e = int(ids[m, j])
            if not 0 <= e < E:
                continue
            g_e = (gate[0][e], gate[1][e], gate[2][e])
            u_e = (up[0][e], up[1][e], up[2][e])
            d_e = (down[0][e], down[1][e], down[2][e])
            _, _, h = ffn(x[m:m + 1], g_e, u_e, d_e, "aff4_g64")
            terms.append((Fraction(float(p[m, j])), dequantize(*d_e, "aff4_g64"), h[0]))
        _, _, hs = ffn(x[m:m + 1], *shared, "aff4_g64")
        terms.append((Fraction(1), dequantize(*shared[2], "aff4_g64"), hs[0]))
        for n in range(0, D, 7):
            exact = Fraction(0)
            for w, Wd, h in terms:
                hv = bf16_to_f32(h).astype(np.float64)
                exact += w * sum(abs(Fraction(float(Wd[n, f]))) * abs(Fraction(float(hv[f])))
                                 for f in range(Wd.shape[1]))
            assert abs(Fraction(float(S[m, n])) - exact) <= exact * Fraction(1, 10 ** 12), (m, n)
            assert S[m, n] >= abs(y[m, n])
