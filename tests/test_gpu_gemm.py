"""GPU parity for the prefill GEMM (airllm article §3.3: prefill is the
compute-dense phase): Y = X · dequant(W)^T with bf16 output, per element within
2e-3·sum|w||x| + 1e-5 of the oracle's fp64 product plus the rounding of the
bf16 result itself (2^-8 of its magnitude), on ragged small shapes, same-sign
inputs (where |y| = sum|w||x|) and sampled rows and columns of the two prefill
shapes."""
import numpy as np
import pytest
import torch

import bit_weight_only_quantize_amd as w4
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host_bits16, tolerance_ratio_bf16_out

pytestmark = pytest.mark.gpu


def _bf16_to_f64(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def _case(scheme, M, N, K, name, rows=None, cols=None, same_sign=False):
    print(f"[gemm] {name} {scheme} M={M} N={N} K={K} same_sign={same_sign}", flush=True)
    W = synth.weights(N, K, 0.02, seed=0, name=name)
    X = synth.activations_bf16(M, K, seed=0, name=name + ".X")
    if same_sign:
        # |x| and |w| + 0.01: every product is >= 0 (affine biases are then
        # positive too), so y = sum|w||x| and no cancellation hides an error
        X = X & np.uint16(0x7FFF)
        W = np.abs(W) + np.float32(0.01)
    c, s, b = oracle.quantize_pack(W, scheme)
    q = w4.quantize_pack(dev_f32(W), scheme)
    Y = _bf16_to_f64(host_bits16(w4.gemm(q, dev_bf16(X))))
    assert Y.shape == (M, N)
    worst = 0.0
    if rows is None and cols is None:
        yr, S = oracle.gemv_reference(c, s, b, scheme, X)
        worst = tolerance_ratio_bf16_out(Y, yr, S)
    if rows is not None:
        yr, S = oracle.gemv_reference(c, s, b, scheme, X[rows])
        worst = max(worst, tolerance_ratio_bf16_out(Y[rows], yr, S))
    if cols is not None:
        yr, S = oracle.gemv_reference(c, s, b, scheme, X, rows=cols)
        worst = max(worst, tolerance_ratio_bf16_out(Y[:, cols], yr, S))
    assert worst <= 1.0, f"worst error {worst:.3f} x tolerance"
    return q, X, Y


@pytest.mark.parametrize("scheme", ["sym4_g128", "aff4_g64"])
@pytest.mark.parametrize("M,N,K", [(300, 200, 512), (1, 128, 256), (17, 1, 128),
                                   (257, 129, 384), (512, 256, 1024), (65, 130, 192),
                                   (3, 40, 64), (260, 300, 320)])
def test_gemm_small_and_ragged(scheme, M, N, K):
    if K % (128 if scheme == "sym4_g128" else 64):
        pytest.skip("K not a multiple of the group")
    _case(scheme, M, N, K, f"gemm.{M}x{N}x{K}")


@pytest.mark.parametrize("scheme", ["sym4_g128", "aff4_g64"])
@pytest.mark.parametrize("M,N,K", [(300, 200, 512), (256, 256, 4096), (33, 130, 1152)])
def test_gemm_same_sign_inputs(scheme, M, N, K):
    _case(scheme, M, N, K, f"gemm.pos.{M}x{N}x{K}", same_sign=True)


def _samples(n, k, seed):
    r = np.random.default_rng(seed)
    edge = [0, 1, 127, 128, 255, 256, n - 1]
    return np.unique(np.concatenate([np.array([e for e in edge if e < n]), r.choice(n, k, replace=False)]))


@pytest.mark.parametrize("N,K,tag", [(11008, 4096, "gate_up"), (4096, 11008, "down")])
def test_gemm_prefill_shapes_sampled(N, K, tag):
    M = 2048
    _case("sym4_g128", M, N, K, f"prefill.{tag}", rows=_samples(M, 40, 1), cols=_samples(N, 40, 2))


def test_gemm_rows_agree_with_gemv_and_reject_bad_args():
    q, X, Y = _case("aff4_g64", 96, 1000, 2048, "gemm.vs.gemv")
    y1 = w4.gemv(q, dev_bf16(X[5:6])).cpu().numpy()[0]
    # both are within 2e-3*S + 1e-5 of the oracle, so they agree within twice that
    W = synth.weights(1000, 2048, 0.02, seed=0, name="gemm.vs.gemv")
    c, s, b = oracle.quantize_pack(W, "aff4_g64")
    _, S = oracle.gemv_reference(c, s, b, "aff4_g64", X[5:6])
    assert np.all(np.abs(Y[5] - y1) <= 2 * (2e-3 * S[0] + 1e-5))
    q8 = w4.quantize_pack(dev_f32(synth.weights(64, 128, 0.02, 0, "g8")), "aff8_g64")
    with pytest.raises(w4.W4Error):
        w4.gemm(q8, dev_bf16(X[:, :128].copy()))
    Y2 = w4.gemm(q, dev_bf16(X))
    assert np.array_equal(_bf16_to_f64(host_bits16(Y2)), Y)     # deterministic
