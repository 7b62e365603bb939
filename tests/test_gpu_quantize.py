"""GPU parity: quantize_pack must reproduce the oracle's codes, scales and biases
bit for bit (airllm article §4.2 for sym4_g128; TurboFieldfare article, 量化和精度,
for the affine schemes)."""
import numpy as np
import pytest
import torch

import bit_weight_only_quantize_amd as w4
import oracle
import synth
from gpu_util import dev_f32, host_bits16

pytestmark = pytest.mark.gpu


def _check(W, scheme, tag):
    print(f"[quantize] {tag} scheme={scheme} shape={W.shape}", flush=True)
    c, s, b = oracle.quantize_pack(W, scheme)
    q = w4.quantize_pack(dev_f32(W), scheme)
    torch.cuda.synchronize()
    assert np.array_equal(q.codes.cpu().numpy(), c), "codes differ"
    if scheme == "sym4_g128":
        assert np.array_equal(q.scale.cpu().numpy().view(np.uint32), s.view(np.uint32)), "scales differ"
        assert q.bias is None
    else:
        assert np.array_equal(host_bits16(q.scale), s), "scales differ"
        assert np.array_equal(host_bits16(q.bias), b), "biases differ"


@pytest.mark.parametrize("scheme,N,K,name", [
    ("aff4_g64", 1024, 1024, "gemv1024"),          # single-GEMV workload
    ("sym4_g128", 4096, 4096, "llama7b.wq"),
    ("sym4_g128", 11008, 4096, "llama7b.gate"),
    ("sym4_g128", 4096, 11008, "llama7b.down"),
    ("aff8_g64", 128, 2048, "moe.router"),
    ("aff4_g64", 768, 2048, "moe.gate"),
    ("aff4_g64", 2048, 768, "moe.down"),
    ("aff4_g64", 13824, 5120, "llama13b.gate"),
    ("sym4_g128", 1000, 384, "ragged"),
    ("aff4_g64", 3, 192, "ragged_k"),            # K % 128 != 0
    ("aff8_g64", 5, 64, "tiny"),
    ("sym4_g128", 1, 128, "one_row"),
])
def test_quantize_pack_bit_exact(scheme, N, K, name):
    _check(synth.weights(N, K, 0.02, seed=0, name=name), scheme, name)


@pytest.mark.parametrize("scheme", oracle.SCHEMES)
def test_quantize_pack_special_values(scheme):
    rng = np.random.default_rng(5)
    W = synth.weights(8, 256, 0.02, seed=1, name="special")
    W[0] = 0.0                                        # all-zero row: floor scale
    W[1] = 0.3                                        # constant row
    W[2] = rng.integers(-14, 15, 256) * 0.5           # exact halves: ties
    W[2, ::64] = 7.0
    W[3] = np.float32(1e-30) * rng.standard_normal(256)   # tiny magnitudes
    W[4, :128] = 1e4
    W[4, 128:] = -1e-4
    W[5] = -W[5]
    _check(W.astype(np.float32), scheme, "special")


def test_quantize_pack_is_deterministic():
    W = dev_f32(synth.weights(512, 4096, 0.02, seed=2, name="det"))
    a = w4.quantize_pack(W, "aff4_g64")
    b = w4.quantize_pack(W, "aff4_g64")
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scale.view(torch.int16), b.scale.view(torch.int16))
