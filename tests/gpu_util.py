"""Helpers for the GPU parity tests: host<->device moves and the tolerance check.

Inputs come from `synth` (seeded, host-generated) and expected values from `oracle`;
nothing here computes the method's arithmetic."""
import numpy as np
import torch

import bit_weight_only_quantize_amd as w4

TOL_REL = 2e-3   # |y_gpu - y_ref| <= 2e-3 * sum|w||x| + 1e-5
TOL_ABS = 1e-5


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def upload(codes, scale, bias, scheme, num_experts=1) -> w4.QuantizedMatrix:
    """Oracle-side storage arrays -> device QuantizedMatrix (inputs, not results)."""
    c = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    if scheme == "sym4_g128":
        s = torch.from_numpy(np.ascontiguousarray(scale, dtype=np.float32)).cuda()
        b = None
    else:
        s = dev_bf16(scale)
        b = dev_bf16(bias)
    N = c.shape[-2]
    K = c.shape[-1] * (1 if scheme == "aff8_g64" else 2)
    return w4.QuantizedMatrix(scheme, N, K, c, s, b, num_experts)


def tolerance_ratio(y_gpu: np.ndarray, y_ref: np.ndarray, S: np.ndarray) -> float:
    """max over elements of |err| / (2e-3 S + 1e-5); <= 1 passes."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    return float((err / (TOL_REL * S + TOL_ABS)).max()) if err.size else 0.0


U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits, round to nearest even)


def tolerance_ratio_bf16_out(y_gpu: np.ndarray, y_ref: np.ndarray, S: np.ndarray) -> float:
    """The same check for a result stored as bf16. Rounding the result y^ to bf16
    moves it by at most U_BF16 |y^|, and |y^| <= |y| + e with e within the fp32
    bound, so |bf16(y^) - y| <= (1 + U_BF16)(2e-3 S + 1e-5) + U_BF16 |y|; <= 1 passes."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = (1 + U_BF16) * (TOL_REL * S + TOL_ABS) + U_BF16 * np.abs(y_ref)
    return float((err / bound).max()) if err.size else 0.0
