"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module holds no quantization, packing or matrix-product arithmetic: it only
draws numbers. Weights are fp32 N(0, std^2); activations are N(0, 1) rounded to
bf16 (round-to-nearest-even) and returned as raw bf16 bit patterns (uint16), which
is the form both the oracle and the device path consume.

Every tensor is identified by (seed, name). The name is hashed (CRC-32) into a
stream id so that tensors drawn in any order are reproducible on any host with
the same numpy version.
"""
from __future__ import annotations

import zlib

import numpy as np

__all__ = ["stream_id", "normal_f32", "weights", "activations_bf16",
           "bf16_bits_from_f32", "device_weights"]


def stream_id(name: str) -> int:
    return zlib.crc32(name.encode("utf-8")) & 0xFFFFFFFF


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed) & 0xFFFFFFFF, stream_id(name)])


def normal_f32(shape, std: float = 1.0, seed: int = 0, name: str = "") -> np.ndarray:
    """fp32 array of N(0, std^2) draws (std applied in fp32)."""
    a = _rng(seed, name).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def weights(N: int, K: int, std: float = 0.02, seed: int = 0, name: str = "W") -> np.ndarray:
    """Weight matrix W[N][K] (out x in), fp32, N(0, std^2)."""
    return normal_f32((N, K), std, seed, name)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bit patterns.

    Input preparation only (activations are defined as bf16 values)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def activations_bf16(M: int, K: int, seed: int = 0, name: str = "x") -> np.ndarray:
    """Activations X[M][K] ~ N(0, 1) as bf16 bit patterns (uint16)."""
    return bf16_bits_from_f32(normal_f32((M, K), 1.0, seed, name))


def device_weights(N: int, K: int, std: float, seed: int, name: str, device):
    """Seeded fp32 N(0, std^2) weights drawn directly on a torch device.

    Used where host generation would dominate run time (multi-gigabyte layer
    stacks). Values differ from `weights()` for the same (seed, name)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(((int(seed) & 0xFFFFFFFF) << 32) | stream_id(name))
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    return w.mul_(std)
