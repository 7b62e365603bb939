"""Oracle: group-wise quantization, packing, unpacking and dequantization.

TEST INFRASTRUCTURE (see oracle/__init__.py). Not used by the product path.

Schemes
  sym4_g128  symmetric 4-bit, 128 consecutive weights of a row per group,
             scale = absmax/7 kept in fp32, codes in [-7, 7] stored as
             two's-complement nibbles.          [airllm] §2.1 and §4.2 (group_quantize)
  aff4_g64   affine 4-bit, 64 weights per group, one bf16 scale and one bf16
             bias per group, codes in [0, 15].  [TurboFieldfare] section "量化和精度"
  aff8_g64   the same affine rule with 8-bit codes in [0, 255], one per byte
             (the router projection is 8-bit).  [TurboFieldfare] section "量化和精度"

Readings where the pages are silent (each a single line below):
  * affine rule: plain min/max, s = (max - min)/(2^b - 1), bias = min; both
    rounded to bf16, then codes computed against the stored bf16 values.
  * rounding: round half to even (torch.round in [airllm] §4.2 is half-to-even).
  * zero-range guard: scale >= 1e-8 for both schemes ([airllm] §4.2 clamps sym).
  * groups run along K inside one row of W[N][K] ([airllm] §2.1 "consecutive").
  * packing: element 2j in the low nibble of byte j, element 2j+1 in the high
    nibble ([airllm] §4.2 packs q[0::2] low and q[1::2] high).
"""
from __future__ import annotations

import numpy as np
import torch

SCHEMES = ("sym4_g128", "aff4_g64", "aff8_g64")
GROUP = {"sym4_g128": 128, "aff4_g64": 64, "aff8_g64": 64}
BITS = {"sym4_g128": 4, "aff4_g64": 4, "aff8_g64": 8}
SCALE_FLOOR = np.float32(1e-8)


# ---------------------------------------------------------------- bf16 helpers
def bf16_round(a) -> np.ndarray:
    """fp32 (or fp64) values -> bf16 bit patterns (uint16), round to nearest even.

    Uses PyTorch's CPU dtype conversion as the library primitive for the
    bf16 rounding; pinned in tests against exact rational rounding."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# ---------------------------------------------------------------- quantizers
def _groups(W: np.ndarray, g: int) -> np.ndarray:
    W = np.asarray(W)
    if W.dtype != np.float32:
        raise TypeError("weights must be fp32")
    N, K = W.shape
    if K % g != 0:
        raise ValueError(f"K={K} is not a multiple of the group size {g}")
    return W.reshape(N, K // g, g)


def quantize_sym4(W: np.ndarray):
    """Symmetric 4-bit, group 128, following [airllm] §4.2 (group_quantize, bits=4).

    Per group of 128 consecutive weights of a row:
      absmax a = max |w|               (exact)
      s = a / 7                        (fp32, correctly rounded; 7 = 2^(bits-1) - 1)
      s = max(s, 1e-8)                 (the page's clamp_min)
      q = clamp(round_half_even(w / s), -7, 7)   (fp32 division)
    Returns (q int8 [N][K], s fp32 [N][K/128])."""
    G = _groups(W, 128)
    a = np.abs(G).max(axis=2)
    s = a / np.float32(7.0)
    s = np.maximum(s, SCALE_FLOOR).astype(np.float32)
    q = np.rint(G / s[:, :, None])
    q = np.clip(q, -7, 7).astype(np.int8)
    return q.reshape(W.shape), s


def quantize_affine(W: np.ndarray, bits: int):
    """Affine b-bit, group 64, bf16 scale + bf16 bias ([TurboFieldfare] "量化和精度").

    The page fixes only the format; the rule is the plain min/max reading:
      mn, mx = min w, max w            (exact)
      s32 = max((mx - mn) / (2^b - 1), 1e-8)   (fp32 subtract, fp32 divide)
      s = bf16(s32), b = bf16(mn)      (round to nearest even)
      q = clamp(round_half_even((w - b) / s), 0, 2^b - 1)  (fp32, using the stored bf16 values)
    so that w is approximated by s*q + b.
    Returns (q uint8 [N][K], s bf16 bits [N][K/64], b bf16 bits [N][K/64])."""
    G = _groups(W, 64)
    levels = np.float32(2 ** bits - 1)
    mn = G.min(axis=2)
    mx = G.max(axis=2)
    s32 = np.maximum((mx - mn) / levels, SCALE_FLOOR).astype(np.float32)
    s_b = bf16_round(s32)
    b_b = bf16_round(mn)
    sf = bf16_to_f32(s_b)[:, :, None]
    bf = bf16_to_f32(b_b)[:, :, None]
    q = np.rint((G - bf) / sf)
    q = np.clip(q, 0, 2 ** bits - 1).astype(np.uint8)
    return q.reshape(W.shape), s_b, b_b


def quantize(W: np.ndarray, scheme: str):
    """Dispatch: returns (q, scale, bias-or-None)."""
    if scheme == "sym4_g128":
        q, s = quantize_sym4(W)
        return q, s, None
    if scheme == "aff4_g64":
        return quantize_affine(W, 4)
    if scheme == "aff8_g64":
        return quantize_affine(W, 8)
    raise ValueError(scheme)


# ---------------------------------------------------------------- packing
def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Integer codes [N][K] -> bytes.

    4-bit: byte j of a row = (code[2j] & 0xF) | (code[2j+1] & 0xF) << 4, the
    nibble of a negative code being its two's complement ([airllm] §4.2).
    8-bit: one code per byte."""
    q = np.asarray(q)
    if bits == 8:
        return q.astype(np.uint8).copy()
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed: np.ndarray, bits: int, signed: bool) -> np.ndarray:
    """Bytes -> integer codes [N][K] (int16). Inverse of pack().

    4-bit: low nibble is element 2j, high nibble element 2j+1; signed codes
    are sign-extended from the nibble (v >= 8 -> v - 16)."""
    p = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return p.astype(np.int16)
    N, H = p.shape
    out = np.empty((N, 2 * H), dtype=np.int16)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    if signed:
        out = np.where(out >= 8, out - 16, out).astype(np.int16)
    return out


def quantize_pack(W: np.ndarray, scheme: str):
    """quantize then pack: returns (codes uint8, scale, bias-or-None) in storage form."""
    q, s, b = quantize(W, scheme)
    return pack(q, BITS[scheme]), s, b


def packed_nbytes(scheme: str, N: int, K: int):
    """(codes, scale, bias) byte counts of the storage form."""
    g, bits = GROUP[scheme], BITS[scheme]
    codes = N * K * bits // 8
    if scheme == "sym4_g128":
        return codes, N * (K // g) * 4, 0
    return codes, N * (K // g) * 2, N * (K // g) * 2


# ---------------------------------------------------------------- dequant
def dequantize(codes: np.ndarray, scale: np.ndarray, bias, scheme: str) -> np.ndarray:
    """Stored form -> fp64 weights W'[N][K] (exact in fp64).

    sym:    w' = s * q                  ([airllm] §4.2: split nibbles, multiply by scale)
    affine: w' = s * q + b              ([TurboFieldfare] "量化和精度")"""
    bits, g = BITS[scheme], GROUP[scheme]
    q = unpack(codes, bits, signed=(scheme == "sym4_g128")).astype(np.float64)
    N, K = q.shape
    if scheme == "sym4_g128":
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return (q.reshape(N, K // g, g) * s[:, :, None]).reshape(N, K)
    s = bf16_to_f32(scale).astype(np.float64)
    b = bf16_to_f32(bias).astype(np.float64)
    return (q.reshape(N, K // g, g) * s[:, :, None] + b[:, :, None]).reshape(N, K)
