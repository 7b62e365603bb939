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
    nibble ([airllm] §4.2 puts the even-indexed code of a pair low).
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
def _check(W: np.ndarray, g: int) -> np.ndarray:
    W = np.asarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise TypeError("weights must be a 2-D fp32 array")
    if W.shape[1] % g != 0:
        raise ValueError(f"K={W.shape[1]} is not a multiple of the group size {g}")
    return W


def quantize_sym4(W: np.ndarray):
    """Symmetric 4-bit codes with one fp32 scale per 128 consecutive weights of a
    row ([airllm] §2.1 group size, §4.2 symmetric rule with bits = 4).

    The rule, applied to each group on its own (every row at once):
      the scale is the group's largest magnitude divided by 7 (the largest
      positive 4-bit code), in fp32 with correct rounding, and never below
      1e-8 (the page's floor, which keeps an all-zero group finite);
      a weight's code is its quotient by that scale (fp32 division), rounded
      to the nearest integer with halves to even, then limited to [-7, 7].
    Returns (q int8 [N][K], s fp32 [N][K/128])."""
    W = _check(W, 128)
    N, K = W.shape
    q = np.empty((N, K), dtype=np.int8)
    s = np.empty((N, K // 128), dtype=np.float32)
    for j in range(K // 128):
        cols = slice(128 * j, 128 * (j + 1))
        grp = W[:, cols]                                    # group j of every row
        peak = np.max(np.abs(grp), axis=1)                  # exact in fp32
        sj = np.maximum(peak / np.float32(7.0), SCALE_FLOOR).astype(np.float32)
        codes = np.rint(grp / sj[:, None])                  # fp32 quotient, halves to even
        q[:, cols] = np.clip(codes, -7, 7)
        s[:, j] = sj
    return q, s


def quantize_affine(W: np.ndarray, bits: int):
    """Affine b-bit codes with one bf16 scale and one bf16 bias per 64 weights of a
    row ([TurboFieldfare] "量化和精度": 4-bit, group 64, bf16 scale + bf16 bias;
    the router uses 8 bits).

    The page fixes only the format; the rule is the plain min/max reading, per group:
      the scale spans the group's range over the 2^b - 1 code steps
      ((max - min) / (2^b - 1) in fp32, floored at 1e-8) and the bias is the
      group minimum; both are stored as bf16 (nearest, ties to even);
      a weight's code is (w - bias) / scale computed in fp32 from the STORED
      bf16 values, rounded half to even and limited to [0, 2^b - 1],
    so that a weight reads back as scale * code + bias.
    Returns (q uint8 [N][K], s bf16 bits [N][K/64], b bf16 bits [N][K/64])."""
    W = _check(W, 64)
    N, K = W.shape
    top = np.float32(2 ** bits - 1)
    q = np.empty((N, K), dtype=np.uint8)
    s_b = np.empty((N, K // 64), dtype=np.uint16)
    b_b = np.empty((N, K // 64), dtype=np.uint16)
    for j in range(K // 64):
        cols = slice(64 * j, 64 * (j + 1))
        grp = W[:, cols]
        lo, hi = grp.min(axis=1), grp.max(axis=1)
        step = np.maximum((hi - lo) / top, SCALE_FLOOR).astype(np.float32)
        s_b[:, j] = bf16_round(step)
        b_b[:, j] = bf16_round(lo)
        sf = bf16_to_f32(s_b[:, j])[:, None]
        bf = bf16_to_f32(b_b[:, j])[:, None]
        q[:, cols] = np.clip(np.rint((grp - bf) / sf), 0, 2 ** bits - 1)
    return q, s_b, b_b


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

    4-bit: two codes share a byte; of the pair (element 2j, element 2j + 1) the
    first goes to the low nibble and the second to the high nibble, a negative
    code being stored as its 4-bit two's complement ([airllm] §4.2).
    8-bit: one code per byte."""
    q = np.asarray(q)
    if bits == 8:
        return q.astype(np.uint8).copy()
    N, K = q.shape
    pairs = (q.astype(np.int16) & 0xF).astype(np.uint8).reshape(N, K // 2, 2)
    first, second = pairs[:, :, 0], pairs[:, :, 1]
    return (first | (second << 4)).astype(np.uint8)


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
