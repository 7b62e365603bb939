"""Oracle: the INT4 KV-cache codec and the two fused-dequant products over it.

TEST INFRASTRUCTURE (see oracle/__init__.py). Not used by the product path.

[Shimmy] §3.2 (TurboShimmy INT4 KV cache): each head vector of head_dim values
is quantized on its own. Its scale is max|v| / 7.5 in fp32; a value becomes the
integer round(v / scale) clamped to [-8, 7] and is stored as that integer plus
8 in a nibble, two per byte with element 2j in the low nibble; the shader turns
a nibble back into (nibble - 8) * scale while it computes attention.

Readings where the page is silent or its listing is garbled (its dequantizer
loops over 128 bytes but writes 2i and 2i+1, i.e. 256 values for a 128-wide
head; the reading is 64 bytes per 128-value vector):
  * rounding: the listing's f32::round, i.e. half away from zero (the weight
    schemes round half to even);
  * an all-zero vector gets scale 0 and every code 8 (the listing divides 0 by
    0, and its saturating float-to-int cast sends the NaN to 0);
  * the products: scores[h][t] = sum_i q[h][i] * k[g(h)][t][i] and
    out[h][i] = sum_t p[h][t] * v[g(h)][t][i], k and v the dequantized cached
    vectors and g(h) = h // (Hq // Hkv): query heads share a key/value head in
    equal consecutive groups. The 1/sqrt(head_dim) factor, masking and the
    softmax that turns scores into p are not on the page and stay with the
    caller.
"""
from __future__ import annotations

import numpy as np

KV_LEVEL = np.float32(7.5)


def _round_half_away(r: np.ndarray) -> np.ndarray:
    """Round to the nearest integer, halves away from zero (in fp64, where
    |r| + 0.5 is exact for every fp32 r)."""
    r = np.asarray(r, dtype=np.float64)
    return np.sign(r) * np.floor(np.abs(r) + 0.5)


def kv_quantize(x: np.ndarray):
    """fp32 head vectors [..., D] (D even) -> (codes uint8 [..., D/2], scale fp32 [...]).

    [Shimmy] §3.2 quantize_head_vector: scale = max|x| / 7.5 (fp32 division);
    q = clamp(round(x / scale), -8, 7) with the fp32 quotient; byte j =
    ((q[2j+1] + 8) << 4) | (q[2j] + 8). Zero vector: scale 0, q = 0."""
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("head vectors must be fp32")
    if x.shape[-1] % 2:
        raise ValueError("head_dim must be even")
    a = np.abs(x).max(axis=-1)
    s = (a / KV_LEVEL).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = (x / safe[..., None]).astype(np.float32)
    q = np.clip(_round_half_away(r), -8, 7)
    q = np.where(s[..., None] > 0, q, 0).astype(np.int16)
    u = (q + 8).astype(np.uint8)
    codes = (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
    return codes, s


def kv_unpack(codes: np.ndarray) -> np.ndarray:
    """Bytes [..., D/2] -> integers [..., D] in [-8, 7]: low nibble is element
    2j, high nibble element 2j+1, each minus 8 ([Shimmy] §3.2)."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.int16)
    out[..., 0::2] = (c & 0xF).astype(np.int16) - 8
    out[..., 1::2] = (c >> 4).astype(np.int16) - 8
    return out


def kv_dequant(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Cached vectors in fp64: (nibble - 8) * scale, exact ([Shimmy] §3.2)."""
    return kv_unpack(codes).astype(np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


def _group_of(Hq: int, Hkv: int) -> np.ndarray:
    if Hkv < 1 or Hq % Hkv:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return np.arange(Hq) // (Hq // Hkv)


def kv_scores(q: np.ndarray, codes: np.ndarray, scale: np.ndarray):
    """scores[h][t] = q[h] . k[g(h)][t] in fp64, and S[h][t] = |q[h]| . |k[g(h)][t]|
    (the tolerance's magnitude). q fp32 [Hq][D]; codes [Hkv][T][D/2]; scale
    [Hkv][T]. The dequantized cache, then one matrix product per head."""
    Kd = kv_dequant(codes, scale)                      # [Hkv][T][D]
    g = _group_of(q.shape[0], Kd.shape[0])
    q64 = np.asarray(q, dtype=np.float64)
    y = np.stack([Kd[g[h]] @ q64[h] for h in range(q64.shape[0])])
    S = np.stack([np.abs(Kd[g[h]]) @ np.abs(q64[h]) for h in range(q64.shape[0])])
    return y, S


def kv_weighted_sum(p: np.ndarray, codes: np.ndarray, scale: np.ndarray):
    """out[h][i] = sum_t p[h][t] v[g(h)][t][i] in fp64, and S[h][i] the same sum
    of magnitudes. p fp32 [Hq][T]; codes [Hkv][T][D/2]; scale [Hkv][T]."""
    Vd = kv_dequant(codes, scale)                      # [Hkv][T][D]
    g = _group_of(p.shape[0], Vd.shape[0])
    p64 = np.asarray(p, dtype=np.float64)
    y = np.stack([p64[h] @ Vd[g[h]] for h in range(p64.shape[0])])
    S = np.stack([np.abs(p64[h]) @ np.abs(Vd[g[h]]) for h in range(p64.shape[0])])
    return y, S
