"""Oracle: mixture-of-experts routing and the expert FFN on quantized weights.

TEST INFRASTRUCTURE (see oracle/__init__.py). Not used by the product path.

[TurboFieldfare] (Gemma 4 26B-A4B section, "量化和精度"):
  * 128 routed experts per layer; the router picks 8 per token;
  * a dense shared expert whose output is added to the routed output with no
    routing weight; shared and routed FFNs run side by side;
  * the router projection is 8-bit; no router-logit softcap.
Readings (the pages are silent):
  * top-k is decided on fp32 logits (the kernel's precision), largest first,
    ties to the lower expert index (a stable sort);
  * the weight of a selected expert is its softmax probability over all E raw
    logits; the 8 weights are not renormalized;
  * expert FFN: h = gelu_tanh(W_gate x) * (W_up x), rounded to bf16 (activations
    stay 16-bit), then W_down h; gelu in its tanh form.
"""
from __future__ import annotations

import math

import numpy as np

from .matmul import matmul_f64, abs_matmul_f64
from .quant import bf16_round, dequantize


def route(x_bf16: np.ndarray, r_codes, r_scale, r_bias, top_k: int = 8, scheme: str = "aff8_g64"):
    """Router: logits = x · dequant(W_r)^T (fp64), top-k, softmax weights.

    Returns (logits fp64 [M][E], ids int32 [M][k], p fp64 [M][k], margin fp64 [M])
    where margin = logit32[k-1] - logit32[k] after sorting (the distance of the
    decision to a tie; +inf when k == E)."""
    Wr = dequantize(r_codes, r_scale, r_bias, scheme)
    logits = matmul_f64(x_bf16, Wr)
    M, E = logits.shape
    ids = np.empty((M, top_k), dtype=np.int32)
    p = np.empty((M, top_k), dtype=np.float64)
    margin = np.empty(M, dtype=np.float64)
    for m in range(M):
        l32 = logits[m].astype(np.float32)
        order = sorted(range(E), key=lambda e: (-float(l32[e]), e))
        sel = order[:top_k]
        ids[m] = sel
        mx = logits[m].max()
        ex = np.exp(logits[m] - mx)
        prob = ex / ex.sum()
        p[m] = prob[sel]
        margin[m] = (float(l32[order[top_k - 1]]) - float(l32[order[top_k]])) if top_k < E else math.inf
    return logits, ids, p, margin


def gelu_tanh(g):
    """0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) in fp64."""
    g = np.asarray(g, dtype=np.float64)
    return 0.5 * g * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (g + 0.044715 * g ** 3)))


def ffn(x_bf16: np.ndarray, gate, up, down, scheme: str):
    """One gated FFN on quantized weights, for every row of x.

    gate/up/down are (codes, scale, bias) triples; gate, up are [F][D], down [D][F].
    Returns (y fp64 [M][D], S fp64 [M][D], h bf16 bits [M][F])."""
    Wg = dequantize(*gate, scheme)
    Wu = dequantize(*up, scheme)
    Wd = dequantize(*down, scheme)
    g = matmul_f64(x_bf16, Wg)
    u = matmul_f64(x_bf16, Wu)
    h = bf16_round(gelu_tanh(g) * u)
    y = matmul_f64(h, Wd)
    S = abs_matmul_f64(h, Wd)
    return y, S, h


def _expert(stack, e):
    codes, scale, bias = stack
    return (codes[e], scale[e], None if bias is None else bias[e])


def moe_sparse(x_bf16, ids, p, gate_stack, up_stack, down_stack, shared=None,
               scheme: str = "aff4_g64"):
    """y[m] = sum_j p[m][j] * FFN_{ids[m][j]}(x[m]) + FFN_shared(x[m]), evaluating only
    the selected experts (each selected expert once, for all of its (token, slot)
    pairs; ids outside [0, E) contribute nothing). Returns (y fp64 [M][D], S fp64 [M][D])."""
    x_bf16 = np.atleast_2d(x_bf16)
    M = x_bf16.shape[0]
    E = gate_stack[0].shape[0]
    D = gate_stack[0].shape[2] * (2 if scheme != "aff8_g64" else 1)
    y = np.zeros((M, D), dtype=np.float64)
    S = np.zeros((M, D), dtype=np.float64)
    for e in sorted({int(v) for v in np.asarray(ids).ravel() if 0 <= int(v) < E}):
        sel = [(m, j) for m in range(M) for j in range(ids.shape[1]) if int(ids[m, j]) == e]
        rows = x_bf16[[m for m, _ in sel]]
        ye, Se, _ = ffn(rows, _expert(gate_stack, e), _expert(up_stack, e),
                        _expert(down_stack, e), scheme)
        for r, (m, j) in enumerate(sel):
            y[m] += p[m, j] * ye[r]
            S[m] += p[m, j] * Se[r]
    if shared is not None:
        ys, Ss, _ = ffn(x_bf16, shared[0], shared[1], shared[2], scheme)
        y += ys
        S += Ss
    return y, S


def moe_dense_masked(x_bf16, ids, p, gate_stack, up_stack, down_stack, shared=None,
                     scheme: str = "aff4_g64"):
    """The same layer written densely: every expert is evaluated and weighted by
    p (zero outside the token's selected set). Used to pin moe_sparse."""
    x_bf16 = np.atleast_2d(x_bf16)
    M = x_bf16.shape[0]
    E = gate_stack[0].shape[0]
    w = np.zeros((M, E), dtype=np.float64)
    for m in range(M):
        for j in range(ids.shape[1]):
            w[m, int(ids[m, j])] += p[m, j]
    outs = [ffn(x_bf16, _expert(gate_stack, e), _expert(up_stack, e),
                _expert(down_stack, e), scheme)[0] for e in range(E)]
    y = sum(w[:, e:e + 1] * outs[e] for e in range(E))
    if shared is not None:
        y = y + ffn(x_bf16, shared[0], shared[1], shared[2], scheme)[0]
    return y
