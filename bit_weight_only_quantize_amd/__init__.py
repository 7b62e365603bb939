"""Python binding for libw4a16.so: group-wise 4-bit weight-only quantization with
the dequantization fused into the matrix products, for AMD MI355X (gfx950).

This module only marshals arguments: every step runs in the HIP library's
kernels. PyTorch supplies device memory and the current stream. There is no
CPU fallback: if the library is missing or fails to load, every call raises.

Schemes (see include/w4a16.h):
  "sym4_g128"  symmetric 4-bit, 128 weights/group, fp32 scale = absmax/7
               (airllm article §2.1, §4.2)
  "aff4_g64"   affine 4-bit, 64 weights/group, bf16 scale + bf16 bias
               (TurboFieldfare article, section 量化和精度)
  "aff8_g64"   the same affine format with 8-bit codes (the router)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "SCHEME_IDS", "W4Error", "QuantizedMatrix", "lib", "lib_path", "packed_sizes", "quantize_pack",
    "empty_quantized", "gemv", "gemv_into", "gemv_multi", "gemv_multi_into", "gemm", "moe_route", "moe_workspace_bytes", "moe_gemv",
]

SCHEME_IDS = {"sym4_g128": 0, "aff4_g64": 1, "aff8_g64": 2}
_ERRORS = {-1: "W4_EINVAL", -2: "W4_ESHAPE", -3: "W4_EALIGN", -4: "W4_EHIP", -5: "W4_EWORKSPACE"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libw4a16.so")
_lib: Optional[ctypes.CDLL] = None


class W4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERRORS.get(code, code)}: {msg}")
        self.code = code


class _W4Matrix(ctypes.Structure):
    _fields_ = [("scheme", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "w4_last_error": ([], ctypes.c_char_p),
    "w4_packed_sizes": ([ctypes.c_int, _I64, _I64, ctypes.POINTER(ctypes.c_size_t),
                         ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "w4_quantize_pack": ([ctypes.c_int, _P, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "w4a16_gemv": ([ctypes.POINTER(_W4Matrix), _P, _I64, _P, _P], ctypes.c_int),
    "w4a16_gemm": ([ctypes.POINTER(_W4Matrix), _P, _I64, _P, _P], ctypes.c_int),
    "w4_gemv_workspace_bytes": ([ctypes.POINTER(_W4Matrix), _I64], ctypes.c_size_t),
    "w4_kv_quantize": ([_P, _I64, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "w4_kv_append": ([_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P], ctypes.c_int),
    "w4_kv_scores": ([_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "w4_kv_scores_append": ([_P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "w4_kv_weighted_sum_workspace_bytes": ([_I64, _I64], ctypes.c_size_t),
    "w4_kv_weighted_sum_append": ([_P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t,
                                   _P], ctypes.c_int),
    "w4_kv_weighted_sum": ([_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P],
                           ctypes.c_int),
    "w4a16_gemv_ws": ([ctypes.POINTER(_W4Matrix), _P, _I64, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "w4a16_gemv_multi": ([ctypes.POINTER(ctypes.POINTER(_W4Matrix)), ctypes.c_int, _P, _I64,
                          ctypes.POINTER(ctypes.c_void_p), _P], ctypes.c_int),
    "w4_moe_route": ([ctypes.POINTER(_W4Matrix), _P, _I64, ctypes.c_int, _P, _P, _P, _P], ctypes.c_int),
    "w4_moe_workspace_bytes": ([_I64, ctypes.c_int, _I64, _I64, _I64, _I64], ctypes.c_size_t),
    "w4a16_moe_gemv": ([ctypes.POINTER(_W4Matrix)] * 6 + [_P, _I64, _P, _P, ctypes.c_int, _P,
                                                          ctypes.c_size_t, _P, _P], ctypes.c_int),
    "w4_moe_layer_workspace_bytes": ([_I64, ctypes.c_int, _I64, _I64, _I64, _I64], ctypes.c_size_t),
    "w4a16_moe_layer": ([ctypes.POINTER(_W4Matrix)] * 7 + [_P, _I64, ctypes.c_int, _P, _P, _P, _P,
                                                           ctypes.c_size_t, _P], ctypes.c_int),
    "w4_moe_layer_status": ([_P, ctypes.POINTER(ctypes.c_int32), _P], ctypes.c_int),
    "w4_moe_layer_set_wait": ([_I64, ctypes.c_int], None),
    "w4_moe_layer_set_single_launch": ([ctypes.c_int], None),
    "w4a16_moe_gemv_noalloc": ([ctypes.POINTER(_W4Matrix)] * 6 + [_P, _I64, _P, _P, ctypes.c_int, _P, _P],
                               ctypes.c_int),
    "w4_ffn_workspace_bytes": ([ctypes.POINTER(_W4Matrix), _I64], ctypes.c_size_t),
    "w4a16_ffn": ([ctypes.POINTER(_W4Matrix)] * 3 + [_P, _I64, _P, _P, _P, ctypes.c_size_t, _P],
                  ctypes.c_int),
    "w4_ffn_gate_up_workspace_bytes": ([ctypes.POINTER(_W4Matrix), _I64], ctypes.c_size_t),
    "w4a16_ffn_gate_up": ([ctypes.POINTER(_W4Matrix)] * 2 + [_P, _I64, _P, _P, ctypes.c_size_t, _P],
                          ctypes.c_int),
    "w4_ffn_status": ([_P, ctypes.POINTER(ctypes.c_int32), _P], ctypes.c_int),
    "w4_ffn_set_wait": ([_I64, ctypes.c_int], None),
    "w4_ffn_set_path": ([ctypes.c_int], ctypes.c_int),
    "w4a16_moe_gemv_logits": ([ctypes.POINTER(_W4Matrix)] * 6 + [_P, _I64, _P, ctypes.c_int, _P, _P,
                                                                 _P, ctypes.c_size_t, _P, _P],
                              ctypes.c_int),
}


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libw4a16.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise W4Error(rc, lib().w4_last_error().decode(errors="replace"))


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def packed_sizes(scheme: str, N: int, K: int):
    c, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().w4_packed_sizes(SCHEME_IDS[scheme], N, K, ctypes.byref(c), ctypes.byref(s),
                                 ctypes.byref(b)))
    return c.value, s.value, b.value


@dataclass
class QuantizedMatrix:
    """Storage form of one quantized matrix (or a fixed-stride stack of experts).

    codes: uint8 [E][N][K*bits/8]; scale: fp32 [E][N][K/128] (sym) or bf16
    [E][N][K/64]; bias: bf16 [E][N][K/64] or None. E = num_experts (leading
    dimension omitted when 1)."""
    scheme: str
    N: int
    K: int
    codes: torch.Tensor
    scale: torch.Tensor
    bias: Optional[torch.Tensor]
    num_experts: int = 1

    def desc(self) -> _W4Matrix:
        return _W4Matrix(SCHEME_IDS[self.scheme], self.num_experts, self.N, self.K,
                         _ptr(self.codes), _ptr(self.scale), _ptr(self.bias))

    def expert(self, e: int) -> "QuantizedMatrix":
        if self.num_experts == 1:
            return self
        return QuantizedMatrix(self.scheme, self.N, self.K, self.codes[e], self.scale[e],
                               None if self.bias is None else self.bias[e], 1)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scale, self.bias)
                   if t is not None)


def empty_quantized(scheme: str, N: int, K: int, num_experts: int = 1, device="cuda") -> QuantizedMatrix:
    packed_sizes(scheme, N, K)  # validates the shape
    lead = (num_experts,) if num_experts > 1 else ()
    bits = 8 if scheme == "aff8_g64" else 4
    codes = torch.empty(lead + (N, K * bits // 8), dtype=torch.uint8, device=device)
    if scheme == "sym4_g128":
        scale = torch.empty(lead + (N, K // 128), dtype=torch.float32, device=device)
        bias = None
    else:
        scale = torch.empty(lead + (N, K // 64), dtype=torch.bfloat16, device=device)
        bias = torch.empty(lead + (N, K // 64), dtype=torch.bfloat16, device=device)
    return QuantizedMatrix(scheme, N, K, codes, scale, bias, num_experts)


def quantize_pack(W: torch.Tensor, scheme: str, out: Optional[QuantizedMatrix] = None,
                  expert: Optional[int] = None) -> QuantizedMatrix:
    """Quantize fp32 weights W[N][K] on the device (into `out`, or expert `expert` of it)."""
    _dev(W, "W")
    if W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError("W must be a 2-D float32 tensor")
    N, K = W.shape
    q = out if out is not None else empty_quantized(scheme, N, K, device=W.device)
    tgt = q.expert(expert) if expert is not None else q
    _check(lib().w4_quantize_pack(SCHEME_IDS[scheme], _ptr(W), N, K, _ptr(tgt.codes),
                                  _ptr(tgt.scale), _ptr(tgt.bias), _stream(W.device)))
    return q


def _as_bf16_bits(x: torch.Tensor, name: str) -> torch.Tensor:
    _dev(x, name)
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError(f"{name} must hold bf16 values")
    return x


def gemv_into(W: QuantizedMatrix, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    x = _as_bf16_bits(x, "x")
    M = x.shape[0] if x.dim() == 2 else 1
    d = W.desc()
    _check(lib().w4a16_gemv(ctypes.byref(d), _ptr(x), M, _ptr(y), _stream(x.device)))
    return y


def gemv_workspace_bytes(W: QuantizedMatrix, M: int) -> int:
    """Workspace bytes with which gemv_ws_into splits K across CUs (0: no split)."""
    d = W.desc()
    return int(lib().w4_gemv_workspace_bytes(ctypes.byref(d), M))


def gemv_ws_into(W: QuantizedMatrix, x: torch.Tensor, y: torch.Tensor,
                 workspace: Optional[torch.Tensor]) -> torch.Tensor:
    """gemv_into with a device workspace (>= gemv_workspace_bytes(W, M) bytes, or None when 0)."""
    x = _as_bf16_bits(x, "x")
    M = x.shape[0] if x.dim() == 2 else 1
    d = W.desc()
    wp, wb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    _check(lib().w4a16_gemv_ws(ctypes.byref(d), _ptr(x), M, _ptr(y), wp, wb, _stream(x.device)))
    return y


def gemv_multi_into(Ws, x: torch.Tensor, ys) -> list:
    """Several GEMVs sharing x (one launch at M == 1): ys[i] = x · dequant(Ws[i])^T."""
    x = _as_bf16_bits(x, "x")
    M = x.shape[0] if x.dim() == 2 else 1
    n = len(Ws)
    descs = [W.desc() for W in Ws]
    arr = (ctypes.POINTER(_W4Matrix) * n)(*[ctypes.pointer(d) for d in descs])
    yp = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    _check(lib().w4a16_gemv_multi(arr, n, _ptr(x), M, yp, _stream(x.device)))
    return ys


def gemv_multi(Ws, x: torch.Tensor) -> list:
    M = x.shape[0] if x.dim() == 2 else 1
    ys = [torch.empty((M, W.N), dtype=torch.float32, device=x.device) for W in Ws]
    return gemv_multi_into(Ws, x, ys)


def gemv(W: QuantizedMatrix, x: torch.Tensor) -> torch.Tensor:
    """y[M][N] (fp32) = x[M][K] (bf16) · dequant(W)^T, dequantization fused in the kernel."""
    M = x.shape[0] if x.dim() == 2 else 1
    y = torch.empty((M, W.N), dtype=torch.float32, device=x.device)
    return gemv_into(W, x, y)


def gemm(W: QuantizedMatrix, X: torch.Tensor, Y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prefill: Y[M][N] (bf16) = X[M][K] (bf16) · dequant(W)^T with fp32 accumulation."""
    X = _as_bf16_bits(X, "X")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, W.N), dtype=torch.bfloat16, device=X.device)
    d = W.desc()
    _check(lib().w4a16_gemm(ctypes.byref(d), _ptr(X), M, _ptr(Y), _stream(X.device)))
    return Y


def moe_route(router: QuantizedMatrix, x: torch.Tensor, top_k: int = 8):
    """Router: (ids int32 [M][k], weights fp32 [M][k], logits fp32 [M][E])."""
    x = _as_bf16_bits(x, "x")
    M = x.shape[0]
    ids = torch.empty((M, top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((M, top_k), dtype=torch.float32, device=x.device)
    logits = torch.empty((M, router.N), dtype=torch.float32, device=x.device)
    d = router.desc()
    _check(lib().w4_moe_route(ctypes.byref(d), _ptr(x), M, top_k, _ptr(logits), _ptr(ids), _ptr(w),
                              _stream(x.device)))
    return ids, w, logits


def moe_workspace_bytes(M: int, top_k: int, E: int, D: int, F: int, Fs: int = 0) -> int:
    return int(lib().w4_moe_workspace_bytes(M, top_k, E, D, F, Fs))


def moe_gemv_logits(gate: QuantizedMatrix, up: QuantizedMatrix, down: QuantizedMatrix,
                    x: torch.Tensor, logits: torch.Tensor, top_k: int = 8, shared=None,
                    workspace=None, y: Optional[torch.Tensor] = None, ids=None, weights=None):
    """Selection from router logits [M][E] and the MoE FFN in one call: (y, ids, weights)."""
    x = _as_bf16_bits(x, "x")
    M = x.shape[0]
    E, F, D = gate.num_experts, gate.N, gate.K
    if logits.dtype != torch.float32 or tuple(logits.shape) != (M, E) or not logits.is_contiguous():
        raise ValueError(f"logits must be contiguous fp32 [{M}][{E}]")
    Fs = shared[0].N if shared is not None else 0
    need = moe_workspace_bytes(M, top_k, E, D, F, Fs)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, D), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty((M, top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((M, top_k), dtype=torch.float32, device=x.device)
    descs = [m.desc() for m in (gate, up, down)]
    sh = [s.desc() for s in shared] if shared is not None else [None, None, None]
    refs = [ctypes.byref(d) for d in descs] + [ctypes.byref(s) if s is not None else None for s in sh]
    _check(lib().w4a16_moe_gemv_logits(*refs, _ptr(x), M, _ptr(logits), top_k, _ptr(ids),
                                       _ptr(weights), _ptr(workspace), workspace.numel(), _ptr(y),
                                       _stream(x.device)))
    return y, ids, weights


def moe_gemv(gate: QuantizedMatrix, up: QuantizedMatrix, down: QuantizedMatrix, x: torch.Tensor,
             ids: torch.Tensor, weights: torch.Tensor, shared=None, workspace=None,
             y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MoE FFN over the selected experts plus an optional shared expert (gate, up, down)."""
    x = _as_bf16_bits(x, "x")
    M, top_k = ids.shape
    E, F, D = gate.num_experts, gate.N, gate.K
    Fs = shared[0].N if shared is not None else 0
    need = moe_workspace_bytes(M, top_k, E, D, F, Fs)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, D), dtype=torch.float32, device=x.device)
    descs = [m.desc() for m in (gate, up, down)]
    sh = [s.desc() for s in shared] if shared is not None else [None, None, None]
    refs = [ctypes.byref(d) for d in descs] + [ctypes.byref(s) if s is not None else None for s in sh]
    _check(lib().w4a16_moe_gemv(*refs, _ptr(x), M, _ptr(ids), _ptr(weights), top_k, _ptr(workspace),
                                workspace.numel(), _ptr(y), _stream(x.device)))
    return y


# ---------------------------------------------------------------- INT4 KV cache
KV_HEAD_DIM = 128


def kv_cache(Hkv: int, T_max: int, device="cuda"):
    """An empty INT4 KV cache for one of K or V: (codes uint8 [Hkv][T_max][64], scales fp32 [Hkv][T_max])."""
    codes = torch.empty((Hkv, T_max, KV_HEAD_DIM // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((Hkv, T_max), dtype=torch.float32, device=device)
    return codes, scales


def kv_quantize(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, pos: int) -> None:
    """Quantize x fp32 [n][Hkv][128] (or [Hkv][128]) into the cache at positions pos .. pos+n-1."""
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be contiguous fp32")
    n = 1 if x.dim() == 2 else x.shape[0]
    Hkv, T_max = scales.shape
    _check(lib().w4_kv_quantize(_ptr(x), n, Hkv, pos, T_max, _ptr(codes), _ptr(scales),
                                _stream(x.device)))


def kv_append(k: torch.Tensor, v: torch.Tensor, k_cache, v_cache, pos: int) -> None:
    """Quantize k and v fp32 [n][Hkv][128] into their caches ((codes, scales) pairs) at pos, one launch."""
    for t in (k, v):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("k and v must be contiguous fp32")
    n = 1 if k.dim() == 2 else k.shape[0]
    Hkv, T_max = k_cache[1].shape
    _check(lib().w4_kv_append(_ptr(k), _ptr(v), n, Hkv, pos, T_max, _ptr(k_cache[0]), _ptr(k_cache[1]),
                              _ptr(v_cache[0]), _ptr(v_cache[1]), _stream(k.device)))


def kv_scores(q: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, T: int,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """scores fp32 [Hq][T] = q [Hq][128] . dequant(K cache)[head group][t] for t < T."""
    Hq = q.shape[0]
    Hkv, T_max = scales.shape
    if out is None:
        out = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    _check(lib().w4_kv_scores(_ptr(q), Hq, Hkv, T, T_max, _ptr(codes), _ptr(scales), _ptr(out),
                              _stream(q.device)))
    return out


def kv_scores_append(q: torch.Tensor, k_new: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                     pos: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Quantize k_new fp32 [n][Hkv][128] (or [Hkv][128]) into the key cache at pos .. pos+n-1 and
    return scores fp32 [Hq][pos+n] over every position (one launch for n <= 16)."""
    if k_new.dtype != torch.float32 or not k_new.is_contiguous():
        raise ValueError("k_new must be contiguous fp32")
    n = 1 if k_new.dim() == 2 else k_new.shape[0]
    Hq = q.shape[0]
    Hkv, T_max = scales.shape
    if out is None:
        out = torch.empty((Hq, pos + n), dtype=torch.float32, device=q.device)
    _check(lib().w4_kv_scores_append(_ptr(q), _ptr(k_new), n, Hq, Hkv, pos, T_max, _ptr(codes),
                                     _ptr(scales), _ptr(out), _stream(q.device)))
    return out


def kv_weighted_sum_workspace_bytes(Hq: int, T: int) -> int:
    return int(lib().w4_kv_weighted_sum_workspace_bytes(Hq, T))


def kv_weighted_sum(p: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out fp32 [Hq][128] = sum_t p[h][t] * dequant(V cache)[head group][t], t < p.shape[1]."""
    Hq, T = p.shape
    Hkv, T_max = scales.shape
    if out is None:
        out = torch.empty((Hq, KV_HEAD_DIM), dtype=torch.float32, device=p.device)
    need = kv_weighted_sum_workspace_bytes(Hq, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=p.device)
    _check(lib().w4_kv_weighted_sum(_ptr(p), Hq, Hkv, T, T_max, _ptr(codes), _ptr(scales), _ptr(out),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(p.device)))
    return out


def kv_weighted_sum_append(p: torch.Tensor, v_new: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                           pos: int, workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Quantize v_new fp32 [n][Hkv][128] (or [Hkv][128]) into the value cache at pos .. pos+n-1 and
    return out fp32 [Hq][128] = sum over t < pos+n = p.shape[1] of p[h][t] * dequant(V)[t]."""
    if v_new.dtype != torch.float32 or not v_new.is_contiguous():
        raise ValueError("v_new must be contiguous fp32")
    n = 1 if v_new.dim() == 2 else v_new.shape[0]
    Hq, T = p.shape
    if T != pos + n:
        raise ValueError(f"p covers {T} positions, pos + n = {pos + n}")
    Hkv, T_max = scales.shape
    if out is None:
        out = torch.empty((Hq, KV_HEAD_DIM), dtype=torch.float32, device=p.device)
    need = kv_weighted_sum_workspace_bytes(Hq, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=p.device)
    _check(lib().w4_kv_weighted_sum_append(_ptr(p), _ptr(v_new), n, Hq, Hkv, pos, T_max, _ptr(codes),
                                           _ptr(scales), _ptr(out), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(p.device)))
    return out


MOE_SCRATCH_BYTES = 16 << 20


def moe_gemv_noalloc(gate: QuantizedMatrix, up: QuantizedMatrix, down: QuantizedMatrix,
                     x: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor, shared=None,
                     y: torch.Tensor = None) -> torch.Tensor:
    """moe_gemv with the library's static per-GPU scratch as its workspace (no
    device allocation by the library; calls overlapping on one GPU race)."""
    x = _as_bf16_bits(x, "x")
    M, top_k = ids.shape
    if y is None:
        y = torch.empty((M, gate.K), dtype=torch.float32, device=x.device)
    descs = [m.desc() for m in (gate, up, down)]
    sh = [s.desc() for s in shared] if shared is not None else [None, None, None]
    refs = [ctypes.byref(d) for d in descs] + [ctypes.byref(s) if s is not None else None for s in sh]
    _check(lib().w4a16_moe_gemv_noalloc(*refs, _ptr(x), M, _ptr(ids), _ptr(weights), top_k, _ptr(y),
                                        _stream(x.device)))
    return y


MOE_LAYER_GAVE_UP_LOGITS, MOE_LAYER_GAVE_UP_IDS, MOE_LAYER_GAVE_UP_H = 1, 2, 4


def moe_layer_workspace(M: int, top_k: int, E: int, D: int, F: int, Fs: int = 0,
                        device="cuda") -> torch.Tensor:
    """A workspace for moe_layer (up to M tokens), zero-filled as its first use requires."""
    n = int(lib().w4_moe_layer_workspace_bytes(M, top_k, E, D, F, Fs))
    if n == 0:
        raise ValueError("invalid sizes for a MoE layer workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_layer(router: QuantizedMatrix, gate: QuantizedMatrix, up: QuantizedMatrix,
              down: QuantizedMatrix, x: torch.Tensor, top_k: int = 8, shared=None,
              workspace: torch.Tensor = None, y: torch.Tensor = None, ids: torch.Tensor = None,
              weights: torch.Tensor = None):
    """Router, top-k and the MoE FFN from x [M][D]: (y, ids, weights). One token runs
    as a single launch (see w4a16_moe_layer in include/w4a16.h)."""
    x = _as_bf16_bits(x, "x")
    M = x.shape[0]
    E, F, D = gate.num_experts, gate.N, gate.K
    Fs = shared[0].N if shared is not None else 0
    if workspace is None:
        workspace = moe_layer_workspace(M, top_k, E, D, F, Fs, x.device)
    if y is None:
        y = torch.empty((M, D), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty((M, top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((M, top_k), dtype=torch.float32, device=x.device)
    descs = [m.desc() for m in (router, gate, up, down)]
    sh = [s.desc() for s in shared] if shared is not None else [None, None, None]
    refs = [ctypes.byref(d) for d in descs] + [ctypes.byref(s) if s is not None else None for s in sh]
    _check(lib().w4a16_moe_layer(*refs, _ptr(x), M, top_k, _ptr(ids), _ptr(weights), _ptr(y),
                                 _ptr(workspace), workspace.numel(), _stream(x.device)))
    return y, ids, weights


def moe_layer_status(workspace: torch.Tensor) -> int:
    """0, or the W4_MOE_LAYER_GAVE_UP_* bits of the last single-launch call (synchronizes)."""
    v = ctypes.c_int32()
    _check(lib().w4_moe_layer_status(_ptr(workspace), ctypes.byref(v), _stream(workspace.device)))
    return v.value


def moe_layer_set_single_launch(enable: bool) -> None:
    """Whether one token takes the single launch (where it applies) or the launch sequence."""
    lib().w4_moe_layer_set_single_launch(int(bool(enable)))


def moe_layer_set_wait(max_polls: int = 0, withhold: bool = False) -> None:
    """Testing hook: poll limit of the single-launch layer's waits (0 = default) and
    whether it withholds its expert selection (every wait for it then gives up)."""
    lib().w4_moe_layer_set_wait(int(max_polls), int(bool(withhold)))


# ---------------------------------------------------------------- dense gated FFN
FFN_GAVE_UP_H = 4


def ffn_workspace(down: QuantizedMatrix, M: int, device="cuda") -> torch.Tensor:
    """A workspace for ffn (up to M tokens), zero-filled as its first use requires."""
    d = down.desc()
    n = int(lib().w4_ffn_workspace_bytes(ctypes.byref(d), M))
    if n == 0:
        raise ValueError("invalid sizes for an FFN workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def ffn(gate: QuantizedMatrix, up: QuantizedMatrix, down: QuantizedMatrix, x: torch.Tensor,
        workspace: torch.Tensor = None, y: torch.Tensor = None, h: torch.Tensor = None,
        want_h: bool = False):
    """Gated FFN from x [M][D]: y = W_down · bf16(gelu_tanh(W_gate x) * (W_up x)).
    Returns y (fp32 [M][D]), or (y, h) with h bf16 [M][F] when h is given or
    want_h. The launches follow ffn_set_path (see w4a16_ffn in include/w4a16.h)."""
    x = _as_bf16_bits(x, "x")
    M = x.shape[0] if x.dim() == 2 else 1
    if workspace is None:
        workspace = ffn_workspace(down, M, x.device)
    if y is None:
        y = torch.empty((M, down.N), dtype=torch.float32, device=x.device)
    if h is None and want_h:
        h = torch.empty((M, gate.N), dtype=torch.bfloat16, device=x.device)
    dg, du, dd = gate.desc(), up.desc(), down.desc()
    _check(lib().w4a16_ffn(ctypes.byref(dg), ctypes.byref(du), ctypes.byref(dd), _ptr(x), M, _ptr(h),
                           _ptr(y), _ptr(workspace), workspace.numel(), _stream(x.device)))
    return (y, h) if h is not None else y


def ffn_gate_up_workspace(gate: QuantizedMatrix, M: int, device="cuda") -> torch.Tensor:
    """A workspace for ffn_gate_up (up to M tokens)."""
    d = gate.desc()
    n = int(lib().w4_ffn_gate_up_workspace_bytes(ctypes.byref(d), M))
    if n == 0:
        raise ValueError("invalid sizes for an FFN gate/up workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def ffn_gate_up(gate: QuantizedMatrix, up: QuantizedMatrix, x: torch.Tensor, h: torch.Tensor = None,
                workspace: torch.Tensor = None) -> torch.Tensor:
    """h (bf16 [M][F]) = bf16(gelu_tanh(W_gate x) * (W_up x)): the gate/up half of ffn."""
    x = _as_bf16_bits(x, "x")
    M = x.shape[0] if x.dim() == 2 else 1
    dg, du = gate.desc(), up.desc()
    if workspace is None:
        workspace = ffn_gate_up_workspace(gate, M, x.device)
    if h is None:
        h = torch.empty((M, gate.N), dtype=torch.bfloat16, device=x.device)
    _check(lib().w4a16_ffn_gate_up(ctypes.byref(dg), ctypes.byref(du), _ptr(x), M, _ptr(h),
                                   _ptr(workspace), workspace.numel(), _stream(x.device)))
    return h


def ffn_status(workspace: torch.Tensor) -> int:
    """0, or FFN_GAVE_UP_H if the last single-launch call gave up a wait (synchronizes)."""
    v = ctypes.c_int32()
    _check(lib().w4_ffn_status(_ptr(workspace), ctypes.byref(v), _stream(workspace.device)))
    return v.value


FFN_PATH_DEFAULT, FFN_PATH_SINGLE_LAUNCH, FFN_PATH_SEQUENCE = 0, 1, 2


def ffn_set_path(path: int) -> None:
    """How one token runs: FFN_PATH_DEFAULT (two launches), FFN_PATH_SINGLE_LAUNCH
    (one persistent launch where it applies) or FFN_PATH_SEQUENCE (three launches)."""
    _check(lib().w4_ffn_set_path(int(path)))


def ffn_set_wait(max_polls: int = 0, withhold: bool = False) -> None:
    """Testing hook: poll limit of the single launch's waits (0 = default) and whether
    it withholds the "h complete" flag (every wait for it then gives up)."""
    lib().w4_ffn_set_wait(int(max_polls), int(bool(withhold)))
