"""Oracle: the fused-dequant matrix products, as their plain definition.

TEST INFRASTRUCTURE (see oracle/__init__.py). Not used by the product path.

The method dequantizes inside the product ([airllm] §2.2: conversion right after
the weight load, no intermediate weight tensor); mathematically that is exactly
Y = X · dequant(W)^T, so the oracle writes the definition out: dequantize to a
dense fp64 matrix (exact), widen the bf16 activations to fp64 (exact), and call
one fp64 matrix product (a library primitive). S = |X| · |W'|^T is returned
alongside for the per-element tolerance 2e-3·S + 1e-5.
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_to_f32, dequantize


def matmul_f64(X_bf16: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """Y[m][n] = sum_k x[m][k] * w'[n][k] in fp64; X given as bf16 bit patterns."""
    X = bf16_to_f32(np.atleast_2d(X_bf16)).astype(np.float64)
    return X @ np.asarray(Wd, dtype=np.float64).T


def abs_matmul_f64(X_bf16: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """S[m][n] = sum_k |x[m][k]| * |w'[n][k]| (the tolerance scale)."""
    X = np.abs(bf16_to_f32(np.atleast_2d(X_bf16)).astype(np.float64))
    return X @ np.abs(np.asarray(Wd, dtype=np.float64)).T


def gemv_reference(codes, scale, bias, scheme: str, X_bf16, rows=None):
    """(Y, S) for the stored matrix against activations X; optionally only `rows`."""
    if rows is not None:
        rows = np.asarray(rows)
        codes = np.asarray(codes)[rows]
        scale = np.asarray(scale)[rows]
        bias = None if bias is None else np.asarray(bias)[rows]
    Wd = dequantize(codes, scale, bias, scheme)
    return matmul_f64(X_bf16, Wd), abs_matmul_f64(X_bf16, Wd)
