"""CPU oracle for group-wise 4-bit weight-only quantization and its fused matrix products.

TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg import this package; the product path (the HIP
library and its Python binding) never does, and this package imports nothing
from it. It is deliberately plain and slow: fp32 where the encoding is defined
in fp32, fp64 for every matrix product, numpy/PyTorch-CPU library primitives as
single steps, no blocking or fusion.

Sources (cited by page title and section; see each function):
  [airllm]          "airllm" article, cf-1.com/news/5708464 (page title garbled)
  [TurboFieldfare]  TurboFieldfare / Gemma 4 26B-A4B article, cnblogs.com/32bin/p/23195374
  [Shimmy]          "Shimmy 深度解剖：Airframe 引擎与 TurboShimmy INT4 KV", chenxutan.com/d/5228

Parity status: every function here is pinned by tests/test_oracle_*.py against
closed forms, exhaustive enumeration, exact rational arithmetic or an
independent library routine, except the choices the pages leave open (the
affine min/max rule, the FFN activation, the KV codec's all-zero vector), which
are pinned only by invariants and stated as readings.
"""
from .quant import (SCHEMES, GROUP, BITS, bf16_round, bf16_to_f32, quantize, quantize_sym4,
                    quantize_affine, pack, unpack, dequantize, quantize_pack, packed_nbytes)
from .matmul import matmul_f64, abs_matmul_f64, gemv_reference
from .moe import route, gelu_tanh, ffn, moe_sparse, moe_dense_masked
from .kv import kv_quantize, kv_unpack, kv_dequant, kv_scores, kv_weighted_sum

__all__ = [
    "SCHEMES", "GROUP", "BITS", "bf16_round", "bf16_to_f32", "quantize", "quantize_sym4",
    "quantize_affine", "pack", "unpack", "dequantize", "quantize_pack", "packed_nbytes",
    "matmul_f64", "abs_matmul_f64", "gemv_reference", "route", "gelu_tanh", "ffn",
    "moe_sparse", "moe_dense_masked", "kv_quantize", "kv_unpack", "kv_dequant", "kv_scores",
    "kv_weighted_sum",
]
