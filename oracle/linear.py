"""The linear layer's bias, as the pages add it after the quantized GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* FastVideo nvfp4_config.py, ``NVFP4QuantizeMethod.apply``: ``out = _mm_fp4(..., torch.bfloat16, ...)``
  and then ``out = out + bias`` on bf16 tensors. A bf16 add takes both operands to fp32, adds them
  (IEEE, nearest even) and rounds the sum to bf16 (nearest even). Two bf16 values add exactly in
  fp32 unless their exponents differ by more than 16, and then the smaller is below a quarter of
  the larger's bf16 ulp, so the result is also the single nearest-even rounding of the exact sum.
* vLLM-Omni mxfp8_config.py, ``NPUMxfp8LinearMethod._quant_matmul``: the bias is converted to fp32
  and handed to the quantized matmul, which writes the output dtype; the reading taken is that the
  fp32 bias joins the fp32 result before its one rounding to the output dtype.
"""
from __future__ import annotations

import numpy as np

from .activations import f64_to_bf16_bits


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def add_bias_bf16(out_bits: np.ndarray, bias_bits: np.ndarray) -> np.ndarray:
    """bf16 bits of out + bias (bias broadcast along the last axis): fl32 add, then bf16 RNE."""
    s = bf16_bits_to_f32(out_bits) + bf16_bits_to_f32(bias_bits)      # numpy fp32: IEEE RNE
    return f64_to_bf16_bits(s.astype(np.float64))                      # exact widening, one RNE


def gemm_plus_bias(c_f64: np.ndarray, bias_f32: np.ndarray) -> np.ndarray:
    """The exact GEMM result plus the fp32 bias (fp64), before the output rounding."""
    return np.asarray(c_f64, dtype=np.float64) + np.asarray(bias_f32, dtype=np.float32).astype(np.float64)
