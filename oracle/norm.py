"""RMSNorm oracle for the norm + NVFP4 quantize prologue of a quantized linear layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FastVideo nvfp4_config.py (NVFP4QuantizeMethod.apply) accepts a ``pre_quantized`` triple (packed
FP4 values, block scales, global scale) in place of the activation, produced by FlashInfer's fused
norm + quantize calls, so the norm that precedes a projection can emit NVFP4 directly. The page
names the producer but not the norm. Reading taken: RMSNorm over the last (K) dimension, the norm of
the LTX-2 transformer blocks that page quantizes,
    y[m, k] = x[m, k] / sqrt(mean_k(x[m, :]^2) + eps) * w[k]     (w = 1 when there is no weight),
evaluated in fp64 and rounded once to bf16 (nearest even). The quantize that follows is
``nvfp4.quantize`` applied to those bf16 values, so the fused result is that composition.
"""
from __future__ import annotations

import numpy as np

from . import nvfp4
from .activations import f64_to_bf16_bits


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def rms_norm(x: np.ndarray, w: np.ndarray | None = None, eps: float = 1e-6) -> np.ndarray:
    """fp64 RMSNorm of each row of x (any float array [M, K]); w is an optional [K] gain."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + np.float64(eps))
    if w is not None:
        y = y * np.asarray(w, dtype=np.float64)
    return y


def rms_norm_bf16_bits(x_bits: np.ndarray, w_bits: np.ndarray | None = None,
                       eps: float = 1e-6) -> np.ndarray:
    """bf16 bits [M, K] (and optional bf16 gain bits [K]) -> bf16 bits of the normalized rows."""
    w = None if w_bits is None else bf16_bits_to_f64(w_bits)
    return f64_to_bf16_bits(rms_norm(bf16_bits_to_f64(x_bits), w, eps))


def quantize_rms_norm(x_bits: np.ndarray, gsf: np.float32, w_bits: np.ndarray | None = None,
                      eps: float = 1e-6):
    """NVFP4 quantize of the bf16 RMSNorm output: (packed [M, K/2], 128x4 scale bytes)."""
    return nvfp4.quantize(rms_norm_bf16_bits(x_bits, w_bits, eps), gsf)
