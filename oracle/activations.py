"""GELU (tanh form) oracle for the activation between the FFN projections.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages quantize both Wan FFN projections (FastVideo nvfp4_qat_config.py, the default FP4 layer
list holds ffn.fc_in and ffn.fc_out), so the hidden activation between them is quantized per call;
the Wan FFN applies the tanh-approximated GELU there:
    gelu(x) = 0.5 * x * (1 + tanh(z)),  z = sqrt(2/pi) * (x + 0.044715 * x^3)
evaluated in fp64 through the identity 0.5 * (1 + tanh(z)) = 1 / (1 + exp(-2z)), which avoids the
cancellation of 1 + tanh(z) for negative z, then rounded once to bf16 (nearest even).
"""
from __future__ import annotations

import numpy as np


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    z = np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-2.0 * z))


def f64_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits with a single round-to-nearest-even (normal and subnormal range)."""
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)
    step = np.where(np.abs(y) >= 2.0 ** -126, np.ldexp(1.0, e - 8), 2.0 ** -133)
    r = (np.round(y / step) * step).astype(np.float32)     # exact: <= 8 significant bits
    r = np.where(r == 0, np.copysign(0.0, y), r).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def gelu_tanh_bf16_bits(x_bits: np.ndarray) -> np.ndarray:
    """bf16 bits in -> bf16 bits of gelu_tanh."""
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f64_to_bf16_bits(gelu_tanh(x))
