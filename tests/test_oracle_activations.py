"""Pins for the GELU oracle: library special case, closed-form values and symmetry."""
import numpy as np
import torch

import workloads as W
from oracle import activations as A


def test_matches_torch_fp64_tanh_gelu():
    # where 1 + tanh(z) does not cancel in fp64 the two forms agree to rounding
    x = np.linspace(-5, 12, 20001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.allclose(A.gelu_tanh(x), ref, rtol=1e-14, atol=1e-15)


def test_closed_form_points_and_symmetry():
    assert A.gelu_tanh(np.array([0.0]))[0] == 0.0
    x = np.linspace(-6, 6, 1001)
    assert np.allclose(A.gelu_tanh(x) - A.gelu_tanh(-x), x, atol=1e-14)   # gelu(x) - gelu(-x) = x
    assert abs(A.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12


def test_bf16_rounding_is_single_nearest_even():
    rng = np.random.default_rng(0)
    xb = W.f32_to_bf16_bits(rng.standard_normal(50000).astype(np.float32) * 3)
    got = A.gelu_tanh_bf16_bits(xb)
    y = A.gelu_tanh(W.bf16_bits_to_f32(xb))
    vals = W.bf16_bits_to_f32(got).astype(np.float64)
    # nearest: no other bf16 neighbour is closer
    up = W.bf16_bits_to_f32((got.astype(np.int32) + 1).astype(np.uint16)).astype(np.float64)
    dn = W.bf16_bits_to_f32((got.astype(np.int32) - 1).astype(np.uint16)).astype(np.float64)
    err = np.abs(vals - y)
    d_up = np.nan_to_num(np.abs(up - y), nan=np.inf)
    d_dn = np.nan_to_num(np.abs(dn - y), nan=np.inf)
    assert np.all(err <= d_up) and np.all(err <= d_dn)


def test_far_negative_tail_is_tiny_and_signed():
    y = A.gelu_tanh(np.array([-8.0, -9.0, -30.0]))
    assert np.all(y <= 0) and np.all(np.abs(y) < 1e-20)


def test_bf16_rounding_subnormal_and_ties():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 2^-130 is bf16-subnormal exact
    b = A.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 2.0 ** -130, -2.0 ** -140, 0.0]))
    assert list(b) == [0x3F80, 0x3F82, 0x0008, 0x8000, 0x0000]
