"""Pins for the RMSNorm oracle: library special case, closed forms, invariances and a hand-worked
norm + NVFP4 quantize block."""
import numpy as np
import torch

import workloads as W
from oracle import norm as R
from oracle import nvfp4 as N


def test_matches_torch_fp64_rms_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 160)) * np.array([0.01, 1, 3, 100, 1e-3, 7])[:, None]
    w = rng.standard_normal(160)
    for eps in (1e-6, 1e-2):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (160,), eps=eps).numpy()
        assert np.allclose(R.rms_norm(x, eps=eps), ref, rtol=1e-14, atol=0)
        refw = torch.nn.functional.rms_norm(torch.from_numpy(x), (160,), torch.from_numpy(w),
                                            eps=eps).numpy()
        assert np.allclose(R.rms_norm(x, w, eps=eps), refw, rtol=1e-14, atol=0)


def test_closed_forms():
    # a constant row c normalizes to sign(c) * |c| / sqrt(c^2 + eps); with eps = 0 exactly +-1
    c = np.array([[2.5] * 16, [-0.375] * 16])
    assert np.array_equal(R.rms_norm(c, eps=0.0), np.sign(c))
    y = R.rms_norm(np.array([[3.0] * 16]), eps=1.0)
    assert np.allclose(y, 3.0 / np.sqrt(10.0), rtol=1e-15)
    # alternating 3, 4: mean square 12.5, so y = (3, 4) / (5 / sqrt 2) = (0.6, 0.8) * sqrt 2
    y = R.rms_norm(np.array([[3.0, 4.0] * 8]), eps=0.0)[0]
    assert np.allclose(y[0::2], 0.6 * np.sqrt(2.0), rtol=1e-15)
    assert np.allclose(y[1::2], 0.8 * np.sqrt(2.0), rtol=1e-15)
    # an all-zero row stays zero (0 / sqrt(eps)); its sign bits are kept
    zb = np.array([[0x0000, 0x8000] * 8], dtype=np.uint16)
    assert np.array_equal(R.rms_norm_bf16_bits(zb), zb)


def test_unit_rms_and_power_of_two_invariance():
    rng = np.random.default_rng(2)
    xb = W.f32_to_bf16_bits(rng.standard_normal((8, 256)).astype(np.float32))
    y = R.rms_norm(R.bf16_bits_to_f64(xb), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    # scaling a row by 2^j scales its mean square by 4^j exactly: the bits do not change (eps = 0)
    for j in (-20, -3, 5, 40):
        xs = W.f32_to_bf16_bits((R.bf16_bits_to_f64(xb) * 2.0 ** j).astype(np.float32))
        assert np.array_equal(R.rms_norm_bf16_bits(xs, eps=0.0), R.rms_norm_bf16_bits(xb, eps=0.0))


def test_rows_are_independent_and_gain_is_elementwise():
    rng = np.random.default_rng(3)
    xb = W.f32_to_bf16_bits(rng.standard_normal((5, 64)).astype(np.float32) * 4)
    wb = W.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32))
    full = R.rms_norm_bf16_bits(xb, wb)
    for m in range(5):
        assert np.array_equal(R.rms_norm_bf16_bits(xb[m:m + 1], wb), full[m:m + 1])
    x = R.bf16_bits_to_f64(xb)
    assert np.allclose(R.rms_norm(x, R.bf16_bits_to_f64(wb)), R.rms_norm(x) * R.bf16_bits_to_f64(wb),
                       rtol=1e-15, atol=0)


def test_hand_worked_norm_then_nvfp4_block():
    # a constant row of 3.0 with eps = 0 normalizes to exactly 1.0 (bf16 0x3F80). Quantized with the
    # static global scale 1: block amax 1, s = fl32(1 * fl32(1/6)) = 0.1666667, which lies between the
    # e4m3 values 0.15625 and 0.171875 and rounds to 0.171875 = 2^-3 * 1.375 (code 0x23); the element
    # scale 1 / 0.171875 = 5.818 gives 1 * 5.818 -> e2m1 6.0 (code 7), so every packed byte is 0x77
    xb = np.full((1, 32), 0x4040, dtype=np.uint16)
    assert np.all(R.rms_norm_bf16_bits(xb, eps=0.0) == 0x3F80)
    packed, sf = R.quantize_rms_norm(xb, np.float32(1.0), eps=0.0)
    assert np.all(packed == 0x77)
    assert sf[0] == 0x23 and sf[1] == 0x23 and sf[2] == 0 and sf[3] == 0 and not sf[4:].any()
    # and the chain equals the NVFP4 quantize of the normalized bf16 values
    rng = np.random.default_rng(4)
    x2 = W.f32_to_bf16_bits(rng.standard_t(4, (130, 96)).astype(np.float32))
    p1, s1 = R.quantize_rms_norm(x2, np.float32(1.0))
    p2, s2 = N.quantize(R.rms_norm_bf16_bits(x2), np.float32(1.0))
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
