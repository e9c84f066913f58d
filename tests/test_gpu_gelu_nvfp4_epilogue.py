"""GPU parity of bsp_mm_fp4_gelu_nvfp4: the fc_in GEMM whose epilogue writes the NVFP4 encoding of
gelu_tanh(C) instead of C.

Against the oracle: operands whose every product and partial sum is exact in fp32 (scales that are
powers of two, |products| and K small enough for 24 bits; alpha a power of two), so the GEMM result
C is the same number on both sides and bf16(C) is too. The oracle then takes the pages' chain on
its own: exact C -> bf16 -> gelu (fp64, one rounding to bf16) -> nvfp4 quantize. The kernel's GELU
uses the hardware exp2 and reciprocal (a few fp32 ulps), so a value whose fp64 GELU lies within
2^-20 (relative) of a bf16 rounding boundary may round the other way; the 16-element blocks holding
such a value are compared loosely (scale code within one step, element codes within one e2m1
step), every other block bit for bit (gpu_util.assert_nvfp4_of_gelu), and the padding scale rows
must be zero.

Against the two-kernel path (bsp_mm_fp4 to bf16, then bsp_nvfp4_quantize_gelu), on general
operands including subnormal scales and at the full Wan-14B fc_in size: the same bytes.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsp
from oracle import activations as A
from oracle import nvfp4 as N
from tests.gpu_util import assert_nvfp4_of_gelu, dev_bf16, dev_u8, host_u8, say, scalar, tensor_bits

pytestmark = pytest.mark.gpu

POW2_SCALES = np.array([0x30, 0x38, 0x40], dtype=np.uint8)    # e4m3 codes of 1/2, 1, 2


def _exact_operand(rng, rows, k):
    """Random e2m1 bytes (every code) with power-of-two block scales (some blocks zero)."""
    packed = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    rp, cp = N.sf_padded_shape(rows, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:rows, : k // 16] = rng.choice(POW2_SCALES, size=(rows, k // 16))
    lin[:rows, : k // 16][rng.random((rows, k // 16)) < 0.02] = 0
    return packed, N.swizzle_128x4(lin)


def _general_operand(rng, rows, k):
    packed = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    rp, cp = N.sf_padded_shape(rows, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:rows, : k // 16] = rng.integers(0, 0x7F, size=(rows, k // 16))
    return packed, N.swizzle_128x4(lin)


@pytest.mark.parametrize("m,n,k,gsf", [(1, 128, 64, 1.0), (77, 384, 256, 1.0), (300, 256, 512, 0.75),
                                       (129, 640, 1024, 3.0), (256, 512, 128, 1.0)])
def test_gelu_nvfp4_epilogue_matches_oracle_on_exact_products(m, n, k, gsf):
    say("gelu_nvfp4 epilogue vs oracle", m, n, k, gsf)
    rng = np.random.default_rng(1000 + m + n + k)
    pa, sa = _exact_operand(rng, m, k)
    pb, sb = _exact_operand(rng, n, k)
    al = np.float32(2.0 ** -9)
    # every product has at most 4 significant bits above 2^-4 and |C| * 2^9 <= 144 k < 2^18: the
    # fp32 sums are exact whatever their order
    yb = A.f64_to_bf16_bits(N.mm_fp4(pa, sa, pb, sb, al, m, n, k))

    p, s = bsp.bsp_mm_fp4_gelu_nvfp4(dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(al),
                                     scalar(gsf))
    rp_, cp_ = N.sf_padded_shape(m, n)
    gp, gs = host_u8(p), host_u8(s).ravel()
    assert gp.shape == (m, n // 2) and gs.size == rp_ * cp_
    lin = N.unswizzle_128x4(gs, rp_, cp_)
    assert not lin[m:].any(), "padding scale rows must be zero"
    assert_nvfp4_of_gelu(gp, lin, yb, gsf, f"gelu_nvfp4 epilogue {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 128, 64), (77, 384, 192), (300, 256, 512), (513, 640, 256),
                                   (64, 1024, 1024)])
def test_gelu_nvfp4_epilogue_equals_two_kernel_path(m, n, k):
    say("gelu_nvfp4 epilogue vs two kernels", m, n, k)
    rng = np.random.default_rng(7 * m + n + 3 * k)
    pa, sa = _general_operand(rng, m, k)
    pb, sb = _general_operand(rng, n, k)
    al = np.float32(rng.uniform(0.01, 2.0))
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(al))
    g = scalar(1.5)
    p, s = bsp.bsp_mm_fp4_gelu_nvfp4(*args, g)
    p2, s2 = bsp.bsp_nvfp4_quantize_gelu(bsp.bsp_mm_fp4(*args), g)
    assert torch.equal(p, p2)
    assert torch.equal(s.view(-1), s2.view(-1))


def test_gelu_nvfp4_epilogue_full_size_fc_in():
    """Wan-14B fc_in, X[32760, 5120] x W[13824, 5120]: the same bytes as the two-kernel path over
    the whole output (the two-kernel path is itself checked against the oracle at this size)."""
    xb, wb = tensor_bits(3, "X"), tensor_bits(3, "W")
    say("gelu_nvfp4 epilogue full size", xb.shape, wb.shape)
    one = scalar(1.0)
    px, sx = bsp.bsp_nvfp4_quantize(dev_bf16(xb), one)
    pw, sw, gw, _, _ = bsp.bsp_nvfp4_prequantize_weight(dev_bf16(wb))
    alpha = bsp.bsp_nvfp4_alpha(one, gw)
    p, s = bsp.bsp_mm_fp4_gelu_nvfp4(px, sx, pw, sw, alpha, one)
    y = bsp.bsp_mm_fp4(px, sx, pw, sw, alpha)
    p2, s2 = bsp.bsp_nvfp4_quantize_gelu(y, one)
    del y
    assert torch.equal(p, p2)
    assert torch.equal(s.view(-1), s2.view(-1))


def test_gelu_nvfp4_epilogue_reuses_outputs_and_handles_empty():
    rng = np.random.default_rng(5)
    pa, sa = _general_operand(rng, 100, 128)
    pb, sb = _general_operand(rng, 256, 128)
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(0.5), scalar(1.0))
    p, s = bsp.bsp_mm_fp4_gelu_nvfp4(*args)
    p.fill_(0xAB)
    s.fill_(0xCD)
    p3, s3 = bsp.bsp_mm_fp4_gelu_nvfp4(*args, packed=p, sf=s)
    p2, s2 = bsp.bsp_mm_fp4_gelu_nvfp4(*args)
    assert p3.data_ptr() == p.data_ptr() and torch.equal(p3, p2) and torch.equal(s3, s2)
    e = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    pe, se = bsp.bsp_mm_fp4_gelu_nvfp4(e, e, dev_u8(pb), dev_u8(sb), scalar(1.0), scalar(1.0))
    assert pe.shape == (0, 128) and se.numel() == 0
