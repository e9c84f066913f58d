"""Seeded sweep over random shapes (ragged M and N, several K, strided rows) for every GEMM and
quantizer entry point, against the oracle on every element or byte.

The fixed-shape tests pin known edge cases; this sweep adds breadth: tile remainders in both M and
N at once, K that ends on a half stage, and row strides above K, drawn from one seed so a failure
names a reproducible case.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsp
import workloads as W
from oracle import mxfp4 as X4
from oracle import mxfp8 as X
from oracle import nvfp4 as N
from tests.gpu_util import (REL_FRO_FP4_F32, assert_gemm_f32, check_gemm_outputs, dev_bf16, dev_u8,
                            host_u8, say, scalar)

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(20261203)
GEMM_CASES = [(int(_RNG.integers(1, 700)), int(_RNG.integers(1, 700)), int(_RNG.integers(1, 9)) * 128)
              for _ in range(10)]
QUANT_CASES = [(int(_RNG.integers(1, 600)), int(_RNG.integers(1, 40)) * 32, int(_RNG.integers(0, 3)) * 8)
               for _ in range(10)]


def _nvfp4_operand(rng, rows, k):
    packed = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    rp, cp = N.sf_padded_shape(rows, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:rows, : k // 16] = rng.integers(0, 0x7F, size=(rows, k // 16))
    return packed, N.swizzle_128x4(lin)


def _mxfp4_operand(rng, rows, k):
    packed = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    rp, cp = X4.sf_padded_shape(rows, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:rows, : k // 32] = rng.integers(110, 140, size=(rows, k // 32))
    return packed, N.swizzle_128x4(lin)


def _mx8_operand(rng, rows, k):
    q = rng.integers(0, 256, size=(rows, k), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3F
    return q, rng.integers(110, 140, size=(rows, k // 32), dtype=np.uint8)


@pytest.mark.parametrize("m,n,k", GEMM_CASES)
def test_gemm_sweep(m, n, k):
    """mm_fp4 (K and K - 64, the half-stage tail), mm_mxfp8 and mm_mxfp4 on every element."""
    say("gemm sweep", m, n, k)
    rng = np.random.default_rng(m * 1009 + n * 31 + k)
    for kk in (k, k - 64) if k > 64 else (k,):
        pa, sa = _nvfp4_operand(rng, m, kk)
        pb, sb = _nvfp4_operand(rng, n, kk)
        ref = N.mm_fp4(pa, sa, pb, sb, np.float32(0.75), m, n, kk)
        args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(0.75))
        check_gemm_outputs(bsp.bsp_mm_fp4(*args), bsp.bsp_mm_fp4(*args, out_dtype=torch.float32), ref,
                           f"mm_fp4 {m}x{n}x{kk}", f32_tol=REL_FRO_FP4_F32)
    qa, s8a = _mx8_operand(rng, m, k)
    qb, s8b = _mx8_operand(rng, n, k)
    ref = X.mm_mxfp8(qa, s8a, qb, s8b, m, n, k)
    a8 = (dev_u8(qa), dev_u8(s8a), dev_u8(qb), dev_u8(s8b))
    check_gemm_outputs(bsp.bsp_mm_mxfp8(*a8), bsp.bsp_mm_mxfp8(*a8, out_dtype=torch.float32), ref,
                       f"mm_mxfp8 {m}x{n}x{k}")
    pa, sa = _mxfp4_operand(rng, m, k)
    pb, sb = _mxfp4_operand(rng, n, k)
    ref = X4.mm_mxfp4(pa, sa, pb, sb, np.float32(1.0), m, n, k)
    a4 = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), None)
    check_gemm_outputs(bsp.bsp_mm_mxfp4(*a4), bsp.bsp_mm_mxfp4(*a4, out_dtype=torch.float32), ref,
                       f"mm_mxfp4 {m}x{n}x{k}")


@pytest.mark.parametrize("m,k,pad", QUANT_CASES)
def test_quantize_sweep(m, k, pad):
    """NVFP4 (tensor scale, per token, layout_8x4), MXFP8 and MXFP4 quantizers on rows of stride
    K + pad: every packed, element and scale byte, padding included."""
    say("quantize sweep", m, k, pad)
    xb = W.small_case(m, k, seed=m * 17 + k + pad, std=1.5, outlier_frac=0.03)
    big = np.zeros((m, k + pad), dtype=np.uint16)
    big[:, :k] = xb
    x = dev_bf16(big)[:, :k]
    g = N.global_sf(xb)[0]
    p, sf = bsp.bsp_nvfp4_quantize(x, scalar(g))
    rp, rs = N.quantize(xb, g)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(sf).ravel(), rs)
    p, sf, gr = bsp.bsp_nvfp4_quantize_per_token(x)
    rp, rs, rg = N.quantize_per_token(xb)
    assert np.array_equal(gr.cpu().numpy(), rg)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(sf).ravel(), rs)
    p, sf = bsp.bsp_nvfp4_quantize_8x4(x, scalar(g))
    rp, rs = N.quantize(xb, g, layout="8x4")
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(sf).ravel(), rs)
    q, s = bsp.bsp_mxfp8_quantize(x)
    rq, rs = X.quantize(xb)
    assert np.array_equal(host_u8(q), rq) and np.array_equal(host_u8(s), rs)
    p, sf = bsp.bsp_mxfp4_quantize(x)
    rp, rs = X4.quantize(xb)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(sf).ravel(), rs)


VARIANT_CASES = GEMM_CASES[:6]


@pytest.mark.parametrize("m,n,k", VARIANT_CASES)
def test_gemm_variant_sweep(m, n, k):
    """The GEMM entry points with per-token alphas, layout_8x4 activation scales and fused bias on
    the sweep's shapes, every element against the oracle."""
    from oracle import linear as L
    say("gemm variant sweep", m, n, k)
    rng = np.random.default_rng(m * 7 + n * 13 + k)
    pa, sa = _nvfp4_operand(rng, m, k)
    pb, sb = _nvfp4_operand(rng, n, k)
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb))
    xg = (10.0 ** rng.uniform(-2, 3, size=m)).astype(np.float32)
    wg = np.float32(321.5)
    ref = N.mm_fp4_rowscale(pa, sa, pb, sb, xg, wg, m, n, k)
    pt = (*args, torch.from_numpy(xg).cuda(), scalar(wg))
    check_gemm_outputs(bsp.bsp_mm_fp4_per_token(*pt), bsp.bsp_mm_fp4_per_token(*pt, out_dtype=torch.float32),
                       ref, f"per-token {m}x{n}x{k}", f32_tol=REL_FRO_FP4_F32)
    sa8 = N.swizzle_8x4(N.unswizzle_128x4(sa, *N.sf_padded_shape(m, k))[:N.sf_padded_shape_8x4(m, k)[0]])
    ref = N.mm_fp4(pa, sa8, pb, sb, np.float32(0.5), m, n, k, a_layout="8x4")
    c = bsp.bsp_mm_fp4_8x4(dev_u8(pa), dev_u8(sa8), dev_u8(pb), dev_u8(sb), scalar(0.5), out_dtype=torch.float32)
    assert_gemm_f32(c.cpu().numpy().astype(np.float64), ref, f"8x4 {m}x{n}x{k}")
    # bias: the NVFP4 / MXFP4 outputs are the bf16 product plus the bf16 bias (the pages' bf16 add,
    # compared bit for bit with torch's add on the device); the MXFP8 one is the fp32 product plus the
    # fp32 bias, rounded once, against the oracle's exact product plus bias
    bbits = W.f32_to_bf16_bits(rng.normal(0.0, float(np.std(ref)) + 1e-30, size=n).astype(np.float32))
    bias = dev_bf16(bbits)
    c0 = bsp.bsp_mm_fp4(*args, scalar(0.5))
    check_gemm_outputs(c0, bsp.bsp_mm_fp4(*args, scalar(0.5), out_dtype=torch.float32),
                       N.mm_fp4(pa, sa, pb, sb, np.float32(0.5), m, n, k), f"mm_fp4 {m}x{n}x{k}",
                       f32_tol=REL_FRO_FP4_F32)
    c = bsp.bsp_mm_fp4_bias(*args, scalar(0.5), bias)
    assert torch.equal(c.view(torch.int16), (c0.float() + bias.float()).bfloat16().view(torch.int16))
    qa, s8a = _mx8_operand(rng, m, k)
    qb, s8b = _mx8_operand(rng, n, k)
    ref = X.mm_mxfp8(qa, s8a, qb, s8b, m, n, k)
    bf = rng.normal(0.0, float(np.std(ref)) + 1e-30, size=n).astype(np.float32)
    a8 = (dev_u8(qa), dev_u8(s8a), dev_u8(qb), dev_u8(s8b))
    c32 = bsp.bsp_mm_mxfp8(*a8, out_dtype=torch.float32)
    cb32 = bsp.bsp_mm_mxfp8_bias(*a8, torch.from_numpy(bf).cuda(), out_dtype=torch.float32)
    assert np.array_equal(cb32.cpu().numpy(), (c32.cpu().numpy() + bf).astype(np.float32))
    c = bsp.bsp_mm_mxfp8_bias(*a8, torch.from_numpy(bf).cuda())
    assert torch.equal(c, cb32.bfloat16())
    check_gemm_outputs(c, cb32, L.gemm_plus_bias(ref, bf), f"mxfp8 bias {m}x{n}x{k}")
    pa4, sa4 = _mxfp4_operand(rng, m, k)
    pb4, sb4 = _mxfp4_operand(rng, n, k)
    a4 = (dev_u8(pa4), dev_u8(sa4), dev_u8(pb4), dev_u8(sb4))
    c0 = bsp.bsp_mm_mxfp4(*a4, scalar(0.25))
    check_gemm_outputs(c0, bsp.bsp_mm_mxfp4(*a4, scalar(0.25), out_dtype=torch.float32),
                       X4.mm_mxfp4(pa4, sa4, pb4, sb4, np.float32(0.25), m, n, k), f"mm_mxfp4 {m}x{n}x{k}")
    c = bsp.bsp_mm_mxfp4_bias(*a4, bias, scalar(0.25))
    assert torch.equal(c.view(torch.int16), (c0.float() + bias.float()).bfloat16().view(torch.int16))


@pytest.mark.parametrize("m,n,k", GEMM_CASES)
def test_frag_gemm_sweep(m, n, k):
    """The fragment-layout GEMMs on the sweep's shapes: mm_fp4_frag at K and K - 64, and the MX ones
    at K rounded down to a multiple of 256 (at least 256), every element against the oracle."""
    say("frag gemm sweep", m, n, k)
    rng = np.random.default_rng(m * 2003 + n * 17 + k)
    for kk in (k, k - 64) if k > 64 else (k,):
        pa, sa = _nvfp4_operand(rng, m, kk)
        pb, sb = _nvfp4_operand(rng, n, kk)
        fa, fb = N.to_frag_packed(pa, kk), N.to_frag_packed(pb, kk)
        ref = N.mm_fp4_frag(fa, sa, fb, sb, np.float32(0.75), m, n, kk)
        args = (dev_u8(fa.reshape(-1, kk // 64, 1024)), dev_u8(sa), dev_u8(fb.reshape(-1, kk // 64, 1024)),
                dev_u8(sb), m, n, scalar(0.75))
        check_gemm_outputs(bsp.bsp_mm_fp4_frag(*args), bsp.bsp_mm_fp4_frag(*args, out_dtype=torch.float32),
                           ref, f"mm_fp4_frag {m}x{n}x{kk}", f32_tol=REL_FRO_FP4_F32)
    k4 = max(256, k // 256 * 256)
    pa, pb = (rng.integers(0, 256, size=(r, k4 // 2), dtype=np.uint8) for r in (m, n))
    la, lb = (rng.integers(110, 140, size=(r, k4 // 32), dtype=np.uint8) for r in (m, n))
    (fa, fsa), (fb, fsb) = X4.to_frag(pa, la, k4), X4.to_frag(pb, lb, k4)
    ref = X4.mm_mxfp4_frag(fa, fsa, fb, fsb, np.float32(1.0), m, n, k4)
    a4 = (dev_u8(fa.reshape(-1, k4 // 64, 1024)), dev_u8(fsa.reshape(-1, k4 // 256, 256)),
          dev_u8(fb.reshape(-1, k4 // 64, 1024)), dev_u8(fsb.reshape(-1, k4 // 256, 256)), m, n)
    check_gemm_outputs(bsp.bsp_mm_mxfp4_frag(*a4), bsp.bsp_mm_mxfp4_frag(*a4, out_dtype=torch.float32), ref,
                       f"mm_mxfp4_frag {m}x{n}x{k4}")
    qa, s8a = _mx8_operand(rng, m, k4)
    qb, s8b = _mx8_operand(rng, n, k4)
    (ga, gsa), (gb, gsb) = X.to_frag(qa, s8a, k4), X.to_frag(qb, s8b, k4)
    ref = X.mm_mxfp8_frag(ga, gsa, gb, gsb, m, n, k4)
    a8 = (dev_u8(ga.reshape(-1, k4 // 64, 2048)), dev_u8(gsa.reshape(-1, k4 // 256, 256)),
          dev_u8(gb.reshape(-1, k4 // 64, 2048)), dev_u8(gsb.reshape(-1, k4 // 256, 256)), m, n)
    check_gemm_outputs(bsp.bsp_mm_mxfp8_frag(*a8), bsp.bsp_mm_mxfp8_frag(*a8, out_dtype=torch.float32), ref,
                       f"mm_mxfp8_frag {m}x{n}x{k4}")


@pytest.mark.parametrize("m,k,pad", QUANT_CASES)
def test_frag_quantize_sweep(m, k, pad):
    """The fragment-layout quantizers on rows of stride K + pad (K rounded up to a multiple of 64 for
    NVFP4 and 256 for MX): every packed byte, padding rows included, and every scale byte against
    the oracle's own fragment layout."""
    k64, k256 = -(-k // 64) * 64, -(-k // 256) * 256
    say("frag quantize sweep", m, k64, k256, pad)
    for kk in sorted({k64, k256}):
        xb = W.small_case(m, kk, seed=m * 19 + kk + pad, std=1.5, outlier_frac=0.03)
        big = np.zeros((m, kk + pad), dtype=np.uint16)
        big[:, :kk] = xb
        x = dev_bf16(big)[:, :kk]
        if kk == k64:
            g = N.global_sf(xb)[0]
            p, sf = bsp.bsp_nvfp4_quantize_frag(x, scalar(g))
            rp, rs = N.quantize(xb, g, packed_layout="frag")
            assert np.array_equal(host_u8(p).ravel(), rp) and np.array_equal(host_u8(sf).ravel(), rs)
        if kk == k256:
            p, sf = bsp.bsp_mxfp4_quantize_frag(x)
            rp, rs = X4.to_frag(*X4.quantize(xb, layout="linear"), kk)
            assert np.array_equal(host_u8(p).ravel(), rp) and np.array_equal(host_u8(sf).ravel(), rs)
            q, s = bsp.bsp_mxfp8_quantize_frag(x)
            rq, rs = X.quantize_frag(xb)
            assert np.array_equal(host_u8(q).ravel(), rq) and np.array_equal(host_u8(s).ravel(), rs)
