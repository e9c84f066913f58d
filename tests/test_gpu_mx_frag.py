"""GPU parity of the MX fragment-layout paths (bsp_mxfp4_quantize_frag / bsp_mm_mxfp4_frag and
bsp_mxfp8_quantize_frag / bsp_mm_mxfp8_frag).

The quantizers must write exactly the oracle's bytes (codes, scales and zero padding rows) in the
fragment layout; each GEMM must meet the same bar as its linear-layout counterpart (mm_mxfp4,
mm_mxfp8) against the oracle's fp64 product of the same operand bytes, and, for the same operand
values, equal that counterpart's output bit for bit (same MFMA, same K order), with and without
bias. Small and ragged shapes compare every element; the Wan-14B fc_in shape
(32760 x 13824 x 5120) runs at full size and compares sampled entries.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsp
import workloads as W
from oracle import linear as L
from oracle import mxfp4 as X4
from oracle import mxfp8 as X
from oracle import nvfp4 as N
from tests.gpu_util import (assert_gemm_bf16, check_gemm_outputs, dev_bf16, dev_u8, host_u8,
                            sample_entries, say, scalar, tensor_bits)

pytestmark = pytest.mark.gpu
f32 = np.float32


def _frag_dev(fp: np.ndarray, fs: np.ndarray, rows: int, k: int):
    rt = X4.frag_rows(rows) // 32
    return (dev_u8(fp.reshape(rt, k // 64, 1024)), dev_u8(fs.reshape(rt, k // 256, 256)))


def _quant_frag_filled(xb: np.ndarray):
    """bsp_mxfp4_quantize_frag into buffers pre-filled with 0xA5, so a byte left unwritten shows."""
    m, k = xb.shape
    rt = X4.frag_rows(m) // 32
    p = torch.full((rt, k // 64, 1024), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((rt, k // 256, 256), 0xA5, dtype=torch.uint8, device="cuda")
    bsp.bsp_mxfp4_quantize_frag(dev_bf16(xb), p, s)
    return host_u8(p).ravel(), host_u8(s).ravel()


@pytest.mark.parametrize("m,k", [(1, 256), (33, 512), (128, 256), (130, 768), (300, 1280),
                                 (257, 2048)])
def test_mxfp4_quantize_frag_bit_exact(m, k):
    say("mxfp4_quantize_frag", m, k)
    for xb in (W.small_case(m, k, seed=7 * m + k, outlier_frac=0.02),
               W.special_values_block(seed=m + 1, rows=m, cols=k),
               W.nonfinite_block(seed=m + 2, rows=m, cols=k)):
        fp, fs = _quant_frag_filled(xb)
        rp, rs = X4.quantize(xb, layout="frag")
        assert np.array_equal(fp, rp) and np.array_equal(fs, rs)


def test_mxfp4_quantize_frag_strided_input():
    """A row stride larger than K (a column slice of a wider matrix)."""
    xb = W.small_case(70, 1024, seed=5, outlier_frac=0.02)
    xd = dev_bf16(xb)[:, :768]
    p, s = bsp.bsp_mxfp4_quantize_frag(xd)
    rp, rs = X4.quantize(np.ascontiguousarray(xb[:, :768]), layout="frag")
    assert np.array_equal(host_u8(p).ravel(), rp) and np.array_equal(host_u8(s).ravel(), rs)


def test_mxfp4_quantize_frag_full_size():
    """Wan-14B fc_in activation 32760 x 5120: whole row tiles (first, middle, the ragged last one)
    against the oracle of those rows; every other byte against the linear-layout quantizer's."""
    xb = tensor_bits(4, "X")
    m, k = xb.shape
    p, s = bsp.bsp_mxfp4_quantize_frag(dev_bf16(xb))
    rt = X4.frag_rows(m) // 32
    for t in (0, 517, rt - 1):
        rows = xb[32 * t: min(32 * t + 32, m)]
        rp, rs = X4.quantize(rows, layout="frag")
        assert np.array_equal(host_u8(p[t]).ravel(), rp), t
        assert np.array_equal(host_u8(s[t]).ravel(), rs), t
    # the same codes and scales as bsp_mxfp4_quantize, rearranged on the device
    pl, sl = bsp.bsp_mxfp4_quantize(dev_bf16(xb))
    mp = rt * 32
    plin = torch.zeros((mp, k // 2), dtype=torch.uint8, device="cuda")
    plin[:m] = pl
    want_p = plin.view(rt, 32, k // 64, 2, 16).permute(0, 2, 3, 1, 4).contiguous().view(-1)
    # 128x4 -> row-major [ceil128(m), K/32] -> fragment scale groups
    rt128 = sl.numel() // (128 * (k // 32))
    slin = sl.view(rt128, k // 128, 32, 4, 4).permute(0, 3, 2, 1, 4).reshape(rt128 * 128, k // 32)[:mp]
    want_s = slin.reshape(rt, 32, k // 256, 4, 2).permute(0, 2, 4, 1, 3).contiguous().view(-1)
    assert torch.equal(p.view(-1), want_p) and torch.equal(s.view(-1), want_s)


def _rand_operand(rng, rows, k):
    """Random codes and scales: (fragment-layout flat pair, 128x4-layout pair) of the same values."""
    packed = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    lin = rng.integers(110, 140, size=(rows, k // 32)).astype(np.uint8)
    fp, fs = X4.to_frag(packed, lin, k)
    rp, cp = X4.sf_padded_shape(rows, k)
    pad = np.zeros((rp, cp), dtype=np.uint8)
    pad[:rows, : k // 32] = lin
    return (fp, fs), (packed, N.swizzle_128x4(pad))


@pytest.mark.parametrize("m,n,k", [(1, 64, 256), (77, 200, 256), (256, 256, 512), (300, 130, 768),
                                   (513, 384, 1280), (3, 1, 256), (1, 1, 256), (260, 520, 2304)])
def test_mm_mxfp4_frag_random_operands_all_elements(m, n, k):
    say("mm_mxfp4_frag random", m, n, k)
    rng = np.random.default_rng(m * 7 + n + k)
    (fa, fsa), (pa, sa) = _rand_operand(rng, m, k)
    (fb, fsb), (pb, sb) = _rand_operand(rng, n, k)
    al = f32(0.625)
    ref = X4.mm_mxfp4_frag(fa, fsa, fb, fsb, al, m, n, k)
    a, a_s = _frag_dev(fa, fsa, m, k)
    b, b_s = _frag_dev(fb, fsb, n, k)
    t32 = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(al), out_dtype=torch.float32)
    t16 = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(al))
    check_gemm_outputs(t16, t32, ref, f"mxfp4 frag {m}x{n}x{k}")
    std = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(al))
    assert torch.equal(t32, bsp.bsp_mm_mxfp4(*std, out_dtype=torch.float32))
    assert torch.equal(t16.view(torch.int16), bsp.bsp_mm_mxfp4(*std).view(torch.int16))
    c1 = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, None, out_dtype=torch.float32)
    assert torch.equal(c1, bsp.bsp_mm_mxfp4(*std[:4], None, torch.float32))


@pytest.mark.parametrize("m,n,k", [(77, 200, 256), (256, 256, 512)])
def test_mm_mxfp4_frag_bias(m, n, k):
    say("mm_mxfp4_frag bias", m, n, k)
    rng = np.random.default_rng(m + 3 * n + k)
    (fa, fsa), (pa, sa) = _rand_operand(rng, m, k)
    (fb, fsb), (pb, sb) = _rand_operand(rng, n, k)
    al = f32(0.375)
    ref = X4.mm_mxfp4_frag(fa, fsa, fb, fsb, al, m, n, k)
    bf = (rng.standard_normal(n) * (float(np.std(ref)) + 1e-30)).astype(np.float32)
    bf[::7] = 0.0
    bbits = W.f32_to_bf16_bits(bf)
    bias = dev_bf16(bbits)
    a, a_s = _frag_dev(fa, fsa, m, k)
    b, b_s = _frag_dev(fb, fsb, n, k)
    tb16 = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(al), bias)
    std = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb))
    assert torch.equal(tb16.view(torch.int16), bsp.bsp_mm_mxfp4_bias(*std, bias, scalar(al)).view(torch.int16))
    t32 = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(al), out_dtype=torch.float32)
    from oracle import activations as A
    want = W.bf16_bits_to_f32(L.add_bias_bf16(A.f64_to_bf16_bits(ref), bbits)).astype(np.float64)
    assert_gemm_bf16(tb16.float().cpu().numpy().astype(np.float64), want, t32.cpu().numpy(),
                     f"mxfp4 frag bias {m}x{n}x{k}")
    tb32 = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(al), bias, out_dtype=torch.float32)
    assert torch.equal(tb32, t32 + bias.float())


@pytest.mark.parametrize("m,n,k,grids", [(1100, 1300, 1024, (1, 4, 7)),     # 4 deferred stores per K group
                                         (530, 777, 4096, (3, 8)),          # 2 per group, all inside the K loop
                                         (600, 520, 6144, (2, 5))])         # above the persistent K limit
def test_mm_mxfp4_frag_persistent_grids(m, n, k, grids, monkeypatch):
    """Small grids, so that each workgroup runs many tiles (whole and ragged) and stores each whole
    tile during the next one's K loop: every element against the oracle, and bit for bit equal to
    mm_mxfp4 on the linear-layout operands, with bf16 and fp32 output and with bias."""
    rng = np.random.default_rng(m + n + k)
    (fa, fsa), (pa, sa) = _rand_operand(rng, m, k)
    (fb, fsb), (pb, sb) = _rand_operand(rng, n, k)
    al = f32(0.75)
    ref = X4.mm_mxfp4_frag(fa, fsa, fb, fsb, al, m, n, k)
    a, a_s = _frag_dev(fa, fsa, m, k)
    b, b_s = _frag_dev(fb, fsb, n, k)
    std = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb))
    bias = dev_bf16(W.f32_to_bf16_bits((rng.standard_normal(n) * float(np.std(ref))).astype(np.float32)))
    want16 = bsp.bsp_mm_mxfp4(*std, scalar(al))
    want32 = bsp.bsp_mm_mxfp4(*std, scalar(al), out_dtype=torch.float32)
    wantb = bsp.bsp_mm_mxfp4_bias(*std, bias, scalar(al))
    for g in grids:
        say("mm_mxfp4_frag persistent", m, n, k, "grid", g)
        monkeypatch.setenv("BSP_PERSISTENT_GRID", str(g))
        t16 = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(al))
        t32 = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(al), out_dtype=torch.float32)
        tb = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(al), bias)
        check_gemm_outputs(t16, t32, ref, f"mxfp4 frag {m}x{n}x{k} grid {g}")
        assert torch.equal(t16.view(torch.int16), want16.view(torch.int16)), g
        assert torch.equal(t32, want32), g
        assert torch.equal(tb.view(torch.int16), wantb.view(torch.int16)), g


def test_mm_mxfp4_frag_full_size():
    """Wan-14B fc_in, 32760 x 13824 x 5120, operands from bsp_mxfp4_quantize_frag: sampled entries
    against the oracle, and the whole output equal to mm_mxfp4's on the linear-layout operands."""
    xb, wb = tensor_bits(4, "X"), tensor_bits(4, "W")
    m, n, k = xb.shape[0], wb.shape[0], xb.shape[1]
    px, sx = bsp.bsp_mxfp4_quantize_frag(dev_bf16(xb))
    pw, sw = bsp.bsp_mxfp4_quantize_frag(dev_bf16(wb))
    c = bsp.bsp_mm_mxfp4_frag(px, sx, pw, sw, m, n)
    c32 = bsp.bsp_mm_mxfp4_frag(px, sx, pw, sw, m, n, out_dtype=torch.float32)
    rows, cols = sample_entries(m, n, 3000, 43)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    rpx, rsx = X4.quantize(xb[ur])
    rpw, rsw = X4.quantize(wb[uc])
    ref = X4.mm_mxfp4_entries(rpx, rsx, rpw, rsw, 1.0, len(ur), len(uc), k, ri, ci)
    check_gemm_outputs(c, c32, ref, "fc_in mxfp4 frag", rows, cols)
    lx, lsx = bsp.bsp_mxfp4_quantize(dev_bf16(xb))
    lw, lsw = bsp.bsp_mxfp4_quantize(dev_bf16(wb))
    assert torch.equal(c.view(torch.int16), bsp.bsp_mm_mxfp4(lx, lsx, lw, lsw).view(torch.int16))


# ------------------------------------------------------------------------------------------ MXFP8

def _quant8_frag_filled(xb: np.ndarray):
    m, k = xb.shape
    rt = X4.frag_rows(m) // 32
    q = torch.full((rt, k // 64, 2048), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((rt, k // 256, 256), 0xA5, dtype=torch.uint8, device="cuda")
    bsp.bsp_mxfp8_quantize_frag(dev_bf16(xb), q, s)
    return host_u8(q).ravel(), host_u8(s).ravel()


@pytest.mark.parametrize("m,k", [(1, 256), (33, 512), (64, 256), (130, 768), (300, 1280),
                                 (257, 2048)])
def test_mxfp8_quantize_frag_bit_exact(m, k):
    say("mxfp8_quantize_frag", m, k)
    for xb in (W.small_case(m, k, seed=5 * m + k, outlier_frac=0.02),
               W.special_values_block(seed=m + 3, rows=m, cols=k),
               W.nonfinite_block(seed=m + 4, rows=m, cols=k)):
        fq, fs = _quant8_frag_filled(xb)
        rq, rs = X.quantize_frag(xb)
        assert np.array_equal(fq, rq) and np.array_equal(fs, rs)


def test_mxfp8_quantize_frag_strided_input():
    xb = W.small_case(70, 1024, seed=6, outlier_frac=0.02)
    q, s = bsp.bsp_mxfp8_quantize_frag(dev_bf16(xb)[:, :512])
    rq, rs = X.quantize_frag(np.ascontiguousarray(xb[:, :512]))
    assert np.array_equal(host_u8(q).ravel(), rq) and np.array_equal(host_u8(s).ravel(), rs)


def test_mxfp8_quantize_frag_full_size():
    """Wan-14B fc_in activation 32760 x 5120: whole row tiles against the oracle of those rows;
    every byte against the row-major quantizer's output rearranged on the device."""
    xb = tensor_bits(5, "X")
    m, k = xb.shape
    q, s = bsp.bsp_mxfp8_quantize_frag(dev_bf16(xb))
    rt = X4.frag_rows(m) // 32
    for t in (0, 311, rt - 1):
        rq, rs = X.quantize_frag(xb[32 * t: min(32 * t + 32, m)])
        assert np.array_equal(host_u8(q[t]).ravel(), rq), t
        assert np.array_equal(host_u8(s[t]).ravel(), rs), t
    ql, sl = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
    mp = rt * 32
    qp = torch.zeros((mp, k), dtype=torch.uint8, device="cuda")
    qp[:m] = ql
    sp = torch.zeros((mp, k // 32), dtype=torch.uint8, device="cuda")
    sp[:m] = sl
    want_q = qp.view(rt, 32, k // 64, 2, 2, 16).permute(0, 2, 3, 4, 1, 5).contiguous().view(-1)
    want_s = sp.view(rt, 32, k // 256, 4, 2).permute(0, 2, 4, 1, 3).contiguous().view(-1)
    assert torch.equal(q.view(-1), want_q) and torch.equal(s.view(-1), want_s)


def _rand_operand8(rng, rows, k):
    """Random e4m3 bytes (no NaN codes) and scales: (fragment flat pair, row-major pair)."""
    q = rng.integers(0, 256, size=(rows, k)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3F
    s = rng.integers(110, 140, size=(rows, k // 32)).astype(np.uint8)
    return X.to_frag(q, s, k), (q, s)


def _frag8_dev(fq, fs, rows, k):
    rt = X4.frag_rows(rows) // 32
    return dev_u8(fq.reshape(rt, k // 64, 2048)), dev_u8(fs.reshape(rt, k // 256, 256))


@pytest.mark.parametrize("m,n,k", [(1, 64, 256), (77, 200, 256), (256, 256, 512), (300, 130, 768),
                                   (513, 384, 1280), (3, 1, 256), (260, 520, 3328)])
def test_mm_mxfp8_frag_random_operands_all_elements(m, n, k):
    say("mm_mxfp8_frag random", m, n, k)
    rng = np.random.default_rng(m * 11 + n + k)
    (fa, fsa), (qa, sa) = _rand_operand8(rng, m, k)
    (fb, fsb), (qb, sb) = _rand_operand8(rng, n, k)
    ref = X.mm_mxfp8_frag(fa, fsa, fb, fsb, m, n, k)
    a, a_s = _frag8_dev(fa, fsa, m, k)
    b, b_s = _frag8_dev(fb, fsb, n, k)
    t32 = bsp.bsp_mm_mxfp8_frag(a, a_s, b, b_s, m, n, out_dtype=torch.float32)
    t16 = bsp.bsp_mm_mxfp8_frag(a, a_s, b, b_s, m, n)
    check_gemm_outputs(t16, t32, ref, f"mxfp8 frag {m}x{n}x{k}")
    std = (dev_u8(qa), dev_u8(sa), dev_u8(qb), dev_u8(sb))
    assert torch.equal(t32, bsp.bsp_mm_mxfp8(*std, out_dtype=torch.float32))
    assert torch.equal(t16.view(torch.int16), bsp.bsp_mm_mxfp8(*std).view(torch.int16))


@pytest.mark.parametrize("m,n,k", [(77, 200, 256), (256, 256, 512)])
def test_mm_mxfp8_frag_bias(m, n, k):
    say("mm_mxfp8_frag bias", m, n, k)
    rng = np.random.default_rng(m + 5 * n + k)
    (fa, fsa), (qa, sa) = _rand_operand8(rng, m, k)
    (fb, fsb), (qb, sb) = _rand_operand8(rng, n, k)
    ref = X.mm_mxfp8_frag(fa, fsa, fb, fsb, m, n, k)
    bf = rng.normal(0.0, float(np.std(ref)) + 1e-30, size=n).astype(np.float32)
    bias = torch.from_numpy(bf).cuda()
    a, a_s = _frag8_dev(fa, fsa, m, k)
    b, b_s = _frag8_dev(fb, fsb, n, k)
    tb32 = bsp.bsp_mm_mxfp8_frag(a, a_s, b, b_s, m, n, bias, out_dtype=torch.float32)
    tb16 = bsp.bsp_mm_mxfp8_frag(a, a_s, b, b_s, m, n, bias)
    std = (dev_u8(qa), dev_u8(sa), dev_u8(qb), dev_u8(sb))
    assert torch.equal(tb32, bsp.bsp_mm_mxfp8_bias(*std, bias, out_dtype=torch.float32))
    assert torch.equal(tb16.view(torch.int16), bsp.bsp_mm_mxfp8_bias(*std, bias).view(torch.int16))
    check_gemm_outputs(tb16, tb32, L.gemm_plus_bias(ref, bf), f"mxfp8 frag bias {m}x{n}x{k}")


def test_mm_mxfp8_frag_full_size():
    """Wan-14B fc_in, 32760 x 13824 x 5120, operands from bsp_mxfp8_quantize_frag: sampled entries
    against the oracle, and the whole output equal to mm_mxfp8's on the row-major operands."""
    xb, wb = tensor_bits(5, "X"), tensor_bits(5, "W")
    m, n, k = xb.shape[0], wb.shape[0], xb.shape[1]
    qx, sx = bsp.bsp_mxfp8_quantize_frag(dev_bf16(xb))
    qw, sw = bsp.bsp_mxfp8_quantize_frag(dev_bf16(wb))
    c = bsp.bsp_mm_mxfp8_frag(qx, sx, qw, sw, m, n)
    c32 = bsp.bsp_mm_mxfp8_frag(qx, sx, qw, sw, m, n, out_dtype=torch.float32)
    rows, cols = sample_entries(m, n, 3000, 47)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    rq, rs = X.quantize(xb[ur])
    rqw, rsw = X.quantize(wb[uc])
    ref = X.mm_mxfp8_entries(rq, rs, rqw, rsw, ri, ci)
    check_gemm_outputs(c, c32, ref, "fc_in mxfp8 frag", rows, cols)
    lx, lsx = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
    lw, lsw = bsp.bsp_mxfp8_quantize(dev_bf16(wb))
    assert torch.equal(c.view(torch.int16), bsp.bsp_mm_mxfp8(lx, lsx, lw, lsw).view(torch.int16))
