"""Maximum sizes each entry point accepts, on the GPU, against the oracle.

Quantizers at their largest row count (the grid's tile-row limit: ceil(M/128) < 65536, MXFP8
ceil(M/64) < 65536) with sampled rows, the first and last rows and every padding scale byte
checked; the GEMMs at K = 2^24 (mm_fp4's limit: per-tile 32-bit load offsets) on every element;
GEMMs with 8.4 million rows (int64 row offsets, 32768 tiles) on sampled rows, for mm_fp4 and for the
fragment-layout NVFP4 and MX GEMMs (and the fragment-layout NVFP4 GEMM at K = 2^24). One size past each limit is rejected on the host (tests/test_abi.py).
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsp
import workloads as W
from oracle import mxfp4 as X4
from oracle import mxfp8 as X
from oracle import nvfp4 as N
from tests.gpu_util import (assert_gemm_f32, dev_bf16, dev_u8, host_u8, say, scalar)

pytestmark = pytest.mark.gpu

M_MAX_128 = 65535 * 128      # 8388480 rows: grid.y (128-row tiles) below 65536
M_MAX_64 = 65535 * 64        # 4194240 rows: MXFP8 quantize's 64-row tiles


def _rows(m, seed):
    return np.unique(np.concatenate([np.random.default_rng(seed).integers(0, m, 40),
                                     [0, 1, 127, 128, m // 2, m - 129, m - 2, m - 1]]))


def _tall_bits(m, k, seed):
    """Seeded bf16 rows (the workload recipe) built in chunks so the host copy stays small."""
    out = np.empty((m, k), dtype=np.uint16)
    step = 1 << 20
    for r0 in range(0, m, step):
        r1 = min(m, r0 + step)
        out[r0:r1] = W.small_case(r1 - r0, k, seed=seed + r0 // step, std=2.0, outlier_frac=0.05)
    return out


def test_nvfp4_quantizers_at_max_rows():
    m, k = M_MAX_128, 32
    say("max rows nvfp4", m, k)
    xb = _tall_bits(m, k, 71)
    x = dev_bf16(xb)
    rows = _rows(m, 3)
    ri = torch.from_numpy(rows).cuda()
    rp, cp = N.sf_padded_shape(m, k)
    g = np.float32(0.37)
    p, sf = bsp.bsp_nvfp4_quantize(x, scalar(g))
    ref_p, ref_s = N.quantize(xb[rows], g, layout="linear")
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp, cp)
    assert np.array_equal(host_u8(p[ri]), ref_p)
    assert np.array_equal(lin[rows, : k // 16], ref_s) and not lin[:, k // 16:].any()
    del p, sf
    p, sf, gr = bsp.bsp_nvfp4_quantize_per_token(x)
    ref_p, ref_s, ref_g = N.quantize_per_token(xb[rows], layout="linear")
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp, cp)
    assert np.array_equal(gr[ri].cpu().numpy(), ref_g)
    assert np.array_equal(host_u8(p[ri]), ref_p) and np.array_equal(lin[rows, : k // 16], ref_s)
    del p, sf, gr
    p, sf = bsp.bsp_mxfp4_quantize(x)
    ref_p, ref_s = X4.quantize(xb[rows], layout="linear")
    rp4, cp4 = X4.sf_padded_shape(m, k)
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp4, cp4)
    assert np.array_equal(host_u8(p[ri]), ref_p) and np.array_equal(lin[rows, : k // 32], ref_s)


def test_mxfp8_quantize_at_max_rows():
    m, k = M_MAX_64, 64
    say("max rows mxfp8", m, k)
    xb = _tall_bits(m, k, 83)
    q, s = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
    rows = _rows(m, 4)
    ri = torch.from_numpy(rows).cuda()
    rq, rs = X.quantize(xb[rows])
    assert np.array_equal(host_u8(q[ri]), rq) and np.array_equal(host_u8(s[ri]), rs)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8", "nvfp4", "nvfp4_gelu"])
def test_frag_quantizers_at_max_rows(fmt):
    """The fragment-layout quantizers at their largest row count minus a ragged few (seeded device
    input, K = 256): sampled rows and every padding row of the last row tile, read through the
    layout's offsets, against the oracle (the GELU-fused NVFP4 one on the GPU's own GELU of the
    same rows, the bar of its parity tests)."""
    m = (M_MAX_64 if fmt == "mxfp8" else M_MAX_128) - 7
    k = 256
    say("max rows frag quantize", fmt, m, k)
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    x = (torch.randn((m, k), device="cuda", generator=g) * 2.0).bfloat16()
    gs = np.float32(0.37)
    if fmt == "mxfp4":
        q, s = bsp.bsp_mxfp4_quantize_frag(x)
    elif fmt == "mxfp8":
        q, s = bsp.bsp_mxfp8_quantize_frag(x)
    elif fmt == "nvfp4":
        q, s = bsp.bsp_nvfp4_quantize_frag(x, scalar(gs))
    else:
        q, s = bsp.bsp_nvfp4_quantize_gelu_frag(x, scalar(gs))
    rows = _rows(m, 6)
    xr = x[torch.from_numpy(rows).cuda()]
    if fmt == "nvfp4_gelu":
        xr = bsp.bsp_gelu_tanh_bf16(xr)
    xb = xr.view(torch.int16).cpu().numpy().view(np.uint16)
    rp = -(-m // 32) * 32
    pad = np.arange(m, rp)
    if fmt == "mxfp4":
        ref_q, ref_s = X4.quantize(xb, layout="linear")
        off = lambda r: X4.frag_packed_offset(r[:, None], np.arange(k // 2)[None, :], k)  # noqa: E731
    elif fmt == "mxfp8":
        ref_q, ref_s = X.quantize(xb)
        off = lambda r: X.frag_offset(r[:, None], np.arange(k)[None, :], k)  # noqa: E731
    else:
        ref_q, ref_s = N.quantize(xb, gs, layout="linear")
        off = lambda r: N.frag_packed_offset(r[:, None], np.arange(k // 2)[None, :], k)  # noqa: E731
    if fmt.startswith("nvfp4"):
        cp = N.sf_padded_shape(m, k)[1]
        soff = lambda r: N.sf_offset(r[:, None], np.arange(k // 16)[None, :], cp)  # noqa: E731
        assert N.sf_padded_shape(m, k)[0] == rp     # the 128-row scale padding is the same 7 rows
    else:
        soff = lambda r: X4.frag_sf_offset(r[:, None], np.arange(k // 32)[None, :], k)  # noqa: E731

    def gather(t, o):
        return t.view(-1)[torch.from_numpy(o.ravel()).cuda()].cpu().numpy().reshape(o.shape)

    assert np.array_equal(gather(q, off(rows)), ref_q)
    assert np.array_equal(gather(s, soff(rows)), ref_s)
    assert pad.size == 7 and not gather(q, off(pad)).any() and not gather(s, soff(pad)).any()


def _nvfp4_operand(rng, rows, k):
    packed = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    rp, cp = N.sf_padded_shape(rows, k)
    sfb = np.zeros(rp * cp, dtype=np.uint8)
    r, c = np.meshgrid(np.arange(rows), np.arange(k // 16), indexing="ij")
    sfb[N.sf_offset(r, c, cp)] = rng.integers(0x28, 0x48, size=(rows, k // 16), dtype=np.uint8)
    return packed, sfb


def _mxfp4_operand(rng, rows, k):
    packed = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    rp, cp = X4.sf_padded_shape(rows, k)
    sfb = np.zeros(rp * cp, dtype=np.uint8)
    r, c = np.meshgrid(np.arange(rows), np.arange(k // 32), indexing="ij")
    sfb[N.sf_offset(r, c, cp)] = rng.integers(120, 134, size=(rows, k // 32), dtype=np.uint8)
    return packed, sfb


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4"])
def test_gemm_at_k_2_24(fmt):
    """K = 2^24 (131072 NVFP4 stages per tile) with ragged M, N: every element against the oracle."""
    m, n, k = 3, 5, 1 << 24
    say("K = 2^24", fmt, m, n, k)
    rng = np.random.default_rng(24)
    if fmt == "nvfp4":
        pa, sa = _nvfp4_operand(rng, m, k)
        pb, sb = _nvfp4_operand(rng, n, k)
        c = bsp.bsp_mm_fp4(dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(0.25),
                           out_dtype=torch.float32)
        ref = N.mm_fp4(pa, sa, pb, sb, np.float32(0.25), m, n, k)
    elif fmt == "mxfp8":
        qa = rng.integers(0, 256, size=(m, k), dtype=np.uint8)
        qb = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
        qa[(qa & 0x7F) == 0x7F] = 0x3F
        qb[(qb & 0x7F) == 0x7F] = 0x3F
        sa = rng.integers(120, 134, size=(m, k // 32), dtype=np.uint8)
        sb = rng.integers(120, 134, size=(n, k // 32), dtype=np.uint8)
        c = bsp.bsp_mm_mxfp8(dev_u8(qa), dev_u8(sa), dev_u8(qb), dev_u8(sb), out_dtype=torch.float32)
        ref = X.mm_mxfp8(qa, sa, qb, sb, m, n, k)
    else:
        pa, sa = _mxfp4_operand(rng, m, k)
        pb, sb = _mxfp4_operand(rng, n, k)
        c = bsp.bsp_mm_mxfp4(dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), None, torch.float32)
        ref = X4.mm_mxfp4(pa, sa, pb, sb, np.float32(1.0), m, n, k)
    assert_gemm_f32(c.cpu().numpy().astype(np.float64), ref, f"K=2^24 {fmt}")


def test_mm_fp4_tall_max_rows():
    """M = 8388480 (32768 row tiles, rows addressed past 2^31 bytes of C), N = 136 (ragged), K = 64:
    sampled rows of C on every column against the oracle, in bf16."""
    m, n, k = M_MAX_128, 136, 64
    say("tall mm_fp4", m, n, k)
    rng = np.random.default_rng(99)
    pa, sa = _nvfp4_operand(rng, m, k)
    pb, sb = _nvfp4_operand(rng, n, k)
    c = bsp.bsp_mm_fp4(dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(1.0))
    rows = _rows(m, 5)
    got = c[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    ref = N.dequant_rows(pa, sa, rows, m, k) @ N.dequant_rows(pb, sb, np.arange(n), n, k).T
    err = np.abs(got - ref)
    assert np.all(err <= 8e-3 * np.max(np.abs(ref))), float(err.max())
    assert np.linalg.norm(got - ref) <= 3e-3 * np.linalg.norm(ref)


# --------------------------------------------------------------- NVFP4 GEMM, fragment layout
def test_mm_fp4_frag_at_k_2_24():
    """bsp_mm_fp4_frag at K = 2^24 (262144 K steps per tile; scale loads 2^27 bytes into a row
    tile) with ragged M, N: every element of the fp32 output against the oracle."""
    m, n, k = 3, 5, 1 << 24
    say("frag K = 2^24 nvfp4", m, n, k)
    rng = np.random.default_rng(224)
    pa, sa = _nvfp4_operand(rng, m, k)
    pb, sb = _nvfp4_operand(rng, n, k)
    fa, fb = N.to_frag_packed(pa, k), N.to_frag_packed(pb, k)
    del pa, pb
    a = dev_u8(fa.reshape(-1, k // 64, 1024))
    b = dev_u8(fb.reshape(-1, k // 64, 1024))
    c = bsp.bsp_mm_fp4_frag(a, dev_u8(sa), b, dev_u8(sb), m, n, scalar(0.25), out_dtype=torch.float32)
    ref = N.mm_fp4_frag(fa, sa, fb, sb, np.float32(0.25), m, n, k)
    assert_gemm_f32(c.cpu().numpy().astype(np.float64), ref, "frag K=2^24 nvfp4")


def test_mm_fp4_frag_tall_max_rows():
    """bsp_mm_fp4_frag with M = 8388480 (262140 row tiles, 32768 tile rows; C offsets past 2^31
    bytes), N = 136 (ragged), K = 256, device-random A: sampled rows of C, their operand bytes
    gathered through the layout's offsets, against the oracle, in bf16."""
    m, n, k = M_MAX_128, 136, 256
    say("tall frag nvfp4", m, n, k)
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    a = torch.randint(0, 256, (m // 32, k // 64, 1024), dtype=torch.uint8, device="cuda", generator=g)
    rp, cp = N.sf_padded_shape(m, k)
    a_s = torch.randint(0x28, 0x48, (rp, cp), dtype=torch.uint8, device="cuda", generator=g)
    rng = np.random.default_rng(18)
    pb, sb = _nvfp4_operand(rng, n, k)
    c = bsp.bsp_mm_fp4_frag(a, a_s, dev_u8(N.to_frag_packed(pb, k).reshape(-1, k // 64, 1024)),
                            dev_u8(sb), m, n, scalar(1.0))
    rows = _rows(m, 19)
    off = N.frag_packed_offset(rows[:, None], np.arange(k // 2)[None, :], k)
    soff = N.sf_offset(rows[:, None], np.arange(k // 16)[None, :], cp)
    pr = a.view(-1)[torch.from_numpy(off.ravel()).cuda()].cpu().numpy().reshape(off.shape)
    sr = a_s.view(-1)[torch.from_numpy(soff.ravel()).cuda()].cpu().numpy().reshape(soff.shape)
    # the sampled rows as a small operand of their own (row i of it is row rows[i] of A)
    sl = np.zeros(N.sf_padded_shape(len(rows), k), dtype=np.uint8)
    sl[: len(rows), : k // 16] = sr
    A = N.dequant_rows(pr, N.swizzle_128x4(sl), np.arange(len(rows)), len(rows), k)
    B = N.dequant_rows(pb, sb, np.arange(n), n, k)
    ref = A @ B.T
    got = c[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= 8e-3 * np.max(np.abs(ref))), float(err.max())
    assert np.linalg.norm(got - ref) <= 3e-3 * np.linalg.norm(ref)


# --------------------------------------------------------------- MX GEMMs, fragment layout
def _frag_operand(rng, rows, k, fmt):
    """Random fragment-layout bytes (no NaN codes, scales 2^-17 .. 2^12), padding rows included."""
    rp = -(-rows // 32) * 32
    nbytes = rp * k // 2 if fmt == "mxfp4" else rp * k
    q = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    if fmt == "mxfp8":
        q[(q & 0x7F) == 0x7F] = 0x3F
    s = rng.integers(110, 140, size=rp * k // 32, dtype=np.uint8)
    return q, s


def _frag_dev(q, s, rows, k, fmt):
    rt = -(-rows // 32)
    frag = 1024 if fmt == "mxfp4" else 2048
    return dev_u8(q.reshape(rt, k // 64, frag)), dev_u8(s.reshape(rt, k // 256, 256))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_frag_gemm_at_k_2_24(fmt):
    """Fragment-layout GEMMs at K = 2^24 (262144 K steps per tile) with ragged M, N: every element
    against the oracle."""
    m, n, k = 3, 5, 1 << 24
    say("frag K = 2^24", fmt, m, n, k)
    rng = np.random.default_rng(124)
    qa, sa = _frag_operand(rng, m, k, fmt)
    qb, sb = _frag_operand(rng, n, k, fmt)
    a, a_s = _frag_dev(qa, sa, m, k, fmt)
    b, b_s = _frag_dev(qb, sb, n, k, fmt)
    if fmt == "mxfp4":
        c = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n, scalar(0.5), out_dtype=torch.float32)
        ref = X4.mm_mxfp4_frag(qa, sa, qb, sb, np.float32(0.5), m, n, k)
    else:
        c = bsp.bsp_mm_mxfp8_frag(a, a_s, b, b_s, m, n, out_dtype=torch.float32)
        ref = X.mm_mxfp8_frag(qa, sa, qb, sb, m, n, k)
    assert_gemm_f32(c.cpu().numpy().astype(np.float64), ref, f"frag K=2^24 {fmt}")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_frag_gemm_tall_max_rows(fmt):
    """M = 8388480 (262140 row tiles; operand and C offsets past 2^31 bytes), N = 136, K = 256:
    sampled rows of C, gathered from the fragment layout on the device, against the oracle."""
    m, n, k = M_MAX_128, 136, 256
    say("tall frag", fmt, m, n, k)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    rt = -(-m // 32)
    frag = 1024 if fmt == "mxfp4" else 2048
    a = torch.randint(0, 256, (rt, k // 64, frag), dtype=torch.uint8, device="cuda", generator=g)
    if fmt == "mxfp8":
        a[(a & 0x7F) == 0x7F] = 0x3F
    a_s = torch.randint(115, 135, (rt, k // 256, 256), dtype=torch.uint8, device="cuda", generator=g)
    rng = np.random.default_rng(8)
    qb, sb = _frag_operand(rng, n, k, fmt)
    b, b_s = _frag_dev(qb, sb, n, k, fmt)
    if fmt == "mxfp4":
        c = bsp.bsp_mm_mxfp4_frag(a, a_s, b, b_s, m, n)
    else:
        c = bsp.bsp_mm_mxfp8_frag(a, a_s, b, b_s, m, n)
    rows = _rows(m, 9)
    # the sampled rows' bytes, read through the layout's own offsets
    if fmt == "mxfp4":
        off = X4.frag_packed_offset(rows[:, None], np.arange(k // 2)[None, :], k)
    else:
        off = X.frag_offset(rows[:, None], np.arange(k)[None, :], k)
    soff = X4.frag_sf_offset(rows[:, None], np.arange(k // 32)[None, :], k)
    ra = a.view(-1)[torch.from_numpy(off.ravel()).cuda()].cpu().numpy().reshape(off.shape)
    rs = a_s.view(-1)[torch.from_numpy(soff.ravel()).cuda()].cpu().numpy().reshape(soff.shape)
    if fmt == "mxfp4":
        A = X4.dequant_linear(ra, rs)
        B = X4.dequant_linear(*X4.from_frag(qb, sb, n, k))
    else:
        A = X.dequant_rows(ra, rs, np.arange(len(rows)))
        B = X.dequant_rows(*X.from_frag(qb, sb, n, k), np.arange(n))
    ref = A @ B.T
    got = c[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= 8e-3 * np.max(np.abs(ref))), float(err.max())
    assert np.linalg.norm(got - ref) <= 3e-3 * np.linalg.norm(ref)
