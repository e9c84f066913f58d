"""GPU parity of mm_fp4 and mm_mxfp8 against the oracle's fp64 GEMM of the same operand bytes.

Bar: fp32 output relative Frobenius error <= 1e-3; bf16 output relative Frobenius error against
the bf16-rounded reference <= 1e-3 and max |C - ref| <= 8e-3 * max |ref|. Small and ragged
shapes compare every element; the Wan-shaped configurations run at full size in the bench's
launch configuration and compare sampled entries (plus corners and ragged tails).
"""
import functools

import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsp
import workloads as W
from oracle import activations as A
from oracle import mxfp8 as X
from oracle import nvfp4 as N
from tests.gpu_util import (REL_FRO_FP4_F32, assert_gemm_bf16, assert_gemm_f32,
                            assert_nvfp4_blocks, check_gemm_outputs, dev_bf16, dev_u8, gather,
                            gelu_rounding_ambiguous, host_bits, host_u8, oracle_linear_entries,
                            oracle_quantize_chunked, sample_entries, say, scalar, tensor_bits)

pytestmark = pytest.mark.gpu
f32 = np.float32


@functools.lru_cache(maxsize=2)
def _oracle_weight(cfg, name):
    """The oracle's (packed, sf, gsf) of a whole generated weight (prequantization)."""
    wb = tensor_bits(cfg, name)
    rg = N.global_sf(wb)[0]
    p, s = oracle_quantize_chunked(wb, rg)
    return p, s, rg


def _rand_nvfp4_operand(rng, rows, k):
    packed = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    rp, cp = N.sf_padded_shape(rows, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:rows, : k // 16] = rng.integers(0, 0x7F, size=(rows, k // 16))   # incl. subnormal scales
    return packed, N.swizzle_128x4(lin)


@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (77, 200, 192), (256, 256, 512), (300, 384, 128),
                                   (513, 130, 256), (64, 1000, 64), (5, 1, 128), (1, 1, 64)])
def test_mm_fp4_random_operands_all_elements(m, n, k):
    say("mm_fp4 random", m, n, k)
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    pa, sa = _rand_nvfp4_operand(rng, m, k)
    pb, sb = _rand_nvfp4_operand(rng, n, k)
    al = f32(rng.uniform(0.01, 2.0))
    ref = N.mm_fp4(pa, sa, pb, sb, al, m, n, k)
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(al))
    t32 = bsp.bsp_mm_fp4(*args, out_dtype=torch.float32)
    t16 = bsp.bsp_mm_fp4(*args, out_dtype=torch.bfloat16)
    # the fp32 result is far inside the 1e-3 budget: the products are exact in fp16
    check_gemm_outputs(t16, t32, ref, f"random {m}x{n}x{k}", f32_tol=REL_FRO_FP4_F32)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4"])
def test_long_k_accumulation(fmt):
    """K = 2^18 (2048 NVFP4 stages, 4096 MXFP8 stages, 512 MXFP8 scale blocks) with ragged M and N:
    the long K loop, its 32-bit per-tile load offsets and the fp32 accumulation against the
    oracle on every element."""
    from oracle import mxfp4 as X4
    m, n, k = 130, 70, 1 << 18
    say("long K", fmt, m, n, k)
    rng = np.random.default_rng(2718)
    if fmt == "nvfp4":
        pa, sa = _rand_nvfp4_operand(rng, m, k)
        pb, sb = _rand_nvfp4_operand(rng, n, k)
        ref = N.mm_fp4(pa, sa, pb, sb, f32(0.5), m, n, k)
        c = bsp.bsp_mm_fp4(dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(0.5), out_dtype=torch.float32)
    elif fmt == "mxfp8":
        qa, sa = _rand_mx_operand(rng, m, k)
        qb, sb = _rand_mx_operand(rng, n, k)
        ref = X.mm_mxfp8(qa, sa, qb, sb, m, n, k)
        c = bsp.bsp_mm_mxfp8(dev_u8(qa), dev_u8(sa), dev_u8(qb), dev_u8(sb), out_dtype=torch.float32)
    else:
        pa, sa = _rand_mxfp4_operand(rng, m, k)
        pb, sb = _rand_mxfp4_operand(rng, n, k)
        ref = X4.mm_mxfp4(pa, sa, pb, sb, f32(1.0), m, n, k)
        c = bsp.bsp_mm_mxfp4(dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), None, torch.float32)
    assert_gemm_f32(c.cpu().numpy().astype(np.float64), ref, f"long K {fmt}")


def test_empty_inputs_are_no_ops():
    """M = 0 (no tokens) through every entry point: no launch, empty outputs, no error."""
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    p, sf = bsp.bsp_nvfp4_quantize(x, scalar(1.0))
    assert p.shape == (0, 256) and sf.numel() == 0
    p2, sf2, g2 = bsp.bsp_nvfp4_quantize_per_token(x)
    assert p2.shape == (0, 256) and g2.numel() == 0
    p3, sf3 = bsp.bsp_nvfp4_quantize_gelu(x, scalar(1.0))
    assert p3.shape == (0, 256)
    q, s8 = bsp.bsp_mxfp8_quantize(x)
    assert q.shape == (0, 512) and s8.shape == (0, 16)
    wb = tensor_bits(1, "W")
    pw, sw, gw, _, _ = bsp.bsp_nvfp4_prequantize_weight(dev_bf16(wb))
    c = bsp.bsp_mm_fp4(p, sf, pw, sw, bsp.bsp_nvfp4_alpha(scalar(1.0), gw))
    assert c.shape == (0, wb.shape[0])
    torch.cuda.synchronize()


def test_mm_fp4_output_stride_and_tiny_config():
    """Tiny NVFP4 linear (128x256x512): quantize both on the GPU, GEMM into a strided output."""
    xb, wb = tensor_bits(1, "X"), tensor_bits(1, "W")
    x, w = dev_bf16(xb), dev_bf16(wb)
    pw, sw, gw, inv, _ = bsp.bsp_nvfp4_prequantize_weight(w)
    one = scalar(1.0)
    px, sx = bsp.bsp_nvfp4_quantize(x, one)
    alpha = bsp.bsp_nvfp4_alpha(one, gw)
    rg = N.global_sf(wb)[0]
    rpx, rsx = N.quantize(xb, f32(1.0))
    rpw, rsw = N.quantize(wb, rg)
    assert np.array_equal(host_u8(px), rpx) and np.array_equal(host_u8(pw), rpw)
    ref = N.mm_fp4(rpx, rsx, rpw, rsw, N.alpha(1.0, rg), 128, 256, 512)
    big = torch.full((128, 300), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = big[:, 8:264]
    bsp.bsp_mm_fp4(px, sx, pw, sw, alpha, out=out)
    c = out.float().cpu().numpy().astype(np.float64)
    check_gemm_outputs(out, bsp.bsp_mm_fp4(px, sx, pw, sw, alpha, out_dtype=torch.float32), ref,
                       "tiny config", f32_tol=REL_FRO_FP4_F32)
    b = big.float().cpu().numpy()
    assert np.all(np.isnan(b[:, :8])) and np.all(np.isnan(b[:, 264:]))   # nothing written outside
    # and the layer output is close to the bf16 product it stands for (sanity of the whole chain)
    full = W.bf16_bits_to_f32(xb).astype(np.float64) @ W.bf16_bits_to_f32(wb).astype(np.float64).T
    assert np.linalg.norm(c - full) / np.linalg.norm(full) < 0.15


def _linear_full_size(x_bits, w_bits, name, seed, gsf_x=1.0):
    """Quantize X (static gsf) and prequantize W on the GPU, GEMM at full size with bf16 and with
    fp32 output; the global scale and sampled rows of the quantized activation against the oracle,
    sampled entries of both GEMM outputs against the oracle's own linear layer on the same bf16 X
    and W."""
    m, k = x_bits.shape
    n = w_bits.shape[0]
    w = dev_bf16(w_bits)
    pw, sw, gw, _, _ = bsp.bsp_nvfp4_prequantize_weight(w)
    del w
    gx = scalar(gsf_x)
    px, sx = bsp.bsp_nvfp4_quantize(dev_bf16(x_bits), gx)
    alpha = bsp.bsp_nvfp4_alpha(gx, gw)
    c = bsp.bsp_mm_fp4(px, sx, pw, sw, alpha)
    c32 = bsp.bsp_mm_fp4(px, sx, pw, sw, alpha, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows, cols = sample_entries(m, n, 3000, seed)
    assert gw.item() == N.global_sf(w_bits)[0]
    ur = np.unique(rows)
    rp, _ = N.quantize(x_bits[ur], f32(gsf_x), layout="linear")
    assert np.array_equal(host_u8(px[torch.from_numpy(ur).cuda()]), rp), "activation bytes differ"
    check_gemm_outputs(c, c32, oracle_linear_entries(x_bits, w_bits, rows, cols, gsf_x), name, rows,
                       cols, f32_tol=REL_FRO_FP4_F32)
    return c


@pytest.mark.parametrize("cfg", [2, 4])
def test_mm_fp4_full_size_linear(cfg):
    xb = tensor_bits(cfg, "X")
    wname = "W" if cfg == 2 else "W3"       # cfg 4: to_q 5120x5120
    say("full-size linear cfg", cfg, xb.shape, wname)
    _linear_full_size(xb, tensor_bits(cfg, wname), f"cfg{cfg} {wname}", seed=cfg)


def _frag_to_row_major(frag: torch.Tensor, rows: int, k: int) -> torch.Tensor:
    """Packed bytes in the fragment layout ([rt, K/64, 1024], lane i + 32 h holding row i's bytes
    16 h .. 16 h + 15 of the step) rearranged on the device into row-major [rows, K/2]."""
    rt = frag.shape[0]
    return frag.view(rt, k // 64, 2, 32, 16).permute(0, 3, 1, 2, 4).reshape(rt * 32, k // 2)[:rows]


@pytest.mark.parametrize("cfg,layout", [(3, "linear"), (4, "linear"), (3, "frag"), (4, "frag")])
def test_ffn_chain_full_size(cfg, layout):
    """The FFN step at full size, X -> quantize -> fc_in -> GELU fused into the quantize of H ->
    fc_out, against the oracle's own chain from the same bf16 X, W, W2 on sampled token rows
    (whole rows: fc_out needs all of H's row): fc_in's bf16 and fp32 outputs, H's quantized bytes
    and fc_out's bf16 and fp32 outputs. layout "frag" runs the same chain with every packed operand
    in the fragment layout (bsp_nvfp4_quantize_frag / _gelu_frag, bsp_mm_fp4_frag), as the bench's
    headline step does."""
    xb, w1b, w2b = tensor_bits(cfg, "X"), tensor_bits(cfg, "W"), tensor_bits(cfg, "W2")
    m, k1, n1, n2 = xb.shape[0], xb.shape[1], w1b.shape[0], w2b.shape[0]
    say("ffn chain cfg", cfg, layout, xb.shape, w1b.shape, w2b.shape)
    one = scalar(1.0)
    if layout == "linear":
        px, sx = bsp.bsp_nvfp4_quantize(dev_bf16(xb), one)
        pw1, sw1, g1, _, _ = bsp.bsp_nvfp4_prequantize_weight(dev_bf16(w1b))
        pw2, sw2, g2, _, _ = bsp.bsp_nvfp4_prequantize_weight(dev_bf16(w2b))
        a1, a2 = bsp.bsp_nvfp4_alpha(one, g1), bsp.bsp_nvfp4_alpha(one, g2)
        y = bsp.bsp_mm_fp4(px, sx, pw1, sw1, a1)
        y32 = bsp.bsp_mm_fp4(px, sx, pw1, sw1, a1, out_dtype=torch.float32)
        ph, sh = bsp.bsp_nvfp4_quantize_gelu(y, one)
        out = bsp.bsp_mm_fp4(ph, sh, pw2, sw2, a2)
        out32 = bsp.bsp_mm_fp4(ph, sh, pw2, sw2, a2, out_dtype=torch.float32)
    else:
        px, sx = bsp.bsp_nvfp4_quantize_frag(dev_bf16(xb), one)
        pw1, sw1, g1, _, _ = bsp.bsp_nvfp4_prequantize_weight_frag(dev_bf16(w1b))
        pw2, sw2, g2, _, _ = bsp.bsp_nvfp4_prequantize_weight_frag(dev_bf16(w2b))
        a1, a2 = bsp.bsp_nvfp4_alpha(one, g1), bsp.bsp_nvfp4_alpha(one, g2)
        y = bsp.bsp_mm_fp4_frag(px, sx, pw1, sw1, m, n1, a1)
        y32 = bsp.bsp_mm_fp4_frag(px, sx, pw1, sw1, m, n1, a1, out_dtype=torch.float32)
        phf, sh = bsp.bsp_nvfp4_quantize_gelu_frag(y, one)
        out = bsp.bsp_mm_fp4_frag(phf, sh, pw2, sw2, m, n2, a2)
        out32 = bsp.bsp_mm_fp4_frag(phf, sh, pw2, sw2, m, n2, a2, out_dtype=torch.float32)
        ph = _frag_to_row_major(phf, m, n1)
    torch.cuda.synchronize()

    rows = np.unique(np.concatenate([np.random.default_rng(cfg).integers(0, m, 12), [0, m - 1]]))
    r = len(rows)
    say("oracle chain: quantize W")
    rpw1, rsw1, rg1 = _oracle_weight(cfg, "W")
    rg2 = N.global_sf(w2b)[0]
    assert g1.item() == rg1 and g2.item() == rg2
    rpx, rsx = N.quantize(xb[rows], f32(1.0))
    say("oracle chain: fc_in rows")
    y_ref = N.mm_fp4(rpx, rsx, rpw1, rsw1, N.alpha(1.0, rg1), r, n1, k1)       # [r, n1] exact
    ri = torch.from_numpy(rows).cuda()
    # fc_in on whole sampled rows, both outputs
    check_gemm_outputs(y[ri], y32[ri], y_ref, f"cfg{cfg} {layout} fc_in", f32_tol=REL_FRO_FP4_F32)
    yb_ref = A.f64_to_bf16_bits(y_ref)
    hb_ref = A.gelu_tanh_bf16_bits(yb_ref)
    # H: every 16-element block must equal the oracle chain's bytes unless one of its values is
    # rounding-ambiguous: its fc_in sum in fp32 rounds to another bf16 than the exact sum does (the
    # fp32 output of the same GEMM shows which), or its GELU lies next to a bf16 boundary; those
    # blocks may differ by one step
    y32_rows = y32[ri].cpu().numpy()
    fc_in_amb = W.f32_to_bf16_bits(y32_rows) != yb_ref
    amb = (fc_in_amb | gelu_rounding_ambiguous(yb_ref)).reshape(r, n1 // 16, 16).any(axis=-1)
    say(f"cfg{cfg} H: fc_in-ambiguous values", int(fc_in_amb.sum()), "blocks with any ambiguity",
        int(amb.sum()), "of", amb.size)
    rp_, cp_ = N.sf_padded_shape(m, n1)
    sh_lin = N.unswizzle_128x4(host_u8(sh).ravel(), rp_, cp_)
    rphl, rshl = N.quantize(hb_ref, f32(1.0), layout="linear")
    frac = assert_nvfp4_blocks(host_u8(ph[ri]), sh_lin[rows], rphl, rshl, ~amb, f"cfg{cfg} {layout} H")
    say(f"cfg{cfg} {layout} H blocks differing from the oracle chain:", frac)
    assert amb.mean() < 0.05 and frac <= amb.mean()
    del y, y32
    cols = np.arange(0, n2, max(1, n2 // 512))
    rph, rsh = N.quantize(hb_ref, f32(1.0))
    rpw2, rsw2 = N.quantize(w2b[cols], rg2)
    ref = N.mm_fp4(rph, rsh, rpw2, rsw2, N.alpha(1.0, rg2), r, len(cols), n1)
    rr, cc = np.repeat(rows, len(cols)), np.tile(cols, r)
    check_gemm_outputs(out, out32, ref.ravel(), f"cfg{cfg} {layout} fc_out", rr, cc,
                       f32_tol=REL_FRO_FP4_F32)


def test_mm_fp4_huge_alpha():
    """alpha = 2^120 (and per-token alphas 2^120 from row scales 2^-60 and a weight scale 2^-60) with
    small operand scales: outputs are finite wherever alpha * sum is and exact zeros stay +-0,
    against the oracle (the f16 operands' 2^-16 is undone on the accumulator, not folded into
    alpha, where 2^136 would overflow)."""
    m, n, k = 96, 160, 256
    rng = np.random.default_rng(120)
    pa = rng.integers(0, 256, size=(m, k // 2)).astype(np.uint8)
    pb = rng.integers(0, 256, size=(n, k // 2)).astype(np.uint8)
    pa[:3] = 0                                     # zero rows of A: zero outputs
    pb[5] = 0x88                                   # a column of -0 codes: zero outputs

    def scales(rows):
        rp, cp = N.sf_padded_shape(rows, k)
        lin = np.zeros((rp, cp), dtype=np.uint8)
        lin[:rows, : k // 16] = rng.integers(1, 0x11, size=(rows, k // 16))   # 2^-9 .. 2^-5
        return N.swizzle_128x4(lin)

    sa, sb = scales(m), scales(n)
    al = f32(2.0 ** 120)
    ref = N.mm_fp4(pa, sa, pb, sb, al, m, n, k)
    assert 1e30 < np.max(np.abs(ref)) < 1e38
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb))
    t16 = bsp.bsp_mm_fp4(*args, scalar(al))
    t32 = bsp.bsp_mm_fp4(*args, scalar(al), out_dtype=torch.float32)
    assert torch.isfinite(t32).all() and torch.isfinite(t16.float()).all()
    assert (t32[:3] == 0).all() and (t32[:, 5] == 0).all()
    check_gemm_outputs(t16, t32, ref, "alpha 2^120", f32_tol=REL_FRO_FP4_F32)
    xg = np.full(m, 2.0 ** -60, dtype=np.float32)
    pt = (*args, torch.from_numpy(xg).cuda(), scalar(2.0 ** -60))
    assert N.alpha_rows(xg, f32(2.0 ** -60))[0] == al
    p16 = bsp.bsp_mm_fp4_per_token(*pt)
    p32 = bsp.bsp_mm_fp4_per_token(*pt, out_dtype=torch.float32)
    assert torch.equal(p32, t32) and torch.equal(p16.view(torch.int16), t16.view(torch.int16))


# ------------------------------------------------------------------------------ per-token scales
@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (77, 200, 192), (300, 384, 512)])
def test_mm_fp4_per_token_random_all_elements(m, n, k):
    say("mm_fp4_per_token random", m, n, k)
    rng = np.random.default_rng(m + 11 * n + k)
    pa, sa = _rand_nvfp4_operand(rng, m, k)
    pb, sb = _rand_nvfp4_operand(rng, n, k)
    xg = (10.0 ** rng.uniform(-2, 3, size=m)).astype(np.float32)
    wg = f32(777.25)
    ref = N.mm_fp4_rowscale(pa, sa, pb, sb, xg, wg, m, n, k)
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), torch.from_numpy(xg).cuda(), scalar(wg))
    t32 = bsp.bsp_mm_fp4_per_token(*args, out_dtype=torch.float32)
    t16 = bsp.bsp_mm_fp4_per_token(*args)
    check_gemm_outputs(t16, t32, ref, f"per-token {m}x{n}x{k}", f32_tol=REL_FRO_FP4_F32)
    # with equal row scales it is the tensor-alpha GEMM, bit for bit
    same = torch.full((m,), 2.5, dtype=torch.float32, device="cuda")
    c1 = bsp.bsp_mm_fp4_per_token(*args[:4], same, scalar(wg), out_dtype=torch.float32)
    c2 = bsp.bsp_mm_fp4(*args[:4], bsp.bsp_nvfp4_alpha(scalar(2.5), scalar(wg)), out_dtype=torch.float32)
    assert torch.equal(c1, c2)


def test_per_token_linear_full_size():
    """Wan-14B to_q (32760x5120x5120) with per-token activation scales: quantize on the GPU, check
    sampled rows of the quantization and sampled entries of the GEMM against the oracle."""
    xb, wb = tensor_bits(4, "X"), tensor_bits(4, "W3")
    m, n, k = xb.shape[0], wb.shape[0], xb.shape[1]
    px, sx, gx = bsp.bsp_nvfp4_quantize_per_token(dev_bf16(xb))
    pw, sw, gw, _, _ = bsp.bsp_nvfp4_prequantize_weight(dev_bf16(wb))
    c = bsp.bsp_mm_fp4_per_token(px, sx, pw, sw, gx, gw)
    c32 = bsp.bsp_mm_fp4_per_token(px, sx, pw, sw, gx, gw, out_dtype=torch.float32)
    rows, cols = sample_entries(m, n, 3000, 77)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    rq, rs, rg = N.quantize_per_token(xb[ur])
    rql, _, _ = N.quantize_per_token(xb[ur], layout="linear")
    assert np.array_equal(host_u8(px[torch.from_numpy(ur).cuda()]), rql)
    assert np.array_equal(gx.cpu().numpy()[ur], rg)
    rgw = N.global_sf(wb)[0]
    assert gw.item() == rgw
    rpw, rsw = N.quantize(wb[uc], rgw)
    base = N.mm_fp4_entries(rq, rs, rpw, rsw, f32(1.0), len(ur), len(uc), k, ri, ci)
    ref = base * N.alpha_rows(rg[ri], rgw).astype(np.float64)
    check_gemm_outputs(c, c32, ref, "cfg4 to_q per-token", rows, cols, f32_tol=REL_FRO_FP4_F32)


# ------------------------------------------------------------------------- layout_8x4 activations
@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (3, 256, 192), (13, 200, 512), (77, 384, 256),
                                   (300, 130, 128)])
def test_mm_fp4_8x4_random_all_elements(m, n, k):
    """A's scales in layout_8x4: every element against the oracle, and bit-identical to the same
    GEMM fed the same scale values in the 128x4 layout."""
    say("mm_fp4_8x4 random", m, n, k)
    rng = np.random.default_rng(m * 13 + n + k)
    pa, sa = _rand_nvfp4_operand(rng, m, k)
    pb, sb = _rand_nvfp4_operand(rng, n, k)
    rp8, cp = N.sf_padded_shape_8x4(m, k)
    sa8 = N.swizzle_8x4(N.unswizzle_128x4(sa, *N.sf_padded_shape(m, k))[:rp8])
    al = f32(0.75)
    ref = N.mm_fp4(pa, sa8, pb, sb, al, m, n, k, a_layout="8x4")
    args8 = (dev_u8(pa), dev_u8(sa8), dev_u8(pb), dev_u8(sb), scalar(al))
    t32 = bsp.bsp_mm_fp4_8x4(*args8, out_dtype=torch.float32)
    t16 = bsp.bsp_mm_fp4_8x4(*args8)
    check_gemm_outputs(t16, t32, ref, f"8x4 {m}x{n}x{k}", f32_tol=REL_FRO_FP4_F32)
    c128 = bsp.bsp_mm_fp4(dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(al), out_dtype=torch.float32)
    assert torch.equal(t32, c128)


@pytest.mark.parametrize("m", [1, 8, 13])
def test_small_m_linear_8x4_chain(m):
    """Decode-sized activations: quantize to layout_8x4 and run against a prequantized Wan-14B
    weight (fc_in 13824x5120), checked element by element against the oracle."""
    xb = tensor_bits(4, "X")[:m]
    wb = tensor_bits(4, "W")
    px, sx = bsp.bsp_nvfp4_quantize_8x4(dev_bf16(xb), scalar(1.0))
    pw, sw, gw, _, _ = bsp.bsp_nvfp4_prequantize_weight(dev_bf16(wb))
    alpha = bsp.bsp_nvfp4_alpha(scalar(1.0), gw)
    c = bsp.bsp_mm_fp4_8x4(px, sx, pw, sw, alpha, out_dtype=torch.float32)
    rpx, rsx = N.quantize(xb, f32(1.0), layout="8x4")
    assert np.array_equal(host_u8(px), rpx) and np.array_equal(host_u8(sx).ravel(), rsx)
    rpw, rsw, rg = _oracle_weight(4, "W")
    assert gw.item() == rg
    ref = N.mm_fp4(rpx, rsx, rpw, rsw, N.alpha(1.0, rg), m, wb.shape[0], wb.shape[1], a_layout="8x4")
    assert_gemm_f32(c.cpu().numpy().astype(np.float64), ref, f"small-M 8x4 m={m}")


# ------------------------------------------------------------------------------------------ MXFP8
def _rand_mx_operand(rng, rows, k):
    q = rng.integers(0, 256, size=(rows, k)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3F                                   # no NaN codes
    s = rng.integers(110, 140, size=(rows, k // 32)).astype(np.uint8)
    return q, s


@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (77, 200, 256), (256, 256, 512), (300, 130, 384),
                                   (130, 300, 1536), (257, 129, 2048), (3, 1, 512), (1, 1, 128)])
def test_mm_mxfp8_random_operands_all_elements(m, n, k):
    say("mm_mxfp8 random", m, n, k)
    rng = np.random.default_rng(m + n + k)
    qa, sa = _rand_mx_operand(rng, m, k)
    qb, sb = _rand_mx_operand(rng, n, k)
    ref = X.mm_mxfp8(qa, sa, qb, sb, m, n, k)
    args = (dev_u8(qa), dev_u8(sa), dev_u8(qb), dev_u8(sb))
    t32 = bsp.bsp_mm_mxfp8(*args, out_dtype=torch.float32)
    t16 = bsp.bsp_mm_mxfp8(*args)
    check_gemm_outputs(t16, t32, ref, f"mx random {m}x{n}x{k}")


def _misaligned_copy(t, offset):
    """A copy of contiguous uint8 tensor t whose data starts `offset` bytes past a 256-byte
    boundary."""
    buf = torch.zeros(t.numel() + 256, dtype=torch.uint8, device=t.device)
    assert buf.data_ptr() % 256 == 0
    v = buf[offset: offset + t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("m,n,k", [(300, 257, 1536), (64, 96, 512)])
def test_mm_mxfp8_scale_paths_agree(m, n, k):
    """With K a multiple of 512 and 16-byte aligned scale matrices the MXFP8 kernel reads the scales
    in blocks of 512 K per row; with scales at a 4-byte (not 16-byte) aligned address it gathers one
    dword per row and stage pair. Same inputs: the same fp32 bits either way, and the oracle's
    values."""
    say("mm_mxfp8 scale paths", m, n, k)
    rng = np.random.default_rng(7 * m + n + k)
    qa, sa = _rand_mx_operand(rng, m, k)
    qb, sb = _rand_mx_operand(rng, n, k)
    ref = X.mm_mxfp8(qa, sa, qb, sb, m, n, k)
    da, dsa, db, dsb = dev_u8(qa), dev_u8(sa), dev_u8(qb), dev_u8(sb)
    assert dsa.data_ptr() % 16 == 0 and dsb.data_ptr() % 16 == 0
    c_blk = bsp.bsp_mm_mxfp8(da, dsa, db, dsb, out_dtype=torch.float32)
    msa, msb = _misaligned_copy(dsa, 4), _misaligned_copy(dsb, 4)
    c_gat = bsp.bsp_mm_mxfp8(da, msa, db, msb, out_dtype=torch.float32)
    assert torch.equal(c_blk.view(torch.int32), c_gat.view(torch.int32))
    assert_gemm_f32(c_blk.cpu().numpy().astype(np.float64), ref, f"mx scale paths {m}x{n}x{k}")


def test_mm_mxfp8_full_size():
    xb, wb = tensor_bits(5, "X"), tensor_bits(5, "W")
    qx, sx = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
    qw, sw = bsp.bsp_mxfp8_quantize(dev_bf16(wb))      # online weight conversion
    c = bsp.bsp_mm_mxfp8(qx, sx, qw, sw)
    c32 = bsp.bsp_mm_mxfp8(qx, sx, qw, sw, out_dtype=torch.float32)
    m, n, k = xb.shape[0], wb.shape[0], xb.shape[1]
    rows, cols = sample_entries(m, n, 3000, 5)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    rq, rs = X.quantize(xb[ur])
    assert np.array_equal(host_u8(qx[torch.from_numpy(ur).cuda()]), rq)
    rqw, rsw = X.quantize(wb[uc])
    ref = X.mm_mxfp8_entries(rq, rs, rqw, rsw, ri, ci)
    check_gemm_outputs(c, c32, ref, "cfg5 mxfp8", rows, cols)


# ------------------------------------------------------------------------------------------ MXFP4
def _rand_mxfp4_operand(rng, rows, k):
    from oracle import mxfp4 as X4
    packed = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    rp, cp = X4.sf_padded_shape(rows, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:rows, : k // 32] = rng.integers(110, 140, size=(rows, k // 32))
    return packed, N.swizzle_128x4(lin)


@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (77, 200, 256), (256, 256, 512), (300, 130, 384),
                                   (513, 384, 640), (3, 1, 256), (1, 1, 128)])
def test_mm_mxfp4_random_operands_all_elements(m, n, k):
    from oracle import mxfp4 as X4
    say("mm_mxfp4 random", m, n, k)
    rng = np.random.default_rng(m * 5 + n + k)
    pa, sa = _rand_mxfp4_operand(rng, m, k)
    pb, sb = _rand_mxfp4_operand(rng, n, k)
    al = f32(0.625)
    ref = X4.mm_mxfp4(pa, sa, pb, sb, al, m, n, k)
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(al))
    t32 = bsp.bsp_mm_mxfp4(*args, out_dtype=torch.float32)
    t16 = bsp.bsp_mm_mxfp4(*args)
    check_gemm_outputs(t16, t32, ref, f"mxfp4 random {m}x{n}x{k}")
    c1 = bsp.bsp_mm_mxfp4(dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), None, torch.float32)
    assert_gemm_f32(c1.cpu().numpy().astype(np.float64), ref / float(al), "alpha=None")


def test_mm_mxfp4_full_size():
    from oracle import mxfp4 as X4
    xb, wb = tensor_bits(4, "X"), tensor_bits(4, "W")      # Wan-14B fc_in shape
    px, sx = bsp.bsp_mxfp4_quantize(dev_bf16(xb))
    pw, sw = bsp.bsp_mxfp4_quantize(dev_bf16(wb))
    c = bsp.bsp_mm_mxfp4(px, sx, pw, sw)
    c32 = bsp.bsp_mm_mxfp4(px, sx, pw, sw, out_dtype=torch.float32)
    m, n, k = xb.shape[0], wb.shape[0], xb.shape[1]
    rows, cols = sample_entries(m, n, 3000, 41)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    rp, _ = X4.quantize(xb[ur], layout="linear")
    assert np.array_equal(host_u8(px[torch.from_numpy(ur).cuda()]), rp)
    rpx, rsx = X4.quantize(xb[ur])
    rpw, rsw = X4.quantize(wb[uc])
    ref = X4.mm_mxfp4_entries(rpx, rsx, rpw, rsw, 1.0, len(ur), len(uc), k, ri, ci)
    check_gemm_outputs(c, c32, ref, "cfg4 fc_in mxfp4", rows, cols)


# ------------------------------------------------------------------------------------ bias
def _ref_plus_bias_bf16(ref, bias_bits):
    """The pages' result: the oracle's product rounded to bf16, plus the bf16 bias (bf16 add)."""
    from oracle import linear as L
    return W.bf16_bits_to_f32(L.add_bias_bf16(A.f64_to_bf16_bits(ref), bias_bits)).astype(np.float64)


def _rand_bias(rng, n, scale):
    """bf16 bits and fp32 values of a bias [N] of about the outputs' size, with some exact zeros."""
    v = rng.normal(0.0, scale, size=n).astype(np.float32)
    v[:: 7] = 0.0
    bits = W.f32_to_bf16_bits(v)
    return bits, W.bf16_bits_to_f32(bits)


@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (77, 200, 192), (256, 256, 512), (300, 130, 128)])
def test_mm_fp4_bias_random(m, n, k):
    """bsp_mm_fp4_bias = the bf16 output of bsp_mm_fp4 plus the bf16 bias (bit-exact against
    torch's bf16 add of the two, the pages' out + bias), and within the GEMM tolerance of the
    oracle's exact product plus bias."""
    say("mm_fp4_bias random", m, n, k)
    rng = np.random.default_rng(m * 11 + n + k)
    pa, sa = _rand_nvfp4_operand(rng, m, k)
    pb, sb = _rand_nvfp4_operand(rng, n, k)
    al = f32(rng.uniform(0.01, 2.0))
    ref = N.mm_fp4(pa, sa, pb, sb, al, m, n, k)
    bbits, bf = _rand_bias(rng, n, float(np.std(ref)) + 1e-30)
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(al))
    bias = dev_bf16(bbits)
    t16 = bsp.bsp_mm_fp4(*args)
    tb16 = bsp.bsp_mm_fp4_bias(*args, bias)
    assert torch.equal(tb16.view(torch.int16), (t16.float() + bias.float()).bfloat16().view(torch.int16))
    t32 = bsp.bsp_mm_fp4(*args, out_dtype=torch.float32)
    # the product's own bf16 rounding decides the sum, so ties are those of the product's fp32 value
    assert_gemm_bf16(tb16.float().cpu().numpy().astype(np.float64), _ref_plus_bias_bf16(ref, bbits),
                     t32.cpu().numpy(), f"bias {m}x{n}x{k}")
    tb32 = bsp.bsp_mm_fp4_bias(*args, bias, out_dtype=torch.float32)
    assert np.array_equal(tb32.cpu().numpy(), (t32.cpu().numpy() + bf).astype(np.float32))


def test_mm_fp4_bias_full_size_fc_in():
    """Wan-14B fc_in shape in the bench's launch configuration, with a bias: every element against
    the no-bias output plus the bias (bf16 add on the device), sampled entries against the oracle."""
    hb, wb = tensor_bits(4, "X"), tensor_bits(4, "W")
    pw, sw, gw, _, _ = bsp.bsp_nvfp4_prequantize_weight(dev_bf16(wb))
    px, sx = bsp.bsp_nvfp4_quantize(dev_bf16(hb), scalar(1.0))
    alpha = bsp.bsp_nvfp4_alpha(scalar(1.0), gw)
    m, n, k = hb.shape[0], wb.shape[0], hb.shape[1]
    rng = np.random.default_rng(404)
    bbits, bf = _rand_bias(rng, n, 0.5)
    bias = dev_bf16(bbits)
    c = bsp.bsp_mm_fp4(px, sx, pw, sw, alpha)
    cb = bsp.bsp_mm_fp4_bias(px, sx, pw, sw, alpha, bias)
    assert torch.equal(cb.view(torch.int16), (c.float() + bias.float()).bfloat16().view(torch.int16))
    del c
    c32 = bsp.bsp_mm_fp4(px, sx, pw, sw, alpha, out_dtype=torch.float32)
    rows, cols = sample_entries(m, n, 2000, 404)
    ref = oracle_linear_entries(hb, wb, rows, cols)
    assert_gemm_bf16(gather(cb, rows, cols), _ref_plus_bias_bf16(ref, bbits[cols]),
                     gather(c32, rows, cols).astype(np.float32), "cfg4 fc_in + bias")


@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (77, 200, 256), (300, 130, 384), (129, 260, 1024)])
def test_mm_mxfp8_bias_random(m, n, k):
    """bsp_mm_mxfp8_bias: fp32 output = fp32 product + fp32 bias exactly; bf16 output = its one
    nearest-even rounding; within tolerance of the oracle's exact product plus bias."""
    from oracle import linear as L
    say("mm_mxfp8_bias random", m, n, k)
    rng = np.random.default_rng(m + 3 * n + k)
    qa, sa = _rand_mx_operand(rng, m, k)
    qb, sb = _rand_mx_operand(rng, n, k)
    ref = X.mm_mxfp8(qa, sa, qb, sb, m, n, k)
    bf = rng.normal(0.0, float(np.std(ref)) + 1e-30, size=n).astype(np.float32)
    bias = torch.from_numpy(bf).cuda()
    args = (dev_u8(qa), dev_u8(sa), dev_u8(qb), dev_u8(sb))
    t32 = bsp.bsp_mm_mxfp8(*args, out_dtype=torch.float32)
    tb32 = bsp.bsp_mm_mxfp8_bias(*args, bias, out_dtype=torch.float32)
    assert np.array_equal(tb32.cpu().numpy(), (t32.cpu().numpy() + bf).astype(np.float32))
    tb16 = bsp.bsp_mm_mxfp8_bias(*args, bias)
    check_gemm_outputs(tb16, tb32, L.gemm_plus_bias(ref, bf), f"mxfp8 bias {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(77, 200, 256), (256, 256, 512)])
def test_mm_mxfp4_bias_random(m, n, k):
    from oracle import linear as L
    from oracle import mxfp4 as X4
    say("mm_mxfp4_bias random", m, n, k)
    rng = np.random.default_rng(m * 3 + n + k)
    pa, sa = _rand_mxfp4_operand(rng, m, k)
    pb, sb = _rand_mxfp4_operand(rng, n, k)
    al = f32(0.375)
    ref = X4.mm_mxfp4(pa, sa, pb, sb, al, m, n, k)
    bbits, bf = _rand_bias(rng, n, float(np.std(ref)) + 1e-30)
    args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb))
    bias = dev_bf16(bbits)
    t16 = bsp.bsp_mm_mxfp4(*args, scalar(al))
    tb16 = bsp.bsp_mm_mxfp4_bias(*args, bias, scalar(al))
    assert torch.equal(tb16.view(torch.int16), (t16.float() + bias.float()).bfloat16().view(torch.int16))
    t32 = bsp.bsp_mm_mxfp4(*args, scalar(al), out_dtype=torch.float32)
    assert_gemm_bf16(tb16.float().cpu().numpy().astype(np.float64), _ref_plus_bias_bf16(ref, bbits),
                     t32.cpu().numpy(), f"mxfp4 bias {m}x{n}x{k}")


# ------------------------------------------------------------------- epilogue paths agree
def _strided_out(m, n, ldc, dtype):
    buf = torch.full((m, ldc), float("nan"), dtype=dtype, device="cuda")
    return buf, buf[:, :n]


@pytest.mark.parametrize("kind", ["fp4", "fp4_bias", "mxfp8", "mxfp8_bias", "mxfp4"])
def test_staged_and_direct_epilogues_agree(kind):
    """Whole 256x256 tiles with 16-byte aligned output rows leave through the LDS-staged epilogue,
    others through the direct one: the same product written with row stride N (staged) and with
    an odd row stride (direct) must be bit-identical, and the padding columns untouched."""
    say("epilogue paths", kind)
    m, n, k = 512, 768, 256
    rng = np.random.default_rng(2024)
    if kind.startswith("fp4"):
        pa, sa = _rand_nvfp4_operand(rng, m, k)
        pb, sb = _rand_nvfp4_operand(rng, n, k)
        args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb), scalar(0.75))
    elif kind.startswith("mxfp8"):
        qa, sa = _rand_mx_operand(rng, m, k)
        qb, sb = _rand_mx_operand(rng, n, k)
        args = (dev_u8(qa), dev_u8(sa), dev_u8(qb), dev_u8(sb))
    else:
        pa, sa = _rand_mxfp4_operand(rng, m, k)
        pb, sb = _rand_mxfp4_operand(rng, n, k)
        args = (dev_u8(pa), dev_u8(sa), dev_u8(pb), dev_u8(sb))
    bias16 = dev_bf16(_rand_bias(rng, n, 4.0)[0])
    bias32 = torch.from_numpy(rng.normal(0, 4.0, size=n).astype(np.float32)).cuda()

    def run(out):
        if kind == "fp4":
            return bsp.bsp_mm_fp4(*args, out=out)
        if kind == "fp4_bias":
            return bsp.bsp_mm_fp4_bias(*args, bias16, out=out)
        if kind == "mxfp8":
            return bsp.bsp_mm_mxfp8(*args, out=out)
        if kind == "mxfp8_bias":
            return bsp.bsp_mm_mxfp8_bias(*args, bias32, out=out)
        return bsp.bsp_mm_mxfp4(*args, scalar(0.5), out=out)

    staged = run(torch.empty((m, n), dtype=torch.bfloat16, device="cuda"))
    buf, view = _strided_out(m, n, n + 3, torch.bfloat16)
    direct = run(view)
    assert np.array_equal(host_bits(staged), host_bits(direct))
    assert torch.isnan(buf[:, n:].float()).all()
