"""Pins for the NVFP4 oracle: hand-worked blocks, closed forms, invariants and brute force."""
import itertools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import nvfp4 as N
from tests.conftest import golden_lines

f32 = np.float32


def bits(vals):
    return W.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


# ------------------------------------------------------------------------------------- blocks
def test_hand_worked_blocks():
    for line in golden_lines("nvfp4_blocks.txt"):
        head, s_hex, packed_hex = (p.split() for p in line.split("|"))
        g = f32(head[1])
        x = np.array([float(v) for v in head[2:]], dtype=np.float32)
        assert x.size == 16
        xb = bits(x)
        assert np.array_equal(W.bf16_bits_to_f32(xb), x), "fixture inputs must be bf16-exact"
        packed, sf = N.quantize(xb[None, :], g, layout="linear")
        assert int(sf[0, 0]) == int(s_hex[0], 16), head[0]
        assert [int(b) for b in packed[0]] == [int(h, 16) for h in packed_hex], head[0]


def test_sixth_constant():
    assert N.C_SIXTH.view(np.uint32) == 0x3E2AAAAB


def test_global_sf_cases():
    for amax, gsf in (l.split() for l in golden_lines("global_sf_cases.txt")):
        w = np.zeros((4, 16), dtype=np.float32)
        w[1, 3] = -float(amax)
        w[2, 5] = float(amax) / 2
        g, inv, a = N.global_sf(bits(w))
        assert a == f32(amax)
        assert g == f32(gsf)
        assert inv == f32(1.0) / f32(gsf)


def test_global_sf_split_between_pages_is_pinned():
    # amax 3: FastVideo's one division gives 896 exactly (golden); SGLang's decode scale
    # fl32(3/2688) and its reciprocal give 0x445FFFFF (hand-worked in global_sf_cases.txt)
    w = np.array([[3.0, -1.0]], dtype=np.float32)
    g, _, a = N.global_sf(bits(w))
    two_step = f32(f32(1.0) / f32(f32(3.0) / f32(2688.0)))
    assert two_step.view(np.uint32) == 0x445FFFFF
    assert g == f32(896.0) and g != two_step


def test_global_sf_nan_inf():
    w = np.array([[1.0, np.nan, -3.0, 2.0]], dtype=np.float32)
    g, _, a = N.global_sf(bits(w))
    assert a == 3.0 and g == f32(896.0)
    w = np.array([[1.0, -np.inf]], dtype=np.float32)
    _, _, a = N.global_sf(bits(w))
    assert a == N.BF16_MAX


def test_global_scale_block_gets_448():
    # the block holding the tensor amax gets scale fl32(g * fl32(amax/6)) ~= 448 -> byte 0x7E
    for seed in range(5):
        w = W.small_case(64, 256, seed, std=0.02)
        g, _, amax = N.global_sf(w)
        _, sf = N.quantize(w, g, layout="linear")
        xf = W.bf16_bits_to_f32(w).reshape(64, 16, 16)
        blk = np.argwhere(np.max(np.abs(xf), axis=-1) == amax)[0]
        assert sf[blk[0], blk[1]] == 0x7E


def test_alpha():
    assert N.alpha(1.0, 43008.0) == f32(1.0) / f32(43008.0)
    assert N.alpha(2.0, 3.0) == f32(1.0) / f32(6.0)
    # hand-worked cases where the FastVideo nvfp4_qat_config.py form 1/(x*w) and the FastVideo
    # nvfp4_config.py form (1/w)/x round differently (golden file); the oracle takes the first
    for line in golden_lines("alpha_cases.txt"):
        x, w, bits_hex = line.split()
        want = np.array([int(bits_hex, 16)], dtype=np.uint32).view(np.float32)[0]
        assert N.alpha(float(x), float(w)) == want, line
    # the golden set discriminates: the other page's form misses at least one case
    other = [f32(f32(f32(1.0) / f32(float(w))) / f32(float(x))) for x, w, _ in
             (l.split() for l in golden_lines("alpha_cases.txt"))]
    assert any(o != N.alpha(float(x), float(w)) for o, (x, w, _) in
               zip(other, (l.split() for l in golden_lines("alpha_cases.txt"))))
    # static x_gsf = 1 makes alpha the stored fp32 1/w_gsf bit for bit
    for g in (2688.0, 123456.78, 0.37):
        assert N.alpha(1.0, g) == f32(1.0) / f32(g)


# ---------------------------------------------------------------------------------- invariants
def _blocks(x_bits):
    m, k = x_bits.shape
    return W.bf16_bits_to_f32(x_bits).reshape(m, k // 16, 16)


def test_max_code_is_six_in_normal_unsaturated_blocks():
    x = W.small_case(128, 1024, 11, outlier_frac=0.02)
    for g in (f32(1.0), N.global_sf(x)[0]):
        packed, sf = N.quantize(x, g, layout="linear")
        codes = N.unpack_nibbles(packed).reshape(128, 64, 16)
        sd = F.e4m3_decode(sf)
        a = np.max(np.abs(_blocks(x)), axis=-1)
        normal = (sd >= 2.0 ** -6) & (a.astype(np.float64) * g / 6 < 448)
        assert normal.sum() > 1000
        assert np.all(np.max(codes[normal] & 7, axis=-1) == 7)


def test_zero_blocks_and_saturation():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 16:] = np.linspace(-3e4, 3e4, 16)
    packed, sf = N.quantize(bits(x), f32(1.0), layout="linear")
    assert np.all(packed[0] == 0) and np.all(sf[0] == 0)
    assert sf[1, 1] == 0x7E and sf[1, 0] == 0
    codes = N.unpack_nibbles(packed[1:, 8:])[0]
    assert codes[0] == 0xF and codes[-1] == 0x7


def test_quantization_error_within_half_step():
    # every dequantized element is within half an e2m1 step of x * r (or saturated at 6)
    x = W.small_case(64, 512, 5, outlier_frac=0.05)
    g = N.global_sf(x)[0]
    packed, sf = N.quantize(x, g, layout="linear")
    xf = _blocks(x).astype(np.float64)
    sd = F.e4m3_decode(sf)
    r = np.where(sd == 0, 0.0, (g / np.where(sd == 0, 1, sd).astype(np.float32)).astype(np.float32))
    v = (xf * r[..., None]).astype(np.float32).astype(np.float64)
    q = F.e2m1_decode(N.unpack_nibbles(packed)).reshape(v.shape)
    a = np.abs(v)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    ok = (np.abs(q - v) <= half + 1e-12) | ((a > 6) & (np.abs(q) == 6))
    assert ok.all()
    # and the scale is the e4m3 neighbour of amax*g/6
    s = (g * (np.max(np.abs(_blocks(x)), -1) * N.C_SIXTH).astype(np.float32)).astype(np.float64)
    rel = np.abs(sd - s) / np.maximum(s, 1e-30)
    assert np.all((rel <= 2.0 ** -4 + 1e-9) | (s < 2.0 ** -6))


def test_idempotent_at_unit_global_scale():
    # Q(D(Q(x))) == Q(x) for blocks with normal scales when g = 1
    x = W.small_case(64, 512, 6)
    p1, s1 = N.quantize(x, f32(1.0), layout="linear")
    d = N.dequant_rows(p1, N.swizzle_128x4(np.pad(s1, ((0, 64), (0, 0)))), np.arange(64), 64, 512)
    p2, s2 = N.quantize(bits(d.astype(np.float32)), f32(1.0), layout="linear")
    normal = F.e4m3_decode(s1) >= 2.0 ** -6
    assert normal.all()
    assert np.array_equal(s1, s2) and np.array_equal(p1, p2)
    assert np.array_equal(W.bf16_bits_to_f32(bits(d.astype(np.float32))), d.astype(np.float32))


def test_static_unit_scale_closed_form():
    x = W.small_case(16, 256, 8)
    _, sf = N.quantize(x, f32(1.0), layout="linear")
    a = np.max(np.abs(_blocks(x)), axis=-1).astype(np.float32)
    assert np.array_equal(sf, F.e4m3_encode((a * N.C_SIXTH).astype(np.float32)))


def test_padding_and_shape_contract():
    m, k = 200, 96
    x = W.small_case(m, k, 9)
    packed, sf = N.quantize(x, f32(1.0))
    assert packed.shape == (m, (k + 1) // 2)
    rp, cp = N.sf_padded_shape(m, k)
    assert (rp, cp) == (256, 8) and sf.size == rp * cp
    lin = N.unswizzle_128x4(sf, rp, cp)
    assert np.all(lin[m:] == 0) and np.all(lin[:, k // 16:] == 0)
    # quantize(X) == quantize(pad(X)) narrowed (rows padded with zeros to the 128 tile)
    xp = np.zeros((rp, k), dtype=np.uint16)
    xp[:m] = x
    p2, s2 = N.quantize(xp, f32(1.0))
    assert np.array_equal(p2[:m], packed) and np.array_equal(s2, sf)


def test_row_separability():
    a = W.small_case(256, 128, 10)
    b = W.small_case(128, 128, 11)
    g = f32(37.5)
    pa, sa = N.quantize(a, g)
    pb, sb = N.quantize(b, g)
    pc, sc = N.quantize(np.concatenate([a, b]), g)
    assert np.array_equal(pc, np.concatenate([pa, pb]))
    assert np.array_equal(sc, np.concatenate([sa, sb]))   # split at a multiple of 128 rows
    _, la = N.quantize(a[:77], g, layout="linear")
    _, lc = N.quantize(a, g, layout="linear")
    assert np.array_equal(la, lc[:77])


# ---------------------------------------------------------------------------------- 128x4 layout
def test_sf_offsets_golden():
    for r, c, off in (map(int, l.split()) for l in golden_lines("sf_offsets_128x4.txt")):
        assert int(N.sf_offset(r, c, 8)) == off


def test_sf_layout_bijection_and_tiles():
    rp, cp = 384, 12
    r, c = np.meshgrid(np.arange(rp), np.arange(cp), indexing="ij")
    off = N.sf_offset(r, c, cp)
    assert np.array_equal(np.sort(off.ravel()), np.arange(rp * cp))
    # each 128x4 tile is one contiguous 512-byte run; a row's 4 scales are 4 contiguous bytes
    for tr, tc in itertools.product(range(3), range(3)):
        t = off[tr * 128:(tr + 1) * 128, tc * 4:(tc + 1) * 4]
        assert t.min() == (tr * 3 + tc) * 512 and t.max() == t.min() + 511
        assert np.all(np.diff(t, axis=1) == 1)
    lin = np.arange(rp * cp, dtype=np.int64).reshape(rp, cp).astype(np.uint8)
    assert np.array_equal(N.unswizzle_128x4(N.swizzle_128x4(lin), rp, cp), lin)


# ---------------------------------------------------------------------------------- GEMM
def _rand_operand(rng, rows, k):
    codes = rng.integers(0, 16, size=(rows, k)).astype(np.uint8)
    packed = N.pack_nibbles(codes)
    rp, cp = N.sf_padded_shape(rows, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    # scales over the finite e4m3 range (no NaN codes), including subnormals
    lin[:rows, :k // 16] = rng.integers(0, 0x7F, size=(rows, k // 16))
    return codes, lin, packed, N.swizzle_128x4(lin)


def test_mm_fp4_brute_force_loops():
    rng = np.random.default_rng(3)
    m, n, k = 5, 7, 48
    ca, la, pa, sa = _rand_operand(rng, m, k)
    cb, lb, pb, sb = _rand_operand(rng, n, k)
    e2 = F.e2m1_decode_table()
    e4 = F.e4m3_decode_table()
    al = f32(0.37)
    ref = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                acc += e2[ca[i, kk]] * e4[la[i, kk // 16]] * e2[cb[j, kk]] * e4[lb[j, kk // 16]]
            ref[i, j] = float(al) * acc
    got = N.mm_fp4(pa, sa, pb, sb, al, m, n, k)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    rows = np.array([0, 4, 2, 2])
    cols = np.array([6, 0, 3, 3])
    assert np.allclose(N.mm_fp4_entries(pa, sa, pb, sb, al, m, n, k, rows, cols),
                       ref[rows, cols], rtol=1e-12)


def test_mm_fp4_closed_forms():
    k = 64
    ones = np.full((1, k), 2, dtype=np.uint8)          # e2m1 1.0
    p = N.pack_nibbles(ones)
    lin = np.zeros((128, 4), dtype=np.uint8)
    lin[0, :] = 0x38                                    # scale 1.0
    s1 = N.swizzle_128x4(lin)
    assert N.mm_fp4(p, s1, p, s1, 1.0, 1, 1, k)[0, 0] == 64.0
    lin2 = lin.copy()
    lin2[0, 2] = 0x40                                   # one block with scale 2
    s2 = N.swizzle_128x4(lin2)
    assert N.mm_fp4(p, s1, p, s2, 0.5, 1, 1, k)[0, 0] == 0.5 * (48 + 32)


def test_mm_fp4_operand_orientation():
    # A row i holds 1.0 only at k = i; C[i, j] must then be B[j, i] (catches a transposed operand)
    rng = np.random.default_rng(4)
    m, n, k = 16, 3, 32
    codes = np.zeros((m, k), dtype=np.uint8)
    codes[np.arange(m), np.arange(m)] = 2
    lin = np.zeros((128, 4), dtype=np.uint8)
    lin[:m, :2] = 0x38
    cb, lb, pb, sb = _rand_operand(rng, n, k)
    c = N.mm_fp4(N.pack_nibbles(codes), N.swizzle_128x4(lin), pb, sb, 1.0, m, n, k)
    bdeq = N.dequant_rows(pb, sb, np.arange(n), n, k)
    assert np.array_equal(c, bdeq[:, :m].T)


def test_mm_fp4_equals_torch_fp64_of_dequantized():
    x = W.small_case(96, 256, 12, outlier_frac=0.02)
    w = W.small_case(160, 256, 13, std=0.02)
    gw = N.global_sf(w)[0]
    pa, sa = N.quantize(x, f32(1.0))
    pb, sb = N.quantize(w, gw)
    al = N.alpha(1.0, gw)
    got = N.mm_fp4(pa, sa, pb, sb, al, 96, 160, 256)
    A = torch.from_numpy(N.dequant_rows(pa, sa, np.arange(96), 96, 256, gsf=1.0))
    B = torch.from_numpy(N.dequant_rows(pb, sb, np.arange(160), 160, 256, gsf=gw))
    ref = (A @ B.T).numpy()
    # equal up to alpha's fp32 rounding (relative 2^-24) and summation order
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))
    # and NVFP4 is a reasonable approximation of the bf16 product (sanity of the whole chain)
    X = torch.from_numpy(W.bf16_bits_to_f32(x).astype(np.float64))
    Wt = torch.from_numpy(W.bf16_bits_to_f32(w).astype(np.float64))
    full = (X @ Wt.T).numpy()
    assert np.linalg.norm(got - full) / np.linalg.norm(full) < 0.15


def test_dequantized_products_fit_bf16():
    # every e2m1 value times every e4m3 scale is exactly representable in bf16 and fp16
    e2 = F.e2m1_decode_table()
    e4 = F.e4m3_decode_table()[:0x7F]
    prod = np.outer(e2, e4).ravel().astype(np.float32)
    assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(prod)), prod)
    assert np.array_equal(prod.astype(np.float16).astype(np.float32), prod)


def test_k_must_be_multiple_of_16():
    with pytest.raises(ValueError):
        N.quantize(np.zeros((2, 24), dtype=np.uint16), f32(1.0))


# ---------------------------------------------------------------------- per-token activation scales
def test_per_token_is_scale_invariant_row_by_row():
    """Rows that are power-of-two multiples of one row quantize to identical codes and scale bytes,
    and their per-row encode scales differ by exactly that power of two: the scale is per row (a
    shared tensor scale would give different bytes) and follows 2688/amax row by row."""
    base = W.small_case(1, 256, 21, outlier_frac=0.05)
    exps = np.array([0, 3, -7, 12, -20, 1], dtype=np.int64)
    xf = W.bf16_bits_to_f32(base)[0][None, :] * (2.0 ** exps[:, None]).astype(np.float32)
    xb = W.f32_to_bf16_bits(xf)
    assert np.array_equal(W.bf16_bits_to_f32(xb), xf)        # the scaling is exact in bf16
    packed, sf, g = N.quantize_per_token(xb, layout="linear")
    for r in range(1, len(exps)):
        assert np.array_equal(packed[r], packed[0]) and np.array_equal(sf[r], sf[0])
        assert g[r] == np.float32(g[0] * np.float32(2.0 ** -int(exps[r])))
    # a per-tensor scale quantizes the small rows differently
    gp = N.global_sf(xb)[0]
    _, sf_t = N.quantize(xb, gp, layout="linear")
    assert not np.array_equal(sf_t[4], sf[4])


def test_per_token_row_max_block_gets_448_and_zero_row():
    xb = W.small_case(9, 512, 5, outlier_frac=0.02).copy()
    xb[3] = 0                                                  # an all-zero token
    packed, sf, g = N.quantize_per_token(xb, layout="linear")
    assert g[3] == np.float32(1.0) and not sf[3].any() and not packed[3].any()
    xf = W.bf16_bits_to_f32(xb).reshape(9, 32, 16)
    for r in range(9):
        if r == 3:
            continue
        amax = np.max(np.abs(xf[r]))
        assert g[r] == np.float32(np.float32(2688.0) / amax)
        blk = np.argwhere(np.max(np.abs(xf[r]), axis=-1) == amax)[0][0]
        assert sf[r, blk] == 0x7E


def test_per_token_single_row_reduces_to_tensor_scale():
    xb = W.small_case(1, 1024, 8)
    p1, s1, g1 = N.quantize_per_token(xb)
    g = N.global_sf(xb)[0]
    p2, s2 = N.quantize(xb, g)
    assert g1[0] == g and np.array_equal(p1, p2) and np.array_equal(s1, s2)


def test_mm_fp4_rowscale_brute_force_and_alpha_rows():
    rng = np.random.default_rng(31)
    m, n, k = 4, 6, 32
    ca, la, pa, sa = _rand_operand(rng, m, k)
    cb, lb, pb, sb = _rand_operand(rng, n, k)
    e2 = F.e2m1_decode_table()
    e4 = F.e4m3_decode_table()
    xg = np.array([1.0, 0.37, 2688.0 / 3.0, 1e-3], dtype=np.float32)
    wg = np.float32(512.5)
    ar = N.alpha_rows(xg, wg)
    for i in range(m):
        assert ar[i] == N.alpha(xg[i], wg)
    ref = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                acc += e2[ca[i, kk]] * e4[la[i, kk // 16]] * e2[cb[j, kk]] * e4[lb[j, kk // 16]]
            ref[i, j] = float(ar[i]) * acc
    got = N.mm_fp4_rowscale(pa, sa, pb, sb, xg, wg, m, n, k)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)


def test_per_token_linear_approximates_the_bf16_product():
    """Per-token activation scales + a tensor-scaled weight reconstruct X W^T to NVFP4 accuracy."""
    xb = W.small_case(64, 256, 2, outlier_frac=0.02)
    wb = W.small_case(32, 256, 3, std=0.02)
    px, sx, gx = N.quantize_per_token(xb)
    gw = N.global_sf(wb)[0]
    pw, sw = N.quantize(wb, gw)
    c = N.mm_fp4_rowscale(px, sx, pw, sw, gx, gw, 64, 32, 256)
    full = W.bf16_bits_to_f32(xb).astype(np.float64) @ W.bf16_bits_to_f32(wb).astype(np.float64).T
    assert np.linalg.norm(c - full) / np.linalg.norm(full) < 0.15


# ---------------------------------------------------------------- layout_8x4 and the 4over6 scale
def test_sf_offsets_8x4_golden():
    for line in golden_lines("sf_offsets_8x4.txt"):
        r, c, off = (int(v) for v in line.split())
        assert N.sf_offset_8x4(r, c, 8) == off


def test_sf_layout_8x4_bijection_and_tiles():
    rp, cp = N.sf_padded_shape_8x4(37, 16 * 10)
    assert (rp, cp) == (40, 12)
    r, c = np.meshgrid(np.arange(rp), np.arange(cp), indexing="ij")
    off = N.sf_offset_8x4(r, c, cp)
    assert np.array_equal(np.sort(off.ravel()), np.arange(rp * cp))
    # each 32-byte tile holds exactly one 8-row x 4-column block
    for t in range(rp * cp // 32):
        cells = np.argwhere((off >= 32 * t) & (off < 32 * t + 32))
        assert len(cells) == 32
        assert len(np.unique(cells[:, 0] // 8)) == 1 and len(np.unique(cells[:, 1] // 4)) == 1
    lin = np.random.default_rng(0).integers(0, 256, (rp, cp)).astype(np.uint8)
    assert np.array_equal(N.unswizzle_8x4(N.swizzle_8x4(lin), rp, cp), lin)


def test_quantize_8x4_same_scales_as_128x4_and_padding():
    xb = W.small_case(13, 80, 4)
    p1, s1 = N.quantize(xb, f32(2.0), layout="8x4")
    p2, s2 = N.quantize(xb, f32(2.0), layout="128x4")
    assert np.array_equal(p1, p2)
    rp, cp = N.sf_padded_shape_8x4(13, 80)
    assert s1.size == rp * cp == 16 * 8
    lin8 = N.unswizzle_8x4(s1, rp, cp)
    lin128 = N.unswizzle_128x4(s2, *N.sf_padded_shape(13, 80))
    assert np.array_equal(lin8, lin128[:rp])
    assert not lin8[13:].any() and not lin8[:, 5:].any()


def test_mm_fp4_with_8x4_activation_scales():
    rng = np.random.default_rng(12)
    m, n, k = 11, 20, 128
    ca, la, pa, sa = _rand_operand(rng, m, k)
    _, _, pb, sb = _rand_operand(rng, n, k)
    rp8, cp = N.sf_padded_shape_8x4(m, k)
    lin = N.unswizzle_128x4(sa, *N.sf_padded_shape(m, k))[:rp8]
    sa8 = N.swizzle_8x4(lin)
    c128 = N.mm_fp4(pa, sa, pb, sb, f32(0.5), m, n, k)
    c8 = N.mm_fp4(pa, sa8, pb, sb, f32(0.5), m, n, k, a_layout="8x4")
    assert np.array_equal(c8, c128)


def test_global_sf_4over6_golden_and_256_block():
    for line in golden_lines("global_sf_4over6.txt"):
        amax, gsf = (float(v) for v in line.split())
        w = bits([amax, -amax / 2, 0.0, amax / 4] * 4).reshape(1, 16)
        g, inv, a = N.global_sf_4over6(w)
        assert a == f32(amax) and g == f32(gsf) and inv == f32(1.0) / f32(gsf)
    # the block holding the tensor amax gets the block scale 256 (byte 0x78) instead of 448
    for seed in range(4):
        w = W.small_case(32, 256, 40 + seed, std=0.02)
        g, _, amax = N.global_sf_4over6(w)
        _, sf = N.quantize(w, g, layout="linear")
        xf = W.bf16_bits_to_f32(w).reshape(32, 16, 16)
        blk = np.argwhere(np.max(np.abs(xf), axis=-1) == amax)[0]
        assert sf[blk[0], blk[1]] == 0x78
        assert sf.max() <= 0x78


# ------------------------------------------------------------------------ fragment layout
def test_frag_offsets_hand_worked():
    n = 0
    for line in golden_lines("frag_offsets_nvfp4.txt"):
        r, j, k, off = (int(v) for v in line.split()[:4])
        assert int(N.frag_packed_offset(r, j, k)) == off, line
        n += 1
    assert n == 10


def test_frag_offsets_are_a_permutation_for_any_k_multiple_of_64():
    for rows, k in [(33, 64), (5, 192), (64, 512), (40, 320)]:
        rp = N.frag_rows(rows)
        r, j = np.meshgrid(np.arange(rp), np.arange(k // 2), indexing="ij")
        off = N.frag_packed_offset(r, j, k).ravel()
        assert np.array_equal(np.sort(off), np.arange(rp * k // 2))
    with pytest.raises(ValueError):
        N.to_frag_packed(np.zeros((4, 40), np.uint8), 80)


def test_frag_layout_matches_the_lane_placement():
    """Independent construction by axis permutation: [tile, row i, step, half h, byte] of the padded
    row-major bytes becomes [tile, step, h, i, byte]; the round trip restores every row."""
    rng = np.random.default_rng(21)
    for rows, k in [(70, 192), (32, 64), (45, 768)]:
        packed = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
        fp = N.to_frag_packed(packed, k)
        rp = N.frag_rows(rows)
        pp = np.zeros((rp, k // 2), dtype=np.uint8)
        pp[:rows] = packed
        want = pp.reshape(rp // 32, 32, k // 64, 2, 16).transpose(0, 2, 3, 1, 4).ravel()
        assert np.array_equal(fp, want)
        assert np.array_equal(N.from_frag_packed(fp, rows, k), packed)
        sel = np.array([rows - 1, 0, rows // 2])
        assert np.array_equal(N.from_frag_packed(fp, sel, k), packed[sel])


def test_frag_packed_arrangement_is_the_mxfp4_fragment_arrangement():
    """The MXFP4 oracle's packed fragment offsets (written separately) agree where both apply."""
    from oracle import mxfp4 as X4
    for rows, k in [(64, 256), (33, 768)]:
        r, j = np.meshgrid(np.arange(N.frag_rows(rows)), np.arange(k // 2), indexing="ij")
        assert np.array_equal(N.frag_packed_offset(r, j, k), X4.frag_packed_offset(r, j, k))


def test_frag_quantize_and_gemm_agree_with_the_row_major_layout():
    m, n, k = 45, 37, 320
    xa = W.small_case(m, k, 31, outlier_frac=0.02)
    xb = W.small_case(n, k, 32, std=0.02)
    gb = N.global_sf(xb)[0]
    fa, sfa = N.quantize(xa, f32(1.0), packed_layout="frag")
    pa, sa = N.quantize(xa, f32(1.0))
    assert np.array_equal(sfa, sa)
    assert fa.size == 64 * k // 2
    assert np.array_equal(N.from_frag_packed(fa, m, k), pa)
    pad = N.frag_packed_offset(np.arange(m, 64)[:, None], np.arange(k // 2)[None, :], k)
    assert not fa[pad].any()
    fb, sfb = N.quantize(xb, gb, packed_layout="frag")
    pb, sb = N.quantize(xb, gb)
    al = N.alpha(f32(1.0), gb)
    got = N.mm_fp4_frag(fa, sfa, fb, sfb, al, m, n, k)
    assert np.array_equal(got, N.mm_fp4(pa, sa, pb, sb, al, m, n, k))
    # and the product is the brute-force fp64 sum of the dequantized values
    A = N.dequant_rows(pa, sa, np.arange(m), m, k)
    B = N.dequant_rows(pb, sb, np.arange(n), n, k)
    brute = np.array([[sum(A[i, t] * B[c, t] for t in range(k)) for c in range(n)] for i in range(m)])
    np.testing.assert_allclose(got, np.float64(al) * brute, rtol=1e-12, atol=1e-12)
