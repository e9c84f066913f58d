"""Pins for the MXFP4 oracle: hand-worked groups, the OCP floor rule, exactness, brute force."""
import numpy as np
import torch

import workloads as W
from oracle import formats as F
from oracle import mxfp4 as X4
from oracle import nvfp4 as N
from tests.conftest import golden_lines


def test_hand_worked_groups():
    for line in golden_lines("mxfp4_blocks.txt"):
        head, s_hex, p_hex = (p.split() for p in line.split("|"))
        vals = np.zeros(32, dtype=np.float32)
        pre = [float(v) for v in head[1:]]
        vals[:len(pre)] = pre
        xb = W.f32_to_bf16_bits(vals)
        assert np.array_equal(W.bf16_bits_to_f32(xb), vals)
        packed, s = X4.quantize(xb[None, :], layout="linear")
        assert int(s[0, 0]) == int(s_hex[0], 16), head[0]
        assert [int(b) for b in packed[0, :len(p_hex)]] == [int(h, 16) for h in p_hex], head[0]
        assert np.all(packed[0, len(p_hex):] == 0)


def test_scale_exponent_floor_rule():
    for a, es in [(1.0, -2), (3.99, -1), (4.0, 0), (7.9, 0), (8.0, 1), (6.0, 0), (0.0, -127),
                  (2.0 ** -140, -127), (3e38, 125)]:
        assert int(X4.scale_exponent(np.array([a]))[0]) == es, a


def test_scaled_amax_lands_in_top_binade():
    x = W.small_case(32, 512, 31, outlier_frac=0.02)
    p, s = X4.quantize(x, layout="linear")
    q = np.abs(F.e2m1_decode(N.unpack_nibbles(p))).reshape(32, 16, 32)
    assert np.all((q.max(axis=-1) >= 4) & (q.max(axis=-1) <= 6))


def test_exact_on_the_grid_and_layout():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, size=(130, 128)).astype(np.uint8)
    codes[:, ::32] = 7                                        # amax 6 * 2^E in every group
    E = rng.integers(-30, 30, size=(130, 4))
    vals = (F.e2m1_decode(codes).reshape(130, 4, 32) * np.ldexp(1.0, E)[..., None]).reshape(130, 128)
    xb = W.f32_to_bf16_bits(vals.astype(np.float32))
    p, sf = X4.quantize(xb)
    assert np.array_equal(X4.dequant_rows(p, sf, np.arange(130), 130, 128), vals)
    rp, cp = X4.sf_padded_shape(130, 128)
    assert (rp, cp) == (256, 4) and sf.size == 256 * 4
    lin = N.unswizzle_128x4(sf, rp, cp)
    assert np.all(lin[130:] == 0)


def test_mm_mxfp4_brute_force_and_torch():
    rng = np.random.default_rng(6)
    m, n, k = 3, 5, 64
    ca = rng.integers(0, 16, size=(m, k)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    la = np.zeros((128, 4), dtype=np.uint8)
    lb = np.zeros((128, 4), dtype=np.uint8)
    la[:m, :2] = rng.integers(100, 150, size=(m, 2))
    lb[:n, :2] = rng.integers(100, 150, size=(n, 2))
    e2 = F.e2m1_decode_table()
    al = np.float32(0.75)
    ref = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            ref[i, j] = float(al) * sum(e2[ca[i, kk]] * 2.0 ** (int(la[i, kk // 32]) - 127)
                                        * e2[cb[j, kk]] * 2.0 ** (int(lb[j, kk // 32]) - 127)
                                        for kk in range(k))
    pa, pb = N.pack_nibbles(ca), N.pack_nibbles(cb)
    sa, sb = N.swizzle_128x4(la), N.swizzle_128x4(lb)
    got = X4.mm_mxfp4(pa, sa, pb, sb, al, m, n, k)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    A = torch.from_numpy(e2[ca] * np.ldexp(1.0, la[:m, :2].astype(np.int64) - 127).repeat(32, axis=1))
    B = torch.from_numpy(e2[cb] * np.ldexp(1.0, lb[:n, :2].astype(np.int64) - 127).repeat(32, axis=1))
    assert np.allclose(float(al) * (A @ B.T).numpy(), ref, rtol=1e-12)
    r, c = np.array([2, 0]), np.array([4, 1])
    assert np.allclose(X4.mm_mxfp4_entries(pa, sa, pb, sb, al, m, n, k, r, c), ref[r, c], rtol=1e-12)


# ------------------------------------------------------------------------ fragment layout
def test_frag_offsets_hand_worked():
    n = 0
    for line in golden_lines("frag_offsets_mxfp4.txt"):
        kind, r, c, k, off = line.split()[:5]
        fn = X4.frag_packed_offset if kind == "p" else X4.frag_sf_offset
        assert int(fn(int(r), int(c), int(k))) == int(off), line
        n += 1
    assert n == 15


def test_frag_offsets_are_a_permutation():
    for rows, k in [(33, 256), (64, 512), (5, 768)]:
        rp = X4.frag_rows(rows)
        r, j = np.meshgrid(np.arange(rp), np.arange(k // 2), indexing="ij")
        off = X4.frag_packed_offset(r, j, k).ravel()
        assert np.array_equal(np.sort(off), np.arange(rp * k // 2))
        r, b = np.meshgrid(np.arange(rp), np.arange(k // 32), indexing="ij")
        off = X4.frag_sf_offset(r, b, k).ravel()
        assert np.array_equal(np.sort(off), np.arange(rp * k // 32))


def test_frag_layout_matches_mfma_lane_placement():
    """Independent construction by axis permutation: a fragment is [lane half h][row i][16 bytes]
    of one 32-row tile and 64-K step; a scale group is [h][i][step j of the group]."""
    rng = np.random.default_rng(8)
    rows, k = 70, 768
    packed = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    scales = rng.integers(0, 256, size=(rows, k // 32)).astype(np.uint8)
    fp, fs = X4.to_frag(packed, scales, k)
    rp = X4.frag_rows(rows)
    pp = np.zeros((rp, k // 2), dtype=np.uint8)
    pp[:rows] = packed
    ps = np.zeros((rp, k // 32), dtype=np.uint8)
    ps[:rows] = scales
    # packed [tile, i, step, h, byte] -> [tile, step, h, i, byte]
    want_p = pp.reshape(rp // 32, 32, k // 64, 2, 16).transpose(0, 2, 3, 1, 4).ravel()
    # scales [tile, i, group, j, h] (block = 8 group + 2 j + h) -> [tile, group, h, i, j]
    want_s = ps.reshape(rp // 32, 32, k // 256, 4, 2).transpose(0, 2, 4, 1, 3).ravel()
    assert np.array_equal(fp, want_p) and np.array_equal(fs, want_s)
    back_p, back_s = X4.from_frag(fp, fs, rows, k)
    assert np.array_equal(back_p, packed) and np.array_equal(back_s, scales)


def test_frag_quantize_and_gemm_agree_with_the_linear_layouts():
    xa = W.small_case(45, 512, 11, outlier_frac=0.02)
    xb = W.small_case(37, 512, 12, outlier_frac=0.02)
    fa, fsa = X4.quantize(xa, layout="frag")
    pa, sa = X4.quantize(xa, layout="linear")
    assert np.array_equal(X4.from_frag(fa, fsa, 45, 512)[0], pa)
    assert np.array_equal(X4.from_frag(fa, fsa, 45, 512)[1], sa)
    assert fa.size == 64 * 256 and not fa[X4.frag_packed_offset(np.arange(45, 64)[:, None], np.arange(256)[None, :], 512)].any()
    fb, fsb = X4.quantize(xb, layout="frag")
    got = X4.mm_mxfp4_frag(fa, fsa, fb, fsb, np.float32(0.75), 45, 37, 512)
    a1, s1 = X4.quantize(xa)
    b1, t1 = X4.quantize(xb)
    assert np.array_equal(got, X4.mm_mxfp4(a1, s1, b1, t1, np.float32(0.75), 45, 37, 512))
