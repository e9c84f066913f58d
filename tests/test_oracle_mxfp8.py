"""Pins for the MXFP8 oracle: hand-worked groups, the OCP floor rule, exactness, brute force."""
import numpy as np
import torch

import workloads as W
from oracle import formats as F
from oracle import mxfp8 as X
from tests.conftest import golden_lines


def test_hand_worked_groups():
    for line in golden_lines("mxfp8_blocks.txt"):
        head, s_hex, e_hex = (p.split() for p in line.split("|"))
        vals = np.zeros(32, dtype=np.float32)
        pre = [float(v) for v in head[1:]]
        vals[:len(pre)] = pre
        xb = W.f32_to_bf16_bits(vals)
        assert np.array_equal(W.bf16_bits_to_f32(xb), vals)
        q, s = X.quantize(xb[None, :])
        assert int(s[0, 0]) == int(s_hex[0], 16), head[0]
        assert [int(b) for b in q[0, :len(e_hex)]] == [int(h, 16) for h in e_hex], head[0]
        assert np.all((q[0, len(pre):] & 0x7F) == 0)


def test_scale_exponent_floor_rule():
    for a, es in [(1.0, -8), (1.5, -8), (2.0, -7), (255.9, -1), (256.0, 0), (511.0, 0), (512.0, 1),
                  (2.0 ** -130, -127), (0.0, -127), (3e38, 119)]:
        assert int(X.scale_exponent(np.array([a]))[0]) == es, a


def test_scaled_amax_lands_in_top_binade():
    x = W.small_case(64, 512, 21, outlier_frac=0.02)
    q, s = X.quantize(x)
    qv = np.abs(F.e4m3_decode(q)).reshape(64, 16, 32)
    top = qv.max(axis=-1)
    assert np.all((top >= 256) & (top <= 448))


def test_exact_for_values_on_the_mx_grid():
    # dequant(quant(x)) == x when x already is e4m3 * 2^E with the group's own exponent
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 0x7F, size=(8, 64)).astype(np.uint8)
    codes[:, ::32] = 0x7C                                    # amax 384 * 2^E in every group
    E = rng.integers(-20, 20, size=(8, 2))
    vals = (F.e4m3_decode(codes).reshape(8, 2, 32) * np.ldexp(1.0, E)[..., None]).reshape(8, 64)
    xb = W.f32_to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(xb), vals.astype(np.float32))
    q, s = X.quantize(xb)
    assert np.array_equal(X.dequant_rows(q, s, np.arange(8)), vals)


def test_mm_mxfp8_brute_force_and_torch():
    rng = np.random.default_rng(5)
    m, n, k = 4, 6, 64
    qa = rng.integers(0, 256, size=(m, k)).astype(np.uint8)
    qb = rng.integers(0, 256, size=(n, k)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x11                           # no NaN codes
    qb[(qb & 0x7F) == 0x7F] = 0x22
    sa = rng.integers(100, 150, size=(m, k // 32)).astype(np.uint8)
    sb = rng.integers(100, 150, size=(n, k // 32)).astype(np.uint8)
    e4 = F.e4m3_decode_table()
    ref = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            ref[i, j] = sum(e4[qa[i, kk]] * 2.0 ** (int(sa[i, kk // 32]) - 127)
                            * e4[qb[j, kk]] * 2.0 ** (int(sb[j, kk // 32]) - 127) for kk in range(k))
    got = X.mm_mxfp8(qa, sa, qb, sb, m, n, k)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    A = torch.from_numpy(qa).view(torch.float8_e4m3fn).double() * torch.from_numpy(
        np.ldexp(1.0, sa.astype(np.int64) - 127)).repeat_interleave(32, dim=1)
    B = torch.from_numpy(qb).view(torch.float8_e4m3fn).double() * torch.from_numpy(
        np.ldexp(1.0, sb.astype(np.int64) - 127)).repeat_interleave(32, dim=1)
    assert np.allclose((A @ B.T).numpy(), ref, rtol=1e-12)
    r, c = np.array([3, 0, 1]), np.array([5, 2, 1])
    assert np.allclose(X.mm_mxfp8_entries(qa, sa, qb, sb, r, c), ref[r, c], rtol=1e-12)


def test_zero_group():
    q, s = X.quantize(np.zeros((1, 64), dtype=np.uint16))
    assert np.all(q == 0) and np.all(s == 0)


# ------------------------------------------------------------------------ fragment layout
def test_frag_offsets_hand_worked():
    from tests.conftest import golden_lines
    n = 0
    for line in golden_lines("frag_offsets_mxfp8.txt"):
        r, c, k, off = (int(v) for v in line.split()[:4])
        assert int(X.frag_offset(r, c, k)) == off, line
        n += 1
    assert n == 11


def test_frag_layout_is_a_permutation_and_matches_the_lane_placement():
    """Offsets form a permutation; an independent construction by axis permutation: a fragment is
    [block b][lane half h][row i][16 bytes] of one 32-row tile and 64-K step."""
    from oracle import mxfp4 as X4
    for rows, k in [(33, 256), (70, 768)]:
        rp = X4.frag_rows(rows)
        r, c = np.meshgrid(np.arange(rp), np.arange(k), indexing="ij")
        assert np.array_equal(np.sort(X.frag_offset(r, c, k).ravel()), np.arange(rp * k))
        rng = np.random.default_rng(rows)
        q = rng.integers(0, 256, size=(rows, k)).astype(np.uint8)
        s = rng.integers(0, 256, size=(rows, k // 32)).astype(np.uint8)
        fq, fs = X.to_frag(q, s, k)
        qp = np.zeros((rp, k), dtype=np.uint8)
        qp[:rows] = q
        # [tile, i, step, block, h, byte] -> [tile, step, block, h, i, byte]
        want = qp.reshape(rp // 32, 32, k // 64, 2, 2, 16).transpose(0, 2, 3, 4, 1, 5).ravel()
        assert np.array_equal(fq, want)
        sp = np.zeros((rp, k // 32), dtype=np.uint8)
        sp[:rows] = s
        assert np.array_equal(fs, X4.to_frag(np.zeros((rows, k // 2), np.uint8), s, k)[1])
        assert np.array_equal(fs, sp.reshape(rp // 32, 32, k // 256, 4, 2).transpose(0, 2, 4, 1, 3).ravel())
        bq, bs = X.from_frag(fq, fs, rows, k)
        assert np.array_equal(bq, q) and np.array_equal(bs, s)


def test_frag_quantize_and_gemm_agree_with_the_row_major_layout():
    xa = W.small_case(45, 512, 21, outlier_frac=0.02)
    xb = W.small_case(37, 512, 22, outlier_frac=0.02)
    fa, fsa = X.quantize_frag(xa)
    fb, fsb = X.quantize_frag(xb)
    qa, sa = X.quantize(xa)
    qb, sb = X.quantize(xb)
    assert np.array_equal(X.from_frag(fa, fsa, 45, 512)[0], qa)
    assert np.array_equal(X.mm_mxfp8_frag(fa, fsa, fb, fsb, 45, 37, 512), X.mm_mxfp8(qa, sa, qb, sb, 45, 37, 512))
