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
