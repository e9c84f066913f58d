"""GPU parity of the HBM-bound kernels against the oracle: bit-exact bytes and scalars.

the global scale, NVFP4 quantize (packed nibbles + 128x4 scale bytes, padding included),
alpha, MXFP8 quantize, and the GELU between the FFN projections (within one bf16 ulp).
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsp
import workloads as W
from oracle import activations as A
from oracle import mxfp8 as X
from oracle import nvfp4 as N
from tests.gpu_util import (assert_nvfp4_of_gelu, dev_bf16, gelu_in_table, host_bits, host_u8, say, scalar,
                            tensor_bits)

pytestmark = pytest.mark.gpu
f32 = np.float32


def _quant_gpu(xb, gsf, ld=None):
    m, k = xb.shape
    if ld is not None and ld != k:
        big = np.zeros((m, ld), dtype=np.uint16)
        big[:, :k] = xb
        x = dev_bf16(big)[:, :k]
    else:
        x = dev_bf16(xb)
    packed, sf = bsp.bsp_nvfp4_quantize(x, scalar(gsf))
    return host_u8(packed), host_u8(sf).ravel()


@pytest.mark.parametrize("m,k", [(1, 16), (1, 512), (77, 48), (128, 64), (129, 80), (200, 512),
                                 (300, 1536), (256, 1040)])
@pytest.mark.parametrize("gsf_kind", ["unit", "weight"])
def test_nvfp4_quantize_bit_exact(m, k, gsf_kind):
    say("nvfp4_quantize", m, k, gsf_kind)
    xb = W.small_case(m, k, seed=m * 131 + k, outlier_frac=0.02)
    g = f32(1.0) if gsf_kind == "unit" else N.global_sf(xb)[0]
    packed, sf = _quant_gpu(xb, g)
    rp, ap = N.quantize(xb, g)
    assert np.array_equal(packed, rp)
    assert np.array_equal(sf, ap)


def test_nvfp4_quantize_strided_rows():
    xb = W.small_case(150, 256, seed=5)
    packed, sf = _quant_gpu(xb, f32(3.5), ld=264)
    rp, ap = N.quantize(xb, f32(3.5))
    assert np.array_equal(packed, rp) and np.array_equal(sf, ap)
    packed, sf = _quant_gpu(xb, f32(3.5), ld=259)   # unaligned rows take the scalar-load path
    assert np.array_equal(packed, rp) and np.array_equal(sf, ap)


@pytest.mark.parametrize("gsf", [1.0, 0.37, 2688.0 / 5.0])
def test_nvfp4_quantize_special_values(gsf):
    xb = W.special_values_block(seed=7, rows=256, cols=512)
    packed, sf = _quant_gpu(xb, f32(gsf))
    rp, ap = N.quantize(xb, f32(gsf))
    assert np.array_equal(packed, rp)
    assert np.array_equal(sf, ap)


@pytest.mark.parametrize("cfg,name", [(2, "X"), (3, "X"), (4, "X"), (4, "W"), (4, "W2")])
def test_nvfp4_quantize_full_size_sampled_rows(cfg, name):
    """Full Wan-shaped tensors in the launch configuration the bench uses; the oracle checks
    sampled rows (quantization is row-local given gsf) and every padding byte."""
    xb = tensor_bits(cfg, name)
    m, k = xb.shape
    say("full-size quantize", cfg, name, m, k)
    g = N.global_sf(xb)[0] if name.startswith("W") else f32(1.0)
    x = dev_bf16(xb)
    packed, sf = bsp.bsp_nvfp4_quantize(x, scalar(g))
    rng = np.random.default_rng(cfg)
    rows = np.unique(np.concatenate([rng.integers(0, m, 48), [0, 1, 127, 128, m - 2, m - 1]]))
    got_p = host_u8(packed[torch.from_numpy(rows).cuda()])
    ref_p, ref_s = N.quantize(xb[rows], g, layout="linear")
    assert np.array_equal(got_p, ref_p)
    rp, cp = N.sf_padded_shape(m, k)
    sfh = host_u8(sf).ravel()
    lin = N.unswizzle_128x4(sfh, rp, cp)
    assert np.array_equal(lin[rows, : k // 16], ref_s)
    assert np.all(lin[m:] == 0) and np.all(lin[:, k // 16:] == 0)


@pytest.mark.parametrize("m,k", [(1, 16), (77, 48), (129, 96), (300, 1536), (256, 1040),
                                 (200, 5120), (130, 13824), (70, 16400)])
def test_nvfp4_quantize_per_token_bit_exact(m, k):
    """Per-token scales: packed bytes, 128x4 scale bytes (padding included) and the fp32 row scales
    equal the oracle's; covers the one-pass register path and the two-pass path (K > 16384)."""
    say("nvfp4_quantize_per_token", m, k)
    xb = W.small_case(m, k, seed=m * 17 + k, outlier_frac=0.02).copy()
    xb[m // 2] = 0                                   # an all-zero token
    if m > 3:
        xb[1] = W.small_case(1, k, seed=5, std=1e-30)[0]   # a token of tiny values
        xb[2] = W.small_case(1, k, seed=6, std=1e4)[0]     # and of large ones
    p, sf, g = bsp.bsp_nvfp4_quantize_per_token(dev_bf16(xb))
    rp, rs, rg = N.quantize_per_token(xb)
    assert np.array_equal(g.cpu().numpy(), rg)
    assert np.array_equal(host_u8(p), rp)
    assert np.array_equal(host_u8(sf).ravel(), rs)


def _u8_at(shape, offset):
    """A contiguous uint8 device tensor whose data starts `offset` bytes into its allocation (the
    allocation itself is 256-byte aligned)."""
    n = int(np.prod(shape))
    return torch.zeros(n + offset, dtype=torch.uint8, device="cuda")[offset:].view(*shape)


def test_quantizers_packed_output_not_16_byte_aligned():
    """Packed outputs 4-byte but not 16-byte aligned, at K % 32 == 0: the per-tensor, per-token and
    RMSNorm quantizers write each lane's four bytes instead of their 16-byte row pieces, and the
    bytes are the oracle's."""
    m, k = 130, 512
    xb = W.small_case(m, k, seed=21, outlier_frac=0.02)
    rp, rs = N.quantize(xb, f32(0.5))
    p = _u8_at((m, k // 2), 4)
    _, s = bsp.bsp_nvfp4_quantize(dev_bf16(xb), scalar(0.5), packed=p)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(s).ravel(), rs)
    tp, ts, tg = N.quantize_per_token(xb)
    p = _u8_at((m, k // 2), 4)
    _, s, g = bsp.bsp_nvfp4_quantize_per_token(dev_bf16(xb), packed=p)
    assert np.array_equal(g.cpu().numpy(), tg)
    assert np.array_equal(host_u8(p), tp) and np.array_equal(host_u8(s).ravel(), ts)


def test_nvfp4_quantize_per_token_strided_and_special():
    xb = W.special_values_block(seed=17, rows=140, cols=512)
    big = np.zeros((140, 520), dtype=np.uint16)
    big[:, :512] = xb
    p, sf, g = bsp.bsp_nvfp4_quantize_per_token(dev_bf16(big)[:, :512])
    rp, rs, rg = N.quantize_per_token(xb)
    assert np.array_equal(g.cpu().numpy(), rg)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(sf).ravel(), rs)
    p2, sf2, _ = bsp.bsp_nvfp4_quantize_per_token(dev_bf16(big)[:, 1:513])   # unaligned rows
    rp2, rs2, _ = N.quantize_per_token(big[:, 1:513])
    assert np.array_equal(host_u8(p2), rp2) and np.array_equal(host_u8(sf2).ravel(), rs2)


@pytest.mark.parametrize("cfg,name", [(4, "X"), (3, "X")])
def test_nvfp4_quantize_per_token_full_size_sampled_rows(cfg, name):
    xb = tensor_bits(cfg, name)
    m, k = xb.shape
    say("full-size per-token quantize", cfg, name, m, k)
    p, sf, g = bsp.bsp_nvfp4_quantize_per_token(dev_bf16(xb))
    rows = np.unique(np.concatenate([np.random.default_rng(cfg + 40).integers(0, m, 48), [0, 127, 128, m - 1]]))
    ri = torch.from_numpy(rows).cuda()
    ref_p, ref_s, ref_g = N.quantize_per_token(xb[rows], layout="linear")
    assert np.array_equal(g[ri].cpu().numpy(), ref_g)
    assert np.array_equal(host_u8(p[ri]), ref_p)
    rp, cp = N.sf_padded_shape(m, k)
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp, cp)
    assert np.array_equal(lin[rows, : k // 16], ref_s)
    assert np.all(lin[m:] == 0)


@pytest.mark.parametrize("m,k", [(1, 16), (5, 64), (13, 80), (77, 1536), (129, 96), (300, 512)])
@pytest.mark.parametrize("gsf_kind", ["unit", "weight"])
def test_nvfp4_quantize_8x4_bit_exact(m, k, gsf_kind):
    say("nvfp4_quantize_8x4", m, k, gsf_kind)
    xb = W.small_case(m, k, seed=m * 29 + k, outlier_frac=0.02)
    g = f32(1.0) if gsf_kind == "unit" else N.global_sf(xb)[0]
    p, sf = bsp.bsp_nvfp4_quantize_8x4(dev_bf16(xb), scalar(g))
    rp, rs = N.quantize(xb, g, layout="8x4")
    assert sf.numel() == rs.size
    assert np.array_equal(host_u8(p), rp)
    assert np.array_equal(host_u8(sf).ravel(), rs)


def test_global_sf_4over6_bit_exact():
    cases = [tensor_bits(1, "W"), tensor_bits(2, "W"), W.small_case(3, 100, 4, std=1e-3),
             np.zeros((4, 64), dtype=np.uint16), W.small_case(7, 64, 12, std=30.0)]
    for wb in cases:
        gsf, inv, amax = bsp.bsp_nvfp4_global_sf_4over6(dev_bf16(wb))
        rg, ri, ra = N.global_sf_4over6(wb)
        assert gsf.item() == rg and inv.item() == ri and amax.item() == ra
        if wb.shape[1] % 16:
            continue
        p, sf = bsp.bsp_nvfp4_quantize(dev_bf16(wb), gsf)
        rp, rs = N.quantize(wb, rg)
        assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(sf).ravel(), rs)
        assert rs.max() <= 0x78                        # block scales stay at or below 256


def test_global_sf_bit_exact():
    cases = [tensor_bits(1, "W"), tensor_bits(2, "W"), W.small_case(3, 100, 4, std=1e-3),
             np.zeros((4, 64), dtype=np.uint16)]
    w = W.small_case(8, 64, 9).copy()
    w[2, 5] = 0x7FC0          # NaN
    w[3, 7] = 0xFF80          # -inf
    cases.append(w)
    w2 = W.small_case(8, 64, 10).copy()
    w2[1, 1] = 0x7FC0
    cases.append(w2)
    for wb in cases:
        gsf, inv, amax = bsp.bsp_nvfp4_global_sf(dev_bf16(wb))
        rg, ri, ra = N.global_sf(wb)
        got = (gsf.cpu().numpy()[0], inv.cpu().numpy()[0], amax.cpu().numpy()[0])
        say("global_sf", wb.shape, got, (rg, ri, ra))
        assert got[0] == rg and got[1] == ri and got[2] == ra


def test_global_sf_strided_and_tail_positions():
    """The amax reduction's three paths (contiguous rows, strided rows, unaligned element by
    element), with the largest magnitude planted at the first, a middle and the last element."""
    rng = np.random.default_rng(21)
    for rows, k, ld in [(300, 512, 512), (300, 512, 520), (37, 1000, 1000), (5, 96, 101), (1, 4096, 4096)]:
        for pos in ("first", "middle", "last"):
            big = W.small_case(rows, ld, int(rng.integers(1 << 30)), std=0.5)
            r, c = {"first": (0, 0), "middle": (rows // 2, k // 3), "last": (rows - 1, k - 1)}[pos]
            big[r, c] = 0xC2F6                                   # -123.0, the largest magnitude
            big[:, k:] = 0x7F7F                                  # outside the view: must be ignored
            wb = np.ascontiguousarray(big[:, :k])
            w = dev_bf16(big)[:, :k]
            gsf, inv, amax = bsp.bsp_nvfp4_global_sf(w)
            rg, ri, ra = N.global_sf(wb)
            assert ra == np.float32(123.0), (rows, k, ld, pos)
            assert (gsf.item(), inv.item(), amax.item()) == (rg, ri, ra), (rows, k, ld, pos)


def test_prequantize_weight_matches_separate_calls_and_oracle():
    for cfg in (1, 2):
        wb = tensor_bits(cfg, "W")
        packed, sf, gsf, inv, amax = bsp.bsp_nvfp4_prequantize_weight(dev_bf16(wb))
        rg, ri, _ = N.global_sf(wb)
        assert gsf.item() == rg and inv.item() == ri
        rp, ap = N.quantize(wb, rg)
        assert np.array_equal(host_u8(packed), rp) and np.array_equal(host_u8(sf).ravel(), ap)


def test_alpha_bit_exact():
    rng = np.random.default_rng(3)
    for _ in range(20):
        xg, wg = f32(rng.uniform(0.1, 10)), f32(10 ** rng.uniform(-3, 6))
        got = bsp.bsp_nvfp4_alpha(scalar(xg), scalar(wg)).item()
        assert np.float32(got) == N.alpha(xg, wg)
    assert bsp.bsp_nvfp4_alpha(scalar(1.0), scalar(43008.0)).item() == np.float32(1) / np.float32(43008)


@pytest.mark.parametrize("m,k", [(1, 32), (63, 96), (64, 256), (130, 512), (257, 1056)])
def test_mxfp8_quantize_bit_exact(m, k):
    xb = W.small_case(m, k, seed=m + 7 * k, outlier_frac=0.02)
    q, sf = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
    rq, rs = X.quantize(xb)
    assert np.array_equal(host_u8(q), rq) and np.array_equal(host_u8(sf), rs)


def test_mxfp8_quantize_special_values():
    xb = W.special_values_block(seed=11, rows=128, cols=512)
    q, sf = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
    rq, rs = X.quantize(xb)
    assert np.array_equal(host_u8(q), rq) and np.array_equal(host_u8(sf), rs)


def test_mxfp8_quantize_full_size_sampled_rows():
    for name in ("X", "W"):
        xb = tensor_bits(5, name)
        m, k = xb.shape
        q, sf = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
        rows = np.unique(np.concatenate([np.random.default_rng(5).integers(0, m, 48), [0, m - 1]]))
        ri = torch.from_numpy(rows).cuda()
        rq, rs = X.quantize(xb[rows])
        assert np.array_equal(host_u8(q[ri]), rq) and np.array_equal(host_u8(sf[ri]), rs)


def test_gelu_within_one_bf16_ulp():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(200000) * 3, np.linspace(-12, 12, 4801), np.linspace(-10.5, -9.5, 4001),
                        [0.0, -0.0, 1e-30, -1e-30, 50.0, -50.0]]).astype(np.float32)
    xb = W.f32_to_bf16_bits(v)
    got = host_bits(bsp.bsp_gelu_tanh_bf16(dev_bf16(xb)))
    ref = A.gelu_tanh_bf16_bits(xb)
    gv = W.bf16_bits_to_f32(got).astype(np.float64)
    rv = W.bf16_bits_to_f32(ref).astype(np.float64)
    tol = np.abs(rv) * 2.0 ** -7 + 2.0 ** -126
    assert np.all(np.abs(gv - rv) <= tol)
    assert np.mean(got == ref) > 0.99
    inside = gelu_in_table(xb)            # correctly rounded there: equal to the oracle
    assert inside.mean() > 0.9 and np.array_equal(got[inside], ref[inside])
    # in place, odd length (tail path)
    x = dev_bf16(xb[:1001].copy())
    bsp.bsp_gelu_tanh_bf16(x, out=x)
    assert np.array_equal(host_bits(x), got[:1001])


def _gelu_ref_check(xb, got):
    """GPU GELU bytes against the oracle: within one bf16 ulp everywhere, equal almost everywhere,
    equal on every input inside the GELU table."""
    ref = A.gelu_tanh_bf16_bits(xb)
    gv = W.bf16_bits_to_f32(got).astype(np.float64)
    rv = W.bf16_bits_to_f32(ref).astype(np.float64)
    assert np.all(np.abs(gv - rv) <= np.abs(rv) * 2.0 ** -7 + 2.0 ** -126)
    assert np.mean(got == ref) > 0.99
    inside = gelu_in_table(np.asarray(xb).ravel()).reshape(np.shape(xb))
    assert np.array_equal(np.asarray(got)[inside], ref[inside])


@pytest.mark.parametrize("m,k", [(1, 16), (77, 48), (129, 96), (300, 1536), (256, 1040)])
@pytest.mark.parametrize("gsf", [1.0, 0.37])
def test_nvfp4_quantize_gelu_matches_oracle_chain(m, k, gsf):
    """The fused kernel against the oracle's GELU-then-quantize of the same bf16 y: bit-exact in
    every block whose GELU values are not within a few fp32 ulps of a bf16 rounding boundary; and
    the same bytes as the GPU's own quantize of the GPU's GELU (the stand-alone GELU is checked
    against the oracle to one bf16 ulp)."""
    say("nvfp4_quantize_gelu", m, k, gsf)
    yb = W.small_case(m, k, seed=3 * m + k, std=2.5, outlier_frac=0.02)
    y = dev_bf16(yb)
    h = bsp.bsp_gelu_tanh_bf16(y)
    _gelu_ref_check(yb, host_bits(h))
    p, sf = bsp.bsp_nvfp4_quantize_gelu(y, scalar(gsf))
    rp_, cp_ = N.sf_padded_shape(m, k)
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp_, cp_)
    assert_nvfp4_of_gelu(host_u8(p), lin, yb, gsf, f"quantize_gelu {m}x{k}")
    assert not lin[m:].any()
    p2, sf2 = bsp.bsp_nvfp4_quantize(h, scalar(gsf))
    assert torch.equal(p, p2) and torch.equal(sf, sf2)


def test_nvfp4_quantize_gelu_strided_and_special():
    yb = W.special_values_block(seed=13, rows=200, cols=512)
    big = np.zeros((200, 520), dtype=np.uint16)
    big[:, :512] = yb
    y = dev_bf16(big)[:, :512]
    p, sf = bsp.bsp_nvfp4_quantize_gelu(y, scalar(1.0))
    rp_, cp_ = N.sf_padded_shape(200, 512)
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp_, cp_)
    assert_nvfp4_of_gelu(host_u8(p), lin, yb, 1.0, "quantize_gelu special values", max_ambiguous=0.3)
    p2, sf2 = bsp.bsp_nvfp4_quantize(bsp.bsp_gelu_tanh_bf16(dev_bf16(yb)), scalar(1.0))
    assert torch.equal(p, p2) and torch.equal(sf, sf2)


@pytest.mark.parametrize("m,k", [(32760, 8960), (32760, 13824)])
def test_nvfp4_quantize_gelu_full_size_sampled_rows(m, k):
    """The FFN activations at the Wan-1.3B and Wan-14B fc_in output shapes, in the bench's launch
    configuration; sampled rows against the oracle, every padding scale byte checked."""
    say("full-size quantize_gelu", m, k)
    g = torch.Generator(device="cuda")
    g.manual_seed(k)
    y = (torch.randn((m, k), device="cuda", generator=g) * 2.0).to(torch.bfloat16)
    p, sf = bsp.bsp_nvfp4_quantize_gelu(y, scalar(1.0))
    rows = np.unique(np.concatenate([np.random.default_rng(k).integers(0, m, 40), [0, 127, 128, m - 1]]))
    ri = torch.from_numpy(rows).cuda()
    yb = host_bits(y[ri])                    # the seeded input rows
    rp, cp = N.sf_padded_shape(m, k)
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp, cp)
    assert_nvfp4_of_gelu(host_u8(p[ri]), lin[rows], yb, 1.0, f"full-size quantize_gelu {m}x{k}")
    assert np.all(lin[m:] == 0)


_SW_SCRIPT = r"""
import sys, numpy as np
sys.path.insert(0, sys.argv[1])
import block_scaled_precision_nvfp4_amd as bsp, workloads as W
from oracle import nvfp4 as N, mxfp8 as X
from tests.gpu_util import dev_bf16, host_u8, scalar
for m, k in [(129, 96), (300, 1536)]:
    xb = W.special_values_block(seed=m, rows=m, cols=k)
    p, s = bsp.bsp_nvfp4_quantize(dev_bf16(xb), scalar(0.37))
    rp, rs = N.quantize(xb, np.float32(0.37))
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(s).ravel(), rs)
    q, sq = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
    rq, rsq = X.quantize(xb)
    assert np.array_equal(host_u8(q), rq) and np.array_equal(host_u8(sq), rsq)
print("SW-PATH-OK")
"""


def test_software_encoder_path_bit_exact():
    """BSP_QUANT_SW_CVT=1 switches both quantizers to the software encoders; they must give the
    same bytes as the hardware-convert default (both checked against the oracle)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, BSP_QUANT_SW_CVT="1")
    r = subprocess.run([sys.executable, "-c", _SW_SCRIPT, root], env=env, capture_output=True,
                       text=True, timeout=150)
    assert r.returncode == 0 and "SW-PATH-OK" in r.stdout, r.stdout + r.stderr


@pytest.mark.parametrize("m,k", [(1, 32), (77, 96), (128, 256), (200, 512), (300, 1568)])
def test_mxfp4_quantize_bit_exact(m, k):
    from oracle import mxfp4 as X4
    xb = W.small_case(m, k, seed=3 * m + k, outlier_frac=0.02)
    p, s = bsp.bsp_mxfp4_quantize(dev_bf16(xb))
    rp, rs = X4.quantize(xb)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(s).ravel(), rs)
    xs = W.special_values_block(seed=m, rows=m, cols=k)
    p, s = bsp.bsp_mxfp4_quantize(dev_bf16(xs))
    rp, rs = X4.quantize(xs)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(s).ravel(), rs)


# ---------------------------------------------------------------------------------------------
# non-finite inputs: every quantizer encodes nan_to_num of its input (NaN -> +0, +-inf -> +-largest
# finite bf16), bit-exact against the oracle
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("gsf", [1.0, 0.37, 2688.0 / 5.0])
def test_nvfp4_quantize_nonfinite(gsf):
    say("nvfp4_quantize nonfinite", gsf)
    xb = W.nonfinite_block(seed=23, rows=200, cols=512)
    packed, sf = _quant_gpu(xb, f32(gsf))
    rp, ap = N.quantize(xb, f32(gsf))
    assert np.array_equal(packed, rp) and np.array_equal(sf, ap)
    p8, s8 = bsp.bsp_nvfp4_quantize_8x4(dev_bf16(xb), scalar(f32(gsf)))
    rp8, rs8 = N.quantize(xb, f32(gsf), layout="8x4")
    assert np.array_equal(host_u8(p8), rp8) and np.array_equal(host_u8(s8).ravel(), rs8)


@pytest.mark.parametrize("k", [512, 16400])   # one-pass register path and two-pass path
def test_nvfp4_quantize_per_token_nonfinite(k):
    say("nvfp4_quantize_per_token nonfinite", k)
    xb = W.nonfinite_block(seed=29, rows=70, cols=k)
    p, sf, g = bsp.bsp_nvfp4_quantize_per_token(dev_bf16(xb))
    rp, rs, rg = N.quantize_per_token(xb)
    assert np.array_equal(g.cpu().numpy(), rg)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(sf).ravel(), rs)


def test_mx_quantize_nonfinite():
    from oracle import mxfp4 as X4
    say("mx quantize nonfinite")
    xb = W.nonfinite_block(seed=31, rows=130, cols=512)
    q, sf = bsp.bsp_mxfp8_quantize(dev_bf16(xb))
    rq, rs = X.quantize(xb)
    assert np.array_equal(host_u8(q), rq) and np.array_equal(host_u8(sf), rs)
    p, s = bsp.bsp_mxfp4_quantize(dev_bf16(xb))
    rp, rs4 = X4.quantize(xb)
    assert np.array_equal(host_u8(p), rp) and np.array_equal(host_u8(s).ravel(), rs4)
