"""GPU parity of the RMSNorm + NVFP4 quantize prologue against the oracle (oracle/norm.py).

The GPU evaluates RMSNorm in IEEE fp32 with a fixed summation order; the oracle in fp64. Their
relative difference is bounded by `norm_rel_bound` below (three fp32 roundings), so a bf16 output can round differently
only where the exact value lies that close to a bf16 rounding boundary ("ambiguous"). Every other
element must be bit-equal, and every 16-element block free of ambiguous elements must quantize to
the oracle's bytes exactly. Expected values come from the oracle applied to the seeded inputs.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsp
import workloads as W
from oracle import activations as A
from oracle import norm as R
from oracle import nvfp4 as N
from tests.gpu_util import (assert_nvfp4_blocks, dev_bf16, host_bits, host_u8, say, scalar,
                            tensor_bits)

pytestmark = pytest.mark.gpu


def norm_rel_bound(k: int) -> float:
    """Bound on |y_gpu / y_exact - 1| before the bf16 rounding: r is the fp32 rounding of an fp64
    evaluation (sum of exact squares, division, sqrt, reciprocal: a few fp64 ulps, far below
    2^-40 for any K the kernel takes), then the fp32 products x * r and * w: three roundings of
    at most 2^-24 relative each."""
    return 3 * 2.0 ** -24 + 2.0 ** -40


def ambiguous(y_exact: np.ndarray, rel: float) -> np.ndarray:
    """Elements whose bf16 rounding can change within a relative perturbation of 1.5 * rel."""
    d = 1.5 * rel
    return A.f64_to_bf16_bits(y_exact * (1 - d)) != A.f64_to_bf16_bits(y_exact * (1 + d))


def check_norm(got_bits, xb, wb, eps, what):
    """GPU bf16 RMSNorm output against the oracle: equal outside ambiguous elements, within one
    bf16 step on them."""
    w = None if wb is None else R.bf16_bits_to_f64(wb)
    y = R.rms_norm(R.bf16_bits_to_f64(xb), w, eps)
    ref = A.f64_to_bf16_bits(y)
    amb = ambiguous(y, norm_rel_bound(xb.shape[1]))
    say(what, "ambiguous elements:", int(amb.sum()), "of", amb.size)
    assert amb.mean() < 0.005, what
    assert np.array_equal(got_bits[~amb], ref[~amb]), what
    diff = np.abs(got_bits.astype(np.int32) - ref.astype(np.int32))
    assert np.all(diff[amb] <= 1), what          # adjacent bf16 codes (same sign here)
    return y, amb


def check_fused(p, sf, xb, wb, eps, gsf, what):
    """Fused kernel bytes against the oracle chain (RMSNorm, bf16, NVFP4 quantize)."""
    m, k = xb.shape
    w = None if wb is None else R.bf16_bits_to_f64(wb)
    y = R.rms_norm(R.bf16_bits_to_f64(xb), w, eps)
    rp, rs = N.quantize(A.f64_to_bf16_bits(y), np.float32(gsf), layout="linear")
    amb = ambiguous(y, norm_rel_bound(k)).reshape(m, k // 16, 16).any(axis=-1)
    say(what, "ambiguous blocks:", int(amb.sum()), "of", amb.size)
    assert amb.mean() < 0.05, what
    rp_, cp_ = N.sf_padded_shape(m, k)
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp_, cp_)
    assert_nvfp4_blocks(host_u8(p), lin, rp, rs, ~amb, what)
    assert not lin[m:].any() and not lin[:, k // 16:].any()


SHAPES = [(1, 16), (77, 48), (129, 1536), (300, 5120), (130, 13824), (5, 20000)]


@pytest.mark.parametrize("m,k", SHAPES)
@pytest.mark.parametrize("with_w", [False, True])
def test_rmsnorm_bf16_matches_oracle(m, k, with_w):
    say("rmsnorm", m, k, with_w)
    xb = W.small_case(m, k, seed=5 * m + k, std=1.5, outlier_frac=0.01)
    wb = W.small_case(1, k, seed=k + 7, std=1.0)[0] if with_w else None
    wt = None if wb is None else dev_bf16(wb)
    got = host_bits(bsp.bsp_rmsnorm_bf16(dev_bf16(xb), wt, 1e-6))
    check_norm(got, xb, wb, 1e-6, f"rmsnorm {m}x{k} w={with_w}")


@pytest.mark.parametrize("m,k", SHAPES)
@pytest.mark.parametrize("gsf,with_w", [(1.0, False), (0.37, True)])
def test_nvfp4_quantize_rmsnorm_matches_oracle_chain(m, k, gsf, with_w):
    say("quantize_rmsnorm", m, k, gsf, with_w)
    xb = W.small_case(m, k, seed=11 * m + k, std=2.0, outlier_frac=0.01)
    wb = W.small_case(1, k, seed=k + 3, std=1.0)[0] if with_w else None
    x = dev_bf16(xb)
    wt = None if wb is None else dev_bf16(wb)
    p, sf = bsp.bsp_nvfp4_quantize_rmsnorm(x, scalar(gsf), wt, 1e-6)
    check_fused(p, sf, xb, wb, 1e-6, gsf, f"quantize_rmsnorm {m}x{k}")
    # the fused bytes are the NVFP4 quantize of the standalone kernel's output (same arithmetic)
    p2, sf2 = bsp.bsp_nvfp4_quantize(bsp.bsp_rmsnorm_bf16(x, wt, 1e-6), scalar(gsf))
    assert torch.equal(p, p2) and torch.equal(sf, sf2)


def test_rmsnorm_strided_unaligned_and_zero_rows():
    """Row strides above K, inputs off 16-byte alignment (element-wise path), all-zero rows (y = 0,
    scale 0x00) and a large eps."""
    m, k = 70, 96
    xb = W.small_case(m, k, seed=21, std=3.0)
    xb[5] = 0
    xb[40] = 0x8000                                  # -0.0 everywhere
    big = np.zeros((m, k + 24), dtype=np.uint16)
    big[:, :k] = xb
    xs = dev_bf16(big)[:, :k]                        # ld = K + 24
    for eps in (1e-6, 0.5):
        out = torch.zeros((m, k + 8), dtype=torch.bfloat16, device="cuda")
        bsp.bsp_rmsnorm_bf16(xs, None, eps, out=out[:, :k])
        got = host_bits(out[:, :k])
        check_norm(got, xb, None, eps, f"rmsnorm strided eps={eps}")
        assert not host_bits(out[:, k:]).any()       # nothing written past K
        assert np.array_equal(got[5], xb[5]) and np.array_equal(got[40], xb[40])
        p, sf = bsp.bsp_nvfp4_quantize_rmsnorm(xs, scalar(1.0), None, eps)
        check_fused(p, sf, xb, None, eps, 1.0, f"quantize_rmsnorm strided eps={eps}")
    # unaligned: one element in, so neither x nor the output is 16-byte aligned
    flat = dev_bf16(np.concatenate([[0], xb.ravel()]).astype(np.uint16))
    xu = flat[1:].view(m, k)
    ou = torch.zeros(m * k + 1, dtype=torch.bfloat16, device="cuda")[1:].view(m, k)
    wb = W.small_case(1, k, seed=9, std=1.0)[0]
    flat_w = dev_bf16(np.concatenate([[0], wb]).astype(np.uint16))
    bsp.bsp_rmsnorm_bf16(xu, flat_w[1:], 1e-6, out=ou)
    check_norm(host_bits(ou), xb, wb, 1e-6, "rmsnorm unaligned")
    p, sf = bsp.bsp_nvfp4_quantize_rmsnorm(xu, scalar(1.0), flat_w[1:], 1e-6)
    check_fused(p, sf, xb, wb, 1e-6, 1.0, "quantize_rmsnorm unaligned")


def test_quantize_rmsnorm_packed_not_16_byte_aligned():
    """A packed output 4-byte but not 16-byte aligned at K % 32 == 0: each lane's four bytes are
    stored instead of 16-byte row pieces; the bytes meet the same bar against the oracle chain."""
    m, k = 130, 512
    xb = W.small_case(m, k, seed=23, outlier_frac=0.02)
    p = torch.zeros(m * (k // 2) + 4, dtype=torch.uint8, device="cuda")[4:].view(m, k // 2)
    _, sf = bsp.bsp_nvfp4_quantize_rmsnorm(dev_bf16(xb), scalar(1.0), None, 1e-6, packed=p)
    check_fused(p, sf, xb, None, 1e-6, 1.0, "rmsnorm quantize, packed at a 4-byte offset")


def test_rmsnorm_empty_input():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert bsp.bsp_rmsnorm_bf16(x).shape == (0, 64)
    p, sf = bsp.bsp_nvfp4_quantize_rmsnorm(x, scalar(1.0))
    assert p.shape == (0, 32) and sf.numel() == 0


def test_quantize_rmsnorm_full_size_sampled_rows():
    """X[32760, 5120] of the Wan-14B layers (outlier channels), in the launch configuration the
    bench times; sampled rows against the oracle chain, every padding scale byte checked."""
    xb = tensor_bits(4, "X")
    m, k = xb.shape
    say("full-size quantize_rmsnorm", m, k)
    x = dev_bf16(xb)
    p, sf = bsp.bsp_nvfp4_quantize_rmsnorm(x, scalar(1.0), None, 1e-6)
    rows = np.unique(np.concatenate([np.random.default_rng(5).integers(0, m, 48), [0, 127, 128, m - 1]]))
    ri = torch.from_numpy(rows).cuda()
    rp_, cp_ = N.sf_padded_shape(m, k)
    lin = N.unswizzle_128x4(host_u8(sf).ravel(), rp_, cp_)
    y = R.rms_norm(R.bf16_bits_to_f64(xb[rows]), None, 1e-6)
    rp, rs = N.quantize(A.f64_to_bf16_bits(y), np.float32(1.0), layout="linear")
    amb = ambiguous(y, norm_rel_bound(k)).reshape(len(rows), k // 16, 16).any(axis=-1)
    say("full-size ambiguous blocks:", int(amb.sum()), "of", amb.size)
    assert amb.mean() < 0.05
    assert_nvfp4_blocks(host_u8(p[ri]), lin[rows], rp, rs, ~amb, "full-size quantize_rmsnorm")
    assert np.all(lin[m:] == 0)


@pytest.mark.parametrize("k", [96, 5120, 20000])
def test_rmsnorm_tiny_and_huge_rows(k):
    """Rows whose squares leave fp32's range (|x| near 2^-70 or 2^70 and beyond; eps = 2^-100 so it
    does not dominate): the fp64 sum of squares keeps them exact. Both kernels against the
    oracle."""
    say("rmsnorm tiny/huge", k)
    base = W.small_case(8, k, seed=k + 31, std=1.0)
    scale = np.array([2.0 ** -70, 2.0 ** -64, 2.0 ** -40, 1.0, 2.0 ** 20, 2.0 ** 62, 2.0 ** 70,
                      2.0 ** 100])[:, None]
    xb = W.f32_to_bf16_bits((W.bf16_bits_to_f32(base).astype(np.float64) * scale).astype(np.float32))
    eps = 2.0 ** -100
    x = dev_bf16(xb)
    check_norm(host_bits(bsp.bsp_rmsnorm_bf16(x, None, eps)), xb, None, eps, f"tiny/huge {k}")
    p, sf = bsp.bsp_nvfp4_quantize_rmsnorm(x, scalar(1.0), None, eps)
    check_fused(p, sf, xb, None, eps, 1.0, f"quantize tiny/huge {k}")


def test_quantize_rmsnorm_nonfinite_rows():
    """Rows holding an inf or a NaN: their RMS is infinite or NaN, so y is +-0 or NaN there, which
    the quantize encodes as nan_to_num gives it (zero codes, signed zeros kept); the other rows as
    usual. Bit-exact against the oracle chain on every byte: each finite row is +-2^e for one e per
    row, so its y is +-1 / sqrt(1 + eps 2^-2e), within 3e-5 of +-1 and far from a bf16 rounding
    boundary (no rounding-ambiguous values)."""
    say("quantize_rmsnorm nonfinite rows")
    m, k = 140, 512
    rng = np.random.default_rng(71)
    e = rng.integers(-2, 4, (m, 1))
    xb = W.f32_to_bf16_bits(np.ldexp(np.where(rng.integers(0, 2, (m, k)) == 1, -1.0, 1.0),
                                     np.broadcast_to(e, (m, k))).astype(np.float32))
    xb[3, 17] = 0x7F80           # +inf
    xb[4, 100] = 0xFF80          # -inf
    xb[5, 9] = 0x7FC0            # NaN
    xb[6] = 0x7F81               # a row of NaN patterns
    p, sf = bsp.bsp_nvfp4_quantize_rmsnorm(dev_bf16(xb), scalar(1.0), None, 1e-6)
    rp, rs = N.quantize(R.rms_norm_bf16_bits(xb, None, 1e-6), np.float32(1.0))
    assert np.array_equal(host_u8(p), rp)
    assert np.array_equal(host_u8(sf).ravel(), rs)
