"""Shared helpers of the GPU parity tests (device transfer, seeded inputs, GEMM metrics, oracle
references).

Expected values always come from ``oracle/`` applied to the same seeded input the GPU receives
(the bf16 tensors or the operand bytes a test generates), never to bytes a GPU kernel produced.
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import workloads as W
from oracle import activations as A
from oracle import formats as F
from oracle import nvfp4 as N

DEV = "cuda"

# GEMM tolerances (fp32 accumulation of exact fp16/e4m3 products, then one bf16 rounding)
REL_FRO = 1e-3      # relative Frobenius error
MAX_REL = 8e-3      # max |C - ref| / max |ref| after the bf16 cast


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def scalar(v) -> torch.Tensor:
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device=DEV)


@functools.lru_cache(maxsize=8)
def tensor_bits(cfg: int, name: str) -> np.ndarray:
    return W.generate(W.config(cfg).tensor(name))


def bf16_of(ref: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(A.f64_to_bf16_bits(ref)).astype(np.float64)


def gemm_metrics(c: np.ndarray, ref: np.ndarray) -> dict:
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nref = np.linalg.norm(ref)
    mref = np.max(np.abs(ref))
    b = bf16_of(ref)
    return {
        "rel_fro": float(np.linalg.norm(c - ref) / nref) if nref else float(np.linalg.norm(c)),
        "rel_fro_vs_bf16_ref": float(np.linalg.norm(c - b) / nref) if nref else 0.0,
        "rel_fro_of_bf16_ref": float(np.linalg.norm(b - ref) / nref) if nref else 0.0,
        "max_rel": float(np.max(np.abs(c - ref)) / mref) if mref else float(np.max(np.abs(c))),
    }


def assert_gemm_f32(c: np.ndarray, ref: np.ndarray, what: str = ""):
    m = gemm_metrics(c, ref)
    say(what, "fp32 out", m)
    assert m["rel_fro"] <= REL_FRO, (what, m)


def assert_gemm_bf16(c: np.ndarray, ref: np.ndarray, what: str = ""):
    """bf16 output against the fp64 reference: its relative Frobenius error exceeds that of the
    reference's own nearest-even bf16 rounding by at most REL_FRO (a bf16 cast alone is about
    1.7e-3 from the fp64 product), and every element is within MAX_REL * max|ref|. Measuring the
    excess over the perfectly rounded result rather than the distance to it allows the one-ulp
    flips at exact bf16 ties: MX operands are small integers times powers of two, so a product can
    sit exactly on a tie in fp32 and round to even while the exact sum, nudged by terms below fp32's
    reach, rounds the other way."""
    m = gemm_metrics(c, ref)
    say(what, "bf16 out", m)
    assert m["rel_fro"] <= m["rel_fro_of_bf16_ref"] + REL_FRO, (what, m)
    assert m["max_rel"] <= MAX_REL, (what, m)


def sample_entries(m: int, n: int, count: int, seed: int):
    """Random (row, col) pairs plus the four corners and the last rows/cols (ragged tails)."""
    rng = np.random.default_rng(seed)
    r = rng.integers(0, m, count)
    c = rng.integers(0, n, count)
    extra_r = np.array([0, 0, m - 1, m - 1] + [m - 1 - i for i in range(16)])
    extra_c = np.array([0, n - 1, 0, n - 1] + [n - 1 - 3 * i % n for i in range(16)])
    return np.concatenate([r, extra_r]), np.concatenate([c, extra_c])


def gather(t: torch.Tensor, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    ri = torch.from_numpy(rows).to(DEV)
    ci = torch.from_numpy(cols).to(DEV)
    return t[ri, ci].float().cpu().numpy().astype(np.float64)


# ------------------------------------------------------------------------------ oracle references
def oracle_quantize_chunked(x_bits: np.ndarray, gsf, chunk: int = 256):
    """N.quantize of a large bf16 matrix in row chunks (the quantization is row by row; small
    chunks keep numpy's temporaries in cache): (packed [M, K/2], flat 128x4 scale buffer)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    m, k = x_bits.shape
    parts = [N.quantize(x_bits[i: i + chunk], gsf, layout="linear") for i in range(0, m, chunk)]
    packed = np.concatenate([p for p, _ in parts])
    rp, cp = N.sf_padded_shape(m, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:m, : k // 16] = np.concatenate([s for _, s in parts])
    return packed, N.swizzle_128x4(lin)


def oracle_linear_entries(xb: np.ndarray, wb: np.ndarray, rows: np.ndarray, cols: np.ndarray,
                          x_gsf: float = 1.0) -> np.ndarray:
    """The oracle's NVFP4 linear layer y = x w^T at entries (rows[i], cols[i]), from the bf16 bits
    of x [M, K] and w [N, K]: w's global scale from the whole of w, then only the needed rows of x
    (static global scale x_gsf) and of w are quantized, and their exact product taken."""
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    rg = N.global_sf(wb)[0]
    px, sx = N.quantize(xb[ur], np.float32(x_gsf))
    pw, sw = N.quantize(wb[uc], rg)
    return N.mm_fp4_entries(px, sx, pw, sw, N.alpha(x_gsf, rg), len(ur), len(uc), xb.shape[1], ri, ci)


def gelu_rounding_ambiguous(y_bits: np.ndarray, eps: float = 2.0 ** -20) -> np.ndarray:
    """bf16 inputs whose fp64 GELU lies within eps (relative; about 8 fp32 ulps) of a bf16 rounding
    boundary, so that a GELU accurate to a few fp32 ulps may round it either way (about one input
    in 2^11)."""
    y = (np.asarray(y_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    g = A.gelu_tanh(y.astype(np.float64))
    return A.f64_to_bf16_bits(g * (1 - eps)) != A.f64_to_bf16_bits(g * (1 + eps))


def assert_nvfp4_blocks(got_packed, got_sf_lin, ref_packed, ref_sf_lin, exact: np.ndarray,
                        what: str = "") -> float:
    """NVFP4 rows (packed [M, K/2], scales [M, >= K/16]) against reference rows: bit-exact in the
    16-element blocks where `exact` [M, K/16] is set; in the others the scale code within one step
    and every element within one e2m1 step. Returns the fraction of blocks that differ."""
    gp, rp = np.asarray(got_packed), np.asarray(ref_packed)
    m, k = gp.shape[0], gp.shape[1] * 2

    def codes(p):
        return np.stack([p & 0xF, p >> 4], axis=-1).reshape(m, k // 16, 16)

    gc, rc = codes(gp), codes(rp)
    gs = np.asarray(got_sf_lin)[:m, : k // 16]
    rs = np.asarray(ref_sf_lin)[:m, : k // 16]
    assert np.array_equal(gs[exact], rs[exact]), what
    assert np.array_equal(gc[exact], rc[exact]), what
    assert np.all(np.abs(gs.astype(int) - rs) <= 1), what
    assert np.all(np.abs(F.e2m1_decode(gc) - F.e2m1_decode(rc)) <= 2.0), what
    return float(np.mean((gs != rs) | np.any(gc != rc, axis=-1)))


def assert_nvfp4_of_gelu(got_packed: np.ndarray, got_sf_lin: np.ndarray, y_bits: np.ndarray, gsf,
                         what: str = "", max_ambiguous: float = 0.03):
    """The GPU's NVFP4 encoding of gelu(y) (packed [M, K/2], scales unswizzled to [M, K/16])
    against the oracle's own chain on the same bf16 y: fp64 GELU rounded once to bf16, then the
    NVFP4 quantize. The GPU's GELU (hardware exp2 and reciprocal) is within a few fp32 ulps, so
    every 16-element block without a rounding-ambiguous value must be bit-exact (the others within
    one step, assert_nvfp4_blocks). For smooth data about 16 / 2^11 of the blocks are ambiguous;
    inputs built from rounding ties and tiny values may set max_ambiguous higher."""
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    m, k = y_bits.shape
    rp, rs = N.quantize(A.gelu_tanh_bf16_bits(y_bits), np.float32(gsf), layout="linear")
    amb = gelu_rounding_ambiguous(y_bits).reshape(m, k // 16, 16).any(axis=-1)
    say(what, "gelu-ambiguous blocks:", int(amb.sum()), "of", amb.size)
    assert amb.mean() < max_ambiguous, (what, amb.mean())
    assert_nvfp4_blocks(got_packed, got_sf_lin, rp, rs, ~amb, what)
