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
REL_FRO_FP4_F32 = 1e-5   # mm_fp4's fp32 output: exact fp16 products summed in fp32 (K up to ~2^14)


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


def assert_gemm_f32(c: np.ndarray, ref: np.ndarray, what: str = "", tol: float = REL_FRO):
    """C11 (i): fp32 output within `tol` (relative Frobenius) of the fp64 reference."""
    m = gemm_metrics(c, ref)
    say(what, "fp32 out", m)
    assert m["rel_fro"] <= tol, (what, m, tol)


def f32_bf16_ties(c32: np.ndarray) -> np.ndarray:
    """Elements whose fp32 value lies exactly halfway between two bf16 values (low 16 bits 0x8000).
    Both neighbours are equally near such a value, so its nearest-even bf16 need not be the one the
    exact sum rounds to: MX operands are small integers times powers of two, and their fp32 sums
    land on such ties far more often than random data would."""
    b = np.ascontiguousarray(c32, dtype=np.float32).view(np.uint32)
    return (b & np.uint32(0xFFFF)) == np.uint32(0x8000)


def assert_bf16_is_rne_of_f32(c16_bits: np.ndarray, c32: np.ndarray, what: str = ""):
    """The bf16 epilogue rounds the same fp32 value the fp32 epilogue stores, to nearest even."""
    want = W.f32_to_bf16_bits(np.asarray(c32, dtype=np.float32))
    assert np.array_equal(np.asarray(c16_bits, dtype=np.uint16), want), what


def assert_gemm_bf16(c16: np.ndarray, ref: np.ndarray, c32: np.ndarray, what: str = ""):
    """C11 (ii) and (iii) for bf16 output, given the fp32 output c32 of the same GEMM:
    (ii) ||C16 - bf16(ref)||_F <= REL_FRO ||ref||_F, summed over every element whose fp32 value is
         not an exact bf16 tie (f32_bf16_ties: there either neighbour is a correct rounding);
    (iii) max |C16 - ref| <= MAX_REL max |ref| over all elements."""
    c16 = np.asarray(c16, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = gemm_metrics(c16, ref)
    tie = f32_bf16_ties(c32)
    d = c16 - bf16_of(ref)
    d[tie] = 0.0
    nref = np.linalg.norm(ref)
    m["rel_fro_vs_bf16_ref_outside_ties"] = float(np.linalg.norm(d) / nref) if nref else float(np.linalg.norm(d))
    m["tie_fraction"] = float(np.mean(tie))
    say(what, "bf16 out", m)
    assert m["rel_fro_vs_bf16_ref_outside_ties"] <= REL_FRO, (what, m)
    assert m["max_rel"] <= MAX_REL, (what, m)


def gather_bits(t: torch.Tensor, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of t at entries (rows[i], cols[i])."""
    ri = torch.from_numpy(rows).to(DEV)
    ci = torch.from_numpy(cols).to(DEV)
    return t.view(torch.int16)[ri, ci].cpu().numpy().view(np.uint16)


def check_gemm_outputs(t16: torch.Tensor, t32: torch.Tensor, ref: np.ndarray, what: str = "",
                       rows=None, cols=None, f32_tol: float = REL_FRO):
    """Both outputs of one GEMM, bf16 (t16) and fp32 (t32), on every element or at sampled entries
    (rows[i], cols[i]) against the oracle's fp64 values `ref` there: C11 (i) on the fp32 output
    (bound f32_tol), the bf16 output equal to the nearest-even rounding of the fp32 one bit for
    bit, and C11 (ii), (iii) on the bf16 output."""
    if rows is None:
        c32 = t32.contiguous().cpu().numpy().astype(np.float32)
        b16 = host_bits(t16)
    else:
        c32 = gather(t32, rows, cols).astype(np.float32)
        b16 = gather_bits(t16, rows, cols)
    assert_gemm_f32(c32.astype(np.float64), ref, what, f32_tol)
    assert_bf16_is_rne_of_f32(b16, c32, what)
    assert_gemm_bf16(W.bf16_bits_to_f32(b16).astype(np.float64), ref, c32, what)


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


# The kernels' GELU table covers the bf16 inputs with |x| in [2^-12, 2^6) (magnitude bits in
# [115 << 7, 133 << 7)) and holds the correctly rounded bf16 of gelu there; other inputs take an fp32
# evaluation accurate to a few fp32 ulps.
GELU_TABLE_MAG = (115 << 7, 133 << 7)


def gelu_in_table(y_bits: np.ndarray) -> np.ndarray:
    mag = np.asarray(y_bits, dtype=np.uint16) & 0x7FFF
    return (mag >= GELU_TABLE_MAG[0]) & (mag < GELU_TABLE_MAG[1])


def gelu_rounding_ambiguous(y_bits: np.ndarray, eps: float = 2.0 ** -20) -> np.ndarray:
    """bf16 inputs outside the GELU table whose fp64 GELU lies within eps (relative; about 8 fp32
    ulps) of a bf16 rounding boundary, so that the fp32 evaluation may round it either way. Inputs
    in the table are correctly rounded, never ambiguous."""
    y = (np.asarray(y_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    g = A.gelu_tanh(y.astype(np.float64))
    near = A.f64_to_bf16_bits(g * (1 - eps)) != A.f64_to_bf16_bits(g * (1 + eps))
    return near & ~gelu_in_table(y_bits)


def e2m1_rank(codes: np.ndarray) -> np.ndarray:
    """Position of each e2m1 code on the signed grid: magnitude index 0..7 with the code's sign
    (both zeros at 0), so that neighbouring grid values differ by one."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 8, -(c & 7), c & 7)


def assert_nvfp4_blocks(got_packed, got_sf_lin, ref_packed, ref_sf_lin, exact: np.ndarray,
                        what: str = "") -> float:
    """NVFP4 rows (packed [M, K/2], scales [M, >= K/16]) against reference rows: bit-exact in the
    16-element blocks where `exact` [M, K/16] is set; in the others the scale code within one step
    and every element within one step of the e2m1 grid. Returns the fraction of blocks that
    differ."""
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
    # one step of the signed e2m1 grid -6 .. -0.5, 0, 0.5 .. 6 (+0 and -0 are the same point)
    assert np.all(np.abs(e2m1_rank(gc) - e2m1_rank(rc)) <= 1), what
    return float(np.mean((gs != rs) | np.any(gc != rc, axis=-1)))


def assert_nvfp4_of_gelu(got_packed: np.ndarray, got_sf_lin: np.ndarray, y_bits: np.ndarray, gsf,
                         what: str = "", max_ambiguous: float = 0.03):
    """The GPU's NVFP4 encoding of gelu(y) (packed [M, K/2], scales unswizzled to [M, K/16])
    against the oracle's own chain on the same bf16 y: fp64 GELU rounded once to bf16, then the
    NVFP4 quantize. The GPU's GELU is correctly rounded inside its table and within a few fp32 ulps
    outside it, so every 16-element block without a rounding-ambiguous value (gelu_rounding_ambiguous)
    must be bit-exact (the others within one step, assert_nvfp4_blocks). Smooth data has almost no
    ambiguous blocks; inputs built from rounding ties and tiny values may set max_ambiguous higher."""
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    m, k = y_bits.shape
    rp, rs = N.quantize(A.gelu_tanh_bf16_bits(y_bits), np.float32(gsf), layout="linear")
    amb = gelu_rounding_ambiguous(y_bits).reshape(m, k // 16, 16).any(axis=-1)
    say(what, "gelu-ambiguous blocks:", int(amb.sum()), "of", amb.size)
    assert amb.mean() < max_ambiguous, (what, amb.mean())
    assert_nvfp4_blocks(got_packed, got_sf_lin, rp, rs, ~amb, what)
