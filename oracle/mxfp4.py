"""MXFP4 oracle: e2m1 elements with one e8m0 scale per 32 K-elements.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FastVideo nvfp4_config.py, ``_mm_fp4`` / its custom op: ``mm_fp4`` takes ``use_nvfp4``; with
``use_nvfp4=False`` the FP4 operands carry OCP MX scales instead of NVFP4's (the module docstring
contrasts NVFP4 with MX-FP4, "AMD's MX-FP4"). The vLLM-Omni mxfp8_config.py page
(``DiffusionMXFP8Config``) fixes the MX convention: 32 consecutive K elements share one e8m0
scale, per the OCP MX specification.

Reading (as for MXFP8, with the e2m1 element):
  Es   = clamp(floor(log2(amax)) - 2, -127, 127)  (2 = exponent of e2m1's largest power of two, 4),
  byte = Es + 127, 0x00 when amax == 0;
  q_i  = e2m1(fl32(x_i * 2^-Es)), nearest even, saturating at +-6.
Scales use the same 128x4 layout as NVFP4's (one byte per 32 K elements instead of 16), the
layout ``mm_fp4`` takes for both kinds of operands.

Fragment layout (``layout="frag"``). The FastVideo quantize op carries a ``do_shuffle`` switch for
operands pre-arranged for the matrix unit, always off there and never defined on the pages: the
arrangement is the library's. This one follows gfx950's block-scaled MFMA
(v_mfma_scale_f32_32x32x64_f8f6f4), whose lane i + 32 h reads, for a 32-row tile and a 64-element
K step, row i's 32-element block h of that step (16 bytes of e2m1) and that block's e8m0 scale.
Operand [R, K], K % 256 == 0, rows padded with zeros to Rp = 32 * ceil(R / 32):
  packed byte (r, j) (elements 2j, 2j+1 of row r) ->
      ((r // 32) * (K // 64) + j // 32) * 1024 + ((j // 16) % 2 * 32 + r % 32) * 16 + j % 16;
  scale (r, b) (block b = k // 32 of row r) ->
      ((r // 32) * (K // 256) + b // 8) * 256 + (b % 2 * 32 + r % 32) * 4 + (b // 2) % 4.
Only the byte order differs from the linear layout: same codes, same scales.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_nan_to_num, e2m1_decode, e2m1_encode, e8m0_decode
from .nvfp4 import pack_nibbles, sf_offset, swizzle_128x4, unpack_nibbles

F32 = np.float32
GROUP = 32
E2M1_EMAX = 2


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def sf_padded_shape(rows: int, k: int):
    cols = (k + GROUP - 1) // GROUP
    return ((rows + 127) // 128) * 128, ((cols + 3) // 4) * 4


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)
    es = np.clip(e.astype(np.int64) - 1 - E2M1_EMAX, -127, 127)
    return np.where(a == 0.0, -127, es)


def quantize_blocks(xf: np.ndarray):
    """fp32 [rows, ngroups, 32] -> (e2m1 codes, e8m0 bytes [rows, ngroups])."""
    xf = np.asarray(xf, dtype=np.float32)
    es = scale_exponent(np.max(np.abs(xf), axis=-1))
    inv = np.ldexp(np.float32(1.0), (-es).astype(np.int32)).astype(np.float32)
    v = (xf * inv[..., None]).astype(np.float32)
    return e2m1_encode(v), (es + 127).astype(np.uint8)


def quantize(x_bits: np.ndarray, layout: str = "128x4"):
    """bf16 X [M, K] (K % 32 == 0) -> (packed [M, K/2], scales: flat 128x4 bytes or [M, K/32]);
    layout "frag" (K % 256 == 0): both flat in the fragment layout."""
    x_bits = bf16_nan_to_num(x_bits)   # NaN -> 0, +-inf -> +-largest finite bf16 (reading U9)
    m, k = x_bits.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 32")
    ng = k // GROUP
    codes, s = quantize_blocks(bf16_to_f32(x_bits).reshape(m, ng, GROUP))
    packed = pack_nibbles(codes.reshape(m, k))
    if layout == "linear":
        return packed, s
    if layout == "frag":
        return to_frag(packed, s, k)
    rp, cp = sf_padded_shape(m, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:m, :ng] = s
    return packed, swizzle_128x4(lin)


def frag_rows(rows: int) -> int:
    return (rows + 31) // 32 * 32


def frag_packed_offset(r, j, k: int):
    """Byte offset in the fragment layout of packed byte j (elements 2j, 2j+1) of row r."""
    r = np.asarray(r, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    row_tile, lane_row = r // 32, r % 32
    k_step, half, byte = j // 32, (j // 16) % 2, j % 16
    return (row_tile * (k // 64) + k_step) * 1024 + (half * 32 + lane_row) * 16 + byte


def frag_sf_offset(r, b, k: int):
    """Byte offset in the fragment layout of the scale of block b (K elements 32b..32b+31) of row r."""
    r = np.asarray(r, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    row_tile, lane_row = r // 32, r % 32
    group, step_in_group, half = b // 8, (b // 2) % 4, b % 2
    return (row_tile * (k // 256) + group) * 256 + (half * 32 + lane_row) * 4 + step_in_group


def to_frag(packed: np.ndarray, scales: np.ndarray, k: int):
    """(packed [R, K/2], linear scales [R, K/32]) -> flat fragment-layout (packed, scales), zero rows
    to the next multiple of 32."""
    if k % 256:
        raise ValueError("the fragment layout needs K % 256 == 0")
    rows = packed.shape[0]
    rp = frag_rows(rows)
    fp = np.zeros(rp * k // 2, dtype=np.uint8)
    fs = np.zeros(rp * k // 32, dtype=np.uint8)
    r, j = np.meshgrid(np.arange(rows), np.arange(k // 2), indexing="ij")
    fp[frag_packed_offset(r, j, k)] = packed
    r, b = np.meshgrid(np.arange(rows), np.arange(k // 32), indexing="ij")
    fs[frag_sf_offset(r, b, k)] = scales
    return fp, fs


def from_frag(fp: np.ndarray, fs: np.ndarray, rows: int, k: int):
    """Flat fragment-layout (packed, scales) -> (packed [rows, K/2], linear scales [rows, K/32])."""
    fp = np.asarray(fp, dtype=np.uint8).ravel()
    fs = np.asarray(fs, dtype=np.uint8).ravel()
    r, j = np.meshgrid(np.arange(rows), np.arange(k // 2), indexing="ij")
    packed = fp[frag_packed_offset(r, j, k)]
    r, b = np.meshgrid(np.arange(rows), np.arange(k // 32), indexing="ij")
    return packed, fs[frag_sf_offset(r, b, k)]


def dequant_linear(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """packed [R, K/2] with linear e8m0 scales [R, K/32] -> fp64 values [R, K]."""
    rows, k = packed.shape[0], packed.shape[1] * 2
    codes = unpack_nibbles(np.asarray(packed)).astype(np.int64)
    vals = e2m1_decode(codes).reshape(rows, k // GROUP, GROUP) * e8m0_decode(scales)[..., None]
    return vals.reshape(rows, k)


def mm_mxfp4_frag(a_fp, a_fs, b_fp, b_fs, alpha_val, m: int, n: int, k: int) -> np.ndarray:
    """C[m, n] = alpha * sum_k A[m, k] B[n, k] in fp64 for fragment-layout operands."""
    A = dequant_linear(*from_frag(a_fp, a_fs, m, k))
    B = dequant_linear(*from_frag(b_fp, b_fs, n, k))
    return np.float64(F32(alpha_val)) * (A @ B.T)


def dequant_rows(packed, sf_flat, rows, n_rows_total: int, k: int) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    _, cp = sf_padded_shape(n_rows_total, k)
    ng = k // GROUP
    codes = unpack_nibbles(np.asarray(packed)[rows]).astype(np.int64)
    r_idx = np.repeat(rows[:, None], ng, axis=1)
    c_idx = np.repeat(np.arange(ng)[None, :], rows.size, axis=0)
    sv = e8m0_decode(np.asarray(sf_flat, dtype=np.uint8)[sf_offset(r_idx, c_idx, cp)])
    vals = e2m1_decode(codes).reshape(rows.size, ng, GROUP) * sv[..., None]
    return vals.reshape(rows.size, k)


def mm_mxfp4(a_packed, a_sf, b_packed, b_sf, alpha_val, m: int, n: int, k: int,
             row_chunk: int = 2048) -> np.ndarray:
    """C[m, n] = alpha * sum_k dequant(A)[m, k] * dequant(B)[n, k] in fp64."""
    B = dequant_rows(b_packed, b_sf, np.arange(n), n, k)
    out = np.empty((m, n), dtype=np.float64)
    for r0 in range(0, m, row_chunk):
        r1 = min(r0 + row_chunk, m)
        out[r0:r1] = dequant_rows(a_packed, a_sf, np.arange(r0, r1), m, k) @ B.T
    return np.float64(F32(alpha_val)) * out


def mm_mxfp4_entries(a_packed, a_sf, b_packed, b_sf, alpha_val, m: int, n: int, k: int, rows, cols):
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    A = dequant_rows(a_packed, a_sf, ur, m, k)
    B = dequant_rows(b_packed, b_sf, uc, n, k)
    return np.float64(F32(alpha_val)) * np.einsum("ik,ik->i", A[ri], B[ci])
