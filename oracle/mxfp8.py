"""MXFP8 (W8A8) oracle: e4m3 elements with one e8m0 scale per 32 K-elements.

TEST INFRASTRUCTURE ONLY (see the package docstring).

vLLM-Omni mxfp8_config.py page, ``DiffusionMXFP8Config``: groups of 32
consecutive K elements share one e8m0 power-of-two scale, following the OCP MX
specification; ``create_weights`` stores the weight scales as uint8 bytes of
shape (rows, ceil(K/32)); ``NPUMxfp8LinearMethod._quantize_activation`` /
``_quant_matmul``: activations are quantized per call, the GEMM takes the
per-row (per-token) e8m0 scales of both operands with a [1, 1, 32] group and
returns the input's dtype; ``NPUMxfp8OnlineLinearMethod`` converts bf16 weights
to MXFP8 once after loading.

Reading U12 (the OCP MX scale rule; the page only cites the spec):
  E   = floor(log2(amax)) of the block's largest magnitude (exact, via frexp),
  Es  = clamp(E - 8, -127, 127)    (8 = exponent of e4m3's largest power of two, 2^8),
  byte = Es + 127, and byte 0x00 when amax == 0;
  q_i = e4m3(fl32(x_i * 2^-Es)), round to nearest even, saturate to +-448
  (values in (448, 512) therefore clamp to 448, as the floor rule implies).

Fragment layout (``quantize_frag``): the operand arrangement for the matrix unit (reading U29, as
for MXFP4 in ``oracle.mxfp4``), here for the e4m3 operand of gfx950's
v_mfma_scale_f32_32x32x64_f8f6f4. For a 32-row tile and a 64-element K step, lane i + 32 h of the
instruction holds 32 bytes of row i: its bytes 0-15 are elements 16h..16h+15 of the step's first
32-element block and bytes 16-31 the same half of the second block; its e8m0 scale is that of
block h of the step. Operand [R, K], K % 256 == 0, rows padded with zeros to Rp = 32 ceil(R/32):
  element (r, k) -> ((r // 32) * (K // 64) + k // 64) * 2048 + (k // 32) % 2 * 1024
                    + ((k // 16) % 2 * 32 + r % 32) * 16 + k % 16;
  scale (r, b)   -> as the MXFP4 fragment layout's scale offset.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_nan_to_num, e4m3_decode, e4m3_encode, e8m0_decode

F32 = np.float32
GROUP = 32
E4M3_EMAX = 8


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Es for each block amax (int64); amax == 0 gives -127 (byte 0x00)."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)                  # a = f * 2^e, f in [0.5, 1)  =>  floor(log2 a) = e - 1
    E = e.astype(np.int64) - 1
    es = np.clip(E - E4M3_EMAX, -127, 127)
    return np.where(a == 0.0, -127, es)


def quantize_blocks(xf: np.ndarray):
    """fp32 [rows, ngroups, 32] -> (e4m3 bytes, e8m0 bytes [rows, ngroups])."""
    xf = np.asarray(xf, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    es = scale_exponent(amax)
    inv = np.ldexp(np.float32(1.0), (-es).astype(np.int32)).astype(np.float32)   # 2^-Es, exact
    v = (xf * inv[..., None]).astype(np.float32)
    return e4m3_encode(v), (es + 127).astype(np.uint8)


def quantize(x_bits: np.ndarray):
    """bf16 X [M, K] (K % 32 == 0) -> (e4m3 [M, K] uint8, e8m0 [M, K/32] uint8), row-major."""
    x_bits = bf16_nan_to_num(x_bits)   # NaN -> 0, +-inf -> +-largest finite bf16 (reading U9)
    m, k = x_bits.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 32")
    xf = bf16_to_f32(x_bits).reshape(m, k // GROUP, GROUP)
    q, s = quantize_blocks(xf)
    return q.reshape(m, k), s


def dequant_rows(q: np.ndarray, sf: np.ndarray, rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    qv = e4m3_decode(np.asarray(q)[rows])                     # [r, K] fp64
    sv = e8m0_decode(np.asarray(sf)[rows])                    # [r, K/32]
    r, k = qv.shape
    return (qv.reshape(r, k // GROUP, GROUP) * sv[..., None]).reshape(r, k)


def mm_mxfp8(a_q, a_sf, b_q, b_sf, m: int, n: int, k: int, row_chunk: int = 2048) -> np.ndarray:
    """C[m, n] = sum_k dequant(A)[m, k] * dequant(B)[n, k] in fp64."""
    B = dequant_rows(b_q, b_sf, np.arange(n))
    out = np.empty((m, n), dtype=np.float64)
    for r0 in range(0, m, row_chunk):
        r1 = min(r0 + row_chunk, m)
        out[r0:r1] = dequant_rows(a_q, a_sf, np.arange(r0, r1)) @ B.T
    return out


def mm_mxfp8_entries(a_q, a_sf, b_q, b_sf, rows, cols) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    A = dequant_rows(a_q, a_sf, ur)
    B = dequant_rows(b_q, b_sf, uc)
    return np.einsum("ik,ik->i", A[ri], B[ci])


def frag_offset(r, k_idx, k: int):
    """Byte offset in the fragment layout of element k_idx of row r."""
    r = np.asarray(r, dtype=np.int64)
    k_idx = np.asarray(k_idx, dtype=np.int64)
    row_tile, lane_row = r // 32, r % 32
    k_step, block, half, byte = k_idx // 64, (k_idx // 32) % 2, (k_idx // 16) % 2, k_idx % 16
    return ((row_tile * (k // 64) + k_step) * 2048 + block * 1024
            + (half * 32 + lane_row) * 16 + byte)


def to_frag(q: np.ndarray, scales: np.ndarray, k: int):
    """(e4m3 [R, K], e8m0 [R, K/32]) -> flat fragment-layout (elements, scales), zero rows to the
    next multiple of 32."""
    from .mxfp4 import frag_rows, frag_sf_offset
    if k % 256:
        raise ValueError("the fragment layout needs K % 256 == 0")
    rows = q.shape[0]
    rp = frag_rows(rows)
    fq = np.zeros(rp * k, dtype=np.uint8)
    fs = np.zeros(rp * k // 32, dtype=np.uint8)
    r, c = np.meshgrid(np.arange(rows), np.arange(k), indexing="ij")
    fq[frag_offset(r, c, k)] = q
    r, b = np.meshgrid(np.arange(rows), np.arange(k // 32), indexing="ij")
    fs[frag_sf_offset(r, b, k)] = scales
    return fq, fs


def from_frag(fq: np.ndarray, fs: np.ndarray, rows: int, k: int):
    """Flat fragment-layout (elements, scales) -> (e4m3 [rows, K], e8m0 [rows, K/32])."""
    from .mxfp4 import frag_sf_offset
    fq = np.asarray(fq, dtype=np.uint8).ravel()
    fs = np.asarray(fs, dtype=np.uint8).ravel()
    r, c = np.meshgrid(np.arange(rows), np.arange(k), indexing="ij")
    q = fq[frag_offset(r, c, k)]
    r, b = np.meshgrid(np.arange(rows), np.arange(k // 32), indexing="ij")
    return q, fs[frag_sf_offset(r, b, k)]


def quantize_frag(x_bits: np.ndarray):
    """bf16 X [M, K] (K % 256 == 0) -> flat fragment-layout (elements, scales)."""
    q, s = quantize(x_bits)
    return to_frag(q, s, x_bits.shape[1])


def mm_mxfp8_frag(a_fq, a_fs, b_fq, b_fs, m: int, n: int, k: int) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] B[n, k] in fp64 for fragment-layout operands."""
    aq, asf = from_frag(a_fq, a_fs, m, k)
    bq, bsf = from_frag(b_fq, b_fs, n, k)
    return mm_mxfp8(aq, asf, bq, bsf, m, n, k)
