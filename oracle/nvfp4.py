"""NVFP4 oracle: weight global scale, alpha, quantize, the 128x4 scale layout, dequant, mm_fp4.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Operation statements followed (pages named by title, section = function on the page):

* FastVideo nvfp4_qat_config.py, ``convert_model_to_fp4``: the weight global
  (encode) scale is (448*6) / amax(|W|) with NaN/inf replaced first; only the
  reduced scalar is fp32.  SGLang nvfp4_online.py, ``_quantize_weight_nvfp4``:
  when amax is 0 the decode scale is 1, so the encode scale is 1 (reading U8).
* FastVideo nvfp4_config.py, ``convert_model_to_nvfp4``: alpha for the weight is
  kept in fp32 as 1/gsf; ``NVFP4QuantizeMethod.apply`` divides it by the
  activation global scale. FastVideo nvfp4_qat_config.py, ``apply``:
  alpha = 1/(x_gsf * w_gsf) with a static activation global scale of 1.0.
* FastVideo nvfp4_config.py, ``_nvfp4_quantize``: for the swizzled layouts the
  rows are zero-padded to the 128-row tile, quantized, and the packed values are
  narrowed back to the logical rows while the scales keep the padded rows; the
  shape kernel gives packed [m, (k+1)//2] and scales [m, (k+15)//16] bytes.
* FastVideo nvfp4_config.py, module docstring: e2m1 values, fp32 alpha,
  layout_128x4, group size 16 along K; ``_mm_fp4`` computes
  out = alpha * (a @ b) with b the transposed view of the [N, K/2] weight.

Readings where the pages are silent (U-numbers as listed in the design notes):
U1 fp32 op order in the quantizer (below); U2 e4m3 scale RNE + saturate to 448;
U3 e2m1 RNE + saturate to 6; U4 sign of zero kept; U5 even k in the low nibble;
U6 the 128x4 byte offset (``sf_offset``); U7 padded scale bytes are 0x00;
U8 gsf = 1 when amax == 0; U9 NaN / +-inf are quantized as nan_to_num gives them;
U10 alpha from the fp32 gsf; U11 2688/amax is one IEEE fp32 division.

Fragment layout of the packed values (``frag_*``, ``quantize(..., packed_layout="frag")``). The
FastVideo nvfp4_config.py ``_nvfp4_quantize`` carries a ``do_shuffle`` switch for operands
pre-arranged for the matrix unit; it is off there and its arrangement is left to the library. This
one lets a wave read a 32-row by 64-element K step of an operand as one contiguous 1 KB: lane
i + 32 h reads the 16 bytes (32 elements) of row i at K offsets 32 h .. 32 h + 31 of the step.
Operand [R, K], K % 64 == 0, rows zero-padded to Rp = 32 * ceil(R / 32):
  packed byte (r, j) (elements 2j, 2j+1 of row r) ->
      ((r // 32) * (K // 64) + j // 32) * 1024 + ((j // 16) % 2 * 32 + r % 32) * 16 + j % 16.
The scales keep the 128x4 layout; only the order of the packed bytes differs.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_nan_to_num, e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode

F32 = np.float32
BLOCK = 16                       # elements per e4m3 scale along K
FP4_MAX = F32(6.0)               # largest e2m1 magnitude
E4M3_MAX = F32(448.0)            # largest e4m3 magnitude
GSF_NUMERATOR = F32(448.0 * 6.0)  # 2688, the pages' 448 * 6
C_SIXTH = F32(1.0) / F32(6.0)    # fl32(1/6) (0x3E2AAAAB)
BF16_MAX = F32(3.3895313892515355e38)  # largest finite bf16 (0x7F7F)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------------
# weight global scale
# ----------------------------------------------------------------------------------------
def tensor_amax(w_bits: np.ndarray) -> np.float32:
    """max |W| after nan_to_num (NaN -> 0, +-inf -> +-largest finite bf16)."""
    w = bf16_to_f32(w_bits)
    w = np.where(np.isnan(w), F32(0.0), w)
    w = np.where(np.isposinf(w), BF16_MAX, w)
    w = np.where(np.isneginf(w), -BF16_MAX, w)
    if w.size == 0:
        return F32(0.0)
    return F32(np.max(np.abs(w)))


def global_sf(w_bits: np.ndarray):
    """Returns (gsf, inv_gsf, amax), all fp32.

    gsf = fl32(2688 / amax), or 1.0 when amax == 0; inv_gsf = fl32(1 / gsf) is
    the fp32 weight alpha the FastVideo nvfp4_config.py page stores at load.
    One division, as both FastVideo pages write it; SGLang nvfp4_online.py takes the
    reciprocal of the decode scale fl32(amax / 2688) instead, one ulp off for some amax.
    """
    amax = tensor_amax(w_bits)
    gsf = F32(1.0) if amax == F32(0.0) else F32(GSF_NUMERATOR / amax)
    inv = F32(F32(1.0) / gsf)
    return gsf, inv, amax


def global_sf_4over6(w_bits: np.ndarray):
    """Weight scales of the 4over6 variant, returns (gsf, inv_gsf, amax), all fp32.

    SGLang nvfp4_online.py, ``_quantize_weight_nvfp4``: with the 4over6 switches the largest e4m3
    block scale is taken as 256 instead of 448; the decode scale is fl32(amax / (256 * 6)) (1 when
    amax is 0) and the encode scale handed to the quantizer is its fl32 reciprocal, in that order.
    """
    amax = tensor_amax(w_bits)
    dec = F32(1.0) if amax == F32(0.0) else F32(amax / F32(256.0 * 6.0))
    gsf = F32(F32(1.0) / dec)
    return gsf, F32(F32(1.0) / gsf), amax


# ----------------------------------------------------------------------------------------
# alpha
# ----------------------------------------------------------------------------------------
def alpha(x_gsf, w_gsf) -> np.float32:
    """alpha = fl32(1 / fl32(x_gsf * w_gsf)) (fp32 throughout, reading U10).

    FastVideo nvfp4_qat_config.py, ``apply``, writes this order. FastVideo nvfp4_config.py,
    ``NVFP4QuantizeMethod.apply``, divides the stored fp32 fl32(1/w_gsf) by x_gsf instead; the two
    agree bit for bit when x_gsf is 1 and may differ by one ulp otherwise."""
    return F32(F32(1.0) / F32(F32(x_gsf) * F32(w_gsf)))


# ----------------------------------------------------------------------------------------
# 128x4 scale layout (reading U6)
# ----------------------------------------------------------------------------------------
def sf_padded_shape(rows: int, k: int):
    """(Rp, Cp): rows padded to 128, scale columns (k/16) padded to 4."""
    cols = (k + BLOCK - 1) // BLOCK
    return ((rows + 127) // 128) * 128, ((cols + 3) // 4) * 4


def sf_offset(r, c, cp: int):
    """Byte offset of scale (row r, column c) in the 128x4 layout.

    512-byte tiles of 128 rows x 4 columns, tiles ordered row-tile-major; inside
    a tile the byte for (r, c) sits at (r % 32) * 16 + ((r // 32) % 4) * 4 + (c % 4).
    """
    r = np.asarray(r, dtype=np.int64)
    c = np.asarray(c, dtype=np.int64)
    tile = (r // 128) * (cp // 4) + (c // 4)
    return tile * 512 + (r % 32) * 16 + ((r // 32) % 4) * 4 + (c % 4)


def swizzle_128x4(sf_linear: np.ndarray) -> np.ndarray:
    """[Rp, Cp] row-major scale bytes -> flat 128x4-layout bytes."""
    rp, cp = sf_linear.shape
    out = np.zeros(rp * cp, dtype=np.uint8)
    r, c = np.meshgrid(np.arange(rp), np.arange(cp), indexing="ij")
    out[sf_offset(r, c, cp)] = sf_linear
    return out


def unswizzle_128x4(sf_flat: np.ndarray, rp: int, cp: int) -> np.ndarray:
    r, c = np.meshgrid(np.arange(rp), np.arange(cp), indexing="ij")
    return np.asarray(sf_flat, dtype=np.uint8)[sf_offset(r, c, cp)]


def sf_padded_shape_8x4(rows: int, k: int):
    """(Rp, Cp) for layout_8x4: rows padded to the 8-row tile, scale columns padded to 4.

    FastVideo nvfp4_config.py, ``_nvfp4_quantize``: the row tile is 8 for layout_8x4."""
    cols = (k + BLOCK - 1) // BLOCK
    return ((rows + 7) // 8) * 8, ((cols + 3) // 4) * 4


def sf_offset_8x4(r, c, cp: int):
    """Byte offset of scale (row r, column c) in the 8x4 layout (reading U23): 32-byte tiles of
    8 rows x 4 columns ordered row-tile-major, each tile stored row by row (r % 8) * 4 + (c % 4)."""
    r = np.asarray(r, dtype=np.int64)
    c = np.asarray(c, dtype=np.int64)
    tile = (r // 8) * (cp // 4) + (c // 4)
    return tile * 32 + (r % 8) * 4 + (c % 4)


def swizzle_8x4(sf_linear: np.ndarray) -> np.ndarray:
    rp, cp = sf_linear.shape
    out = np.zeros(rp * cp, dtype=np.uint8)
    r, c = np.meshgrid(np.arange(rp), np.arange(cp), indexing="ij")
    out[sf_offset_8x4(r, c, cp)] = sf_linear
    return out


def unswizzle_8x4(sf_flat: np.ndarray, rp: int, cp: int) -> np.ndarray:
    r, c = np.meshgrid(np.arange(rp), np.arange(cp), indexing="ij")
    return np.asarray(sf_flat, dtype=np.uint8)[sf_offset_8x4(r, c, cp)]


def _layout_fns(layout: str):
    if layout == "128x4":
        return sf_padded_shape, sf_offset, swizzle_128x4
    if layout == "8x4":
        return sf_padded_shape_8x4, sf_offset_8x4, swizzle_8x4
    raise ValueError(layout)


# ----------------------------------------------------------------------------------------
# quantize
# ----------------------------------------------------------------------------------------
def quantize_blocks(xf: np.ndarray, gsf) -> tuple:
    """Quantize fp32 values [rows, nblocks, 16] under global scale gsf (a scalar, or one per row).

    Returns (codes [rows, nblocks, 16] uint8, scale bytes [rows, nblocks] uint8).
    Reading U1, per 16-element block:
      a  = max |x_i|                       (exact)
      s  = fl32(g * fl32(a * fl32(1/6)))   (two multiplies, in this order)
      S  = e4m3(s), sd = value of S
      r  = 0 if sd == 0 else fl32(g / sd)  (one correctly rounded division)
      q_i = e2m1(fl32(x_i * r))
    """
    g = np.asarray(gsf, dtype=np.float32)
    if g.ndim:                   # one global scale per row (per-token scales): [rows] -> [rows, 1]
        g = g.reshape(g.shape + (1,) * (np.ndim(xf) - 1 - g.ndim))
    xf = np.asarray(xf, dtype=np.float32)
    a = np.max(np.abs(xf), axis=-1).astype(np.float32)
    s = (g * (a * C_SIXTH).astype(np.float32)).astype(np.float32)
    S = e4m3_encode(s)
    sd = e4m3_decode(S).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sd == F32(0.0), F32(0.0), g / np.where(sd == 0, F32(1.0), sd)).astype(np.float32)
    v = (xf * r[..., None]).astype(np.float32)
    return e2m1_encode(v), S


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2j] -> low nibble, [..., 2j+1] -> high nibble (reading U5)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def quantize(x_bits: np.ndarray, gsf, layout: str = "128x4", packed_layout: str = "rows"):
    """NVFP4-quantize bf16 X [M, K] (K % 16 == 0) under fp32 global scale ``gsf``.

    Returns (packed [M, K/2] uint8, sf) where sf is the flat 128x4-layout buffer of
    Rp*Cp bytes (layout "128x4"), the flat 8x4-layout buffer (layout "8x4", rows padded to 8),
    or the [M, K/16] row-major bytes (layout "linear").
    Padded scale rows/columns hold 0x00, the scale of an all-zero padded block.
    NaN and +-inf are encoded as 0 and +-largest finite bf16 (reading U9).
    packed_layout "frag" (K % 64 == 0) returns the packed bytes flat in the fragment layout.
    """
    x_bits = bf16_nan_to_num(x_bits)
    m, k = x_bits.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16")
    nb = k // BLOCK
    xf = bf16_to_f32(x_bits).reshape(m, nb, BLOCK)
    codes, S = quantize_blocks(xf, gsf)
    packed = pack_nibbles(codes.reshape(m, k))
    if packed_layout == "frag":
        packed = to_frag_packed(packed, k)
    elif packed_layout != "rows":
        raise ValueError(f"unknown packed layout {packed_layout!r}")
    if layout == "linear":
        return packed, S
    shape_fn, _, swz = _layout_fns(layout)
    rp, cp = shape_fn(m, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:m, :nb] = S
    return packed, swz(lin)


def row_global_sf(x_bits: np.ndarray) -> np.ndarray:
    """Per-token (per-row) encode scales: gsf_m = fl32(2688 / amax_m), 1.0 for an all-zero row.

    SGLang nvfp4_online.py, ``NVFP4OnlineConfig.__init__``: the weight scale is static while the
    activation fp32 scales are computed per token at run time. Reading U22: each row's scale
    follows the same rule as the tensor scale of ``global_sf`` applied to that row alone.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    return np.array([global_sf(x_bits[i:i + 1])[0] for i in range(x_bits.shape[0])],
                    dtype=np.float32)


def quantize_per_token(x_bits: np.ndarray, layout: str = "128x4"):
    """NVFP4 quantize with one encode scale per row; returns (packed, sf, gsf_rows [M] fp32).
    Row m is quantized exactly as ``quantize`` would with gsf = gsf_rows[m] (non-finite values
    substituted as there, reading U9)."""
    x_bits = bf16_nan_to_num(x_bits)
    m, k = x_bits.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16")
    g_rows = row_global_sf(x_bits)
    nb = k // BLOCK
    codes, S = quantize_blocks(bf16_to_f32(x_bits).reshape(m, nb, BLOCK), g_rows)
    packed = pack_nibbles(codes.reshape(m, k))
    if layout == "linear":
        return packed, S, g_rows
    rp, cp = sf_padded_shape(m, k)
    lin = np.zeros((rp, cp), dtype=np.uint8)
    lin[:m, :nb] = S
    return packed, swizzle_128x4(lin), g_rows


def quantize_rows(x_bits: np.ndarray, gsf):
    """Quantize a subset of rows; returns (packed rows, [rows, K/16] scale bytes)."""
    return quantize(x_bits, gsf, layout="linear")


# ----------------------------------------------------------------------------------------
# dequant and the GEMM
# ----------------------------------------------------------------------------------------
def frag_rows(rows: int) -> int:
    """Rows of a fragment-layout operand: R padded to a multiple of 32."""
    return (rows + 31) // 32 * 32


def frag_packed_offset(r, j, k: int):
    """Byte offset in the fragment layout of packed byte j (elements 2j, 2j+1) of row r."""
    r = np.asarray(r, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    fragment = (r // 32) * (k // 64) + j // 32      # 32-row tile, then 64-element K step
    lane = (j // 16) % 2 * 32 + r % 32              # lane half = which 32 elements of the step
    return fragment * 1024 + lane * 16 + j % 16


def to_frag_packed(packed: np.ndarray, k: int) -> np.ndarray:
    """packed [R, K/2] -> flat fragment-layout bytes (Rp * K/2), zero rows R..Rp-1."""
    if k % 64:
        raise ValueError("the fragment layout needs K % 64 == 0")
    rows = packed.shape[0]
    out = np.zeros(frag_rows(rows) * k // 2, dtype=np.uint8)
    r, j = np.meshgrid(np.arange(rows), np.arange(k // 2), indexing="ij")
    out[frag_packed_offset(r, j, k)] = packed
    return out


def from_frag_packed(fp: np.ndarray, rows, k: int) -> np.ndarray:
    """Flat fragment-layout bytes -> packed [R, K/2] for rows 0..rows-1 (an int) or the listed rows."""
    sel = np.arange(rows) if np.isscalar(rows) else np.asarray(rows, dtype=np.int64)
    r, j = np.meshgrid(sel, np.arange(k // 2), indexing="ij")
    return np.asarray(fp, dtype=np.uint8).ravel()[frag_packed_offset(r, j, k)]


def mm_fp4_frag(a_fp, a_sf, b_fp, b_sf, alpha_val, m: int, n: int, k: int) -> np.ndarray:
    """mm_fp4 for operands whose packed bytes are in the fragment layout (scales in 128x4)."""
    return mm_fp4(from_frag_packed(a_fp, m, k), a_sf, from_frag_packed(b_fp, n, k), b_sf, alpha_val,
                  m, n, k)


def dequant_rows(packed: np.ndarray, sf_flat: np.ndarray, rows, n_rows_total: int, k: int,
                 gsf=None, layout: str = "128x4") -> np.ndarray:
    """fp64 values e2m1(q) * e4m3(S) (/ gsf if given) of the selected rows."""
    rows = np.asarray(rows, dtype=np.int64)
    shape_fn, sf_offset, _ = _layout_fns(layout)
    rp, cp = shape_fn(n_rows_total, k)
    nb = k // BLOCK
    codes = unpack_nibbles(np.asarray(packed)[rows]).astype(np.int64)       # [r, K]
    r_idx = np.repeat(rows[:, None], nb, axis=1)
    c_idx = np.repeat(np.arange(nb)[None, :], rows.size, axis=0)
    sbytes = np.asarray(sf_flat, dtype=np.uint8)[sf_offset(r_idx, c_idx, cp)]
    sd = e4m3_decode(sbytes)                                                 # [r, nb]
    vals = e2m1_decode(codes).reshape(rows.size, nb, BLOCK) * sd[..., None]
    vals = vals.reshape(rows.size, k)
    if gsf is not None:
        vals = vals / np.float64(F32(gsf))
    return vals


def mm_fp4(a_packed, a_sf, b_packed, b_sf, alpha_val, m: int, n: int, k: int,
           row_chunk: int = 2048, a_layout: str = "128x4") -> np.ndarray:
    """C[m, n] = alpha * sum_k e2m1(A)*e4m3(SA) * e2m1(B)*e4m3(SB) in fp64 ([M, N]).

    A is packed [M, K/2] with 128x4 scales over M rows (8x4 with a_layout="8x4", the pages'
    use_8x4_sf_layout for the activation); B is packed [N, K/2] (K-major; the pages pass its
    transposed view) with 128x4 scales over N rows.
    """
    B = dequant_rows(b_packed, b_sf, np.arange(n), n, k)
    out = np.empty((m, n), dtype=np.float64)
    for r0 in range(0, m, row_chunk):
        r1 = min(r0 + row_chunk, m)
        A = dequant_rows(a_packed, a_sf, np.arange(r0, r1), m, k, layout=a_layout)
        out[r0:r1] = A @ B.T
    return np.float64(F32(alpha_val)) * out


def alpha_rows(x_gsf_rows, w_gsf) -> np.ndarray:
    """Per-token alphas fl32(1 / fl32(x_gsf[m] * w_gsf)) (the scalar alpha, row by row)."""
    xg = np.asarray(x_gsf_rows, dtype=np.float32)
    return (F32(1.0) / (xg * F32(w_gsf)).astype(np.float32)).astype(np.float32)


def mm_fp4_rowscale(a_packed, a_sf, b_packed, b_sf, x_gsf_rows, w_gsf, m: int, n: int, k: int):
    """mm_fp4 with per-token activation scales: row m of C is scaled by alpha_rows(...)[m]."""
    c = mm_fp4(a_packed, a_sf, b_packed, b_sf, F32(1.0), m, n, k)
    return c * alpha_rows(x_gsf_rows, w_gsf).astype(np.float64)[:, None]


def mm_fp4_entries(a_packed, a_sf, b_packed, b_sf, alpha_val, m: int, n: int, k: int,
                   rows, cols) -> np.ndarray:
    """The same C as ``mm_fp4``, only at entries (rows[i], cols[i]) (fp64)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    A = dequant_rows(a_packed, a_sf, ur, m, k)
    B = dequant_rows(b_packed, b_sf, uc, n, k)
    return np.float64(F32(alpha_val)) * np.einsum("ik,ik->i", A[ri], B[ci])
