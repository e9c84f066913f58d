"""Element and scale codecs, built from the bit-field definitions of each format.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* e2m1 (FP4): 1 sign, 2 exponent bits with bias 1, 1 mantissa bit; no inf/NaN.
  Named as the NVFP4 element type on the FastVideo nvfp4_config.py page (module
  docstring) and defined in the OCP MX specification that the vLLM-Omni
  mxfp8_config.py page cites.
* e4m3 "fn" (FP8): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; the all-ones
  pattern S.1111.111 is NaN, there is no inf, so the largest finite value is
  1.75 * 2^8 = 448 (the SGLang nvfp4_online.py page takes its e4m3 maximum from
  the float8_e4m3fn format).
* e8m0 (scale): 8-bit biased exponent, value 2^(c-127); c = 255 is NaN (OCP MX).

Encoders round to nearest with ties to the even code and saturate to the largest
finite magnitude (readings U2/U3 of the design notes); the sign of the input is
kept, so -0.0 and negative values that round to zero encode as negative zero
(reading U4). Candidates are compared in fp64, where every difference involved
is exact.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------------------
# e2m1
# ----------------------------------------------------------------------------------------
def e2m1_decode_table() -> np.ndarray:
    """Value of every 4-bit code 0..15 (fp64)."""
    out = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        if e == 0:                      # subnormal: 2^(1-bias) * (m/2)
            mag = m * 0.5
        else:                           # normal: 2^(e-bias) * (1 + m/2)
            mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
        out[code] = sign * mag
    return out


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return e2m1_decode_table()[np.asarray(codes, dtype=np.int64) & 0xF]


def _rne_encode(a: np.ndarray, mags: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of ascending ``mags`` to ``a`` (>= 0), ties to the even
    index, saturating at the last entry. Indices equal codes for e2m1/e4m3 magnitudes."""
    a = np.asarray(a, dtype=np.float64)
    top = mags.size - 1
    lo = np.searchsorted(mags, a, side="right") - 1          # mags[lo] <= a
    lo = np.clip(lo, 0, top)
    hi = np.minimum(lo + 1, top)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= mags[top], top, code)               # saturate (satfinite)
    return code.astype(np.int64)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """fp32 values -> 4-bit codes (uint8), round to nearest even, saturate to +-6."""
    v = np.asarray(v, dtype=np.float32)
    mags = e2m1_decode_table()[:8]                           # 0, .5, 1, 1.5, 2, 3, 4, 6
    code = _rne_encode(np.abs(v), mags)
    sign = np.signbit(v).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


# ----------------------------------------------------------------------------------------
# e4m3 (fn)
# ----------------------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """Value of every byte 0..255 (fp64); NaN for 0x7F / 0xFF."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
            continue
        if e == 0:                      # subnormal: 2^(1-7) * m/8
            mag = m / 8.0 * 2.0 ** -6
        else:
            mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        out[code] = sign * mag
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return e4m3_decode_table()[np.asarray(codes, dtype=np.int64) & 0xFF]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp32 values -> e4m3 bytes, round to nearest even, saturate to +-448 (never NaN)."""
    v = np.asarray(v, dtype=np.float32)
    mags = e4m3_decode_table()[:0x7F]                        # 0 .. 448, codes 0x00..0x7E
    code = _rne_encode(np.abs(v), mags)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


# ----------------------------------------------------------------------------------------
# e8m0
# ----------------------------------------------------------------------------------------
def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, out)


# ----------------------------------------------------------------------------------------
# non-finite inputs
# ----------------------------------------------------------------------------------------
BF16_MAX_BITS = 0x7F7F   # largest finite bf16, 1.9921875 * 2^127


def bf16_nan_to_num(bits: np.ndarray) -> np.ndarray:
    """nan_to_num on bf16 bit patterns: NaN -> +0, +inf -> +largest finite, -inf -> -largest finite.

    The substitution the FastVideo pages (``convert_model_to_fp4``, ``convert_model_to_nvfp4``) and
    the SGLang page (``_quantize_weight_nvfp4``) apply before taking a weight's amax; the quantizers
    here encode the substituted values (reading U9), so a block is encoded from the same values
    its global scale was taken from.
    """
    b = np.asarray(bits, dtype=np.uint16)
    mag = b & np.uint16(0x7FFF)
    out = b.copy()
    out[mag > 0x7F80] = 0
    inf = mag == 0x7F80
    out[inf] = (b[inf] & np.uint16(0x8000)) | np.uint16(BF16_MAX_BITS)
    return out
