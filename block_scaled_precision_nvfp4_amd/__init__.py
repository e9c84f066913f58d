"""Thin Python binding of libbsp.so: NVFP4 W4A4 and MXFP8 W8A8 linear-layer kernels for MI355X.

Every function has the name of the C entry point it calls (include/bsp.h) and does argument
marshalling only: it checks dtypes/devices/shapes, allocates outputs with torch when the caller
does not pass them, and calls the library on torch's current HIP stream. All arithmetic runs in
the library's HIP kernels; there is no fallback. If libbsp.so is missing or fails to load, every
call raises ``BspLibraryError`` (build it with ``python -m block_scaled_precision_nvfp4_amd._build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsp.so")

BSP_OUT_BF16 = 0
BSP_OUT_F32 = 1

_STATUS = {0: "BSP_OK", -1: "BSP_EINVAL", -2: "BSP_ESHAPE", -3: "BSP_EDTYPE",
           -4: "BSP_EUNSUPPORTED", -5: "BSP_EHIP"}

# C signatures (argument ctypes), in include/bsp.h order
_i64, _p, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "bsp_last_error": ([], ctypes.c_char_p),
    "bsp_version": ([], _int),
    "bsp_nvfp4_sf_bytes": ([_i64, _i64, ctypes.POINTER(_i64)], _int),
    "bsp_nvfp4_global_sf": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], _int),
    "bsp_nvfp4_quantize": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], _int),
    "bsp_nvfp4_prequantize_weight": ([_p, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p], _int),
    "bsp_nvfp4_prequantize_weight_frag": ([_p, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p], _int),
    "bsp_nvfp4_alpha": ([_p, _p, _p, _p], _int),
    "bsp_mm_fp4": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_mxfp8_quantize": ([_p, _i64, _i64, _i64, _p, _p, _p], _int),
    "bsp_mm_mxfp8": ([_p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_mxfp4_sf_bytes": ([_i64, _i64, ctypes.POINTER(_i64)], _int),
    "bsp_mxfp4_quantize": ([_p, _i64, _i64, _i64, _p, _p, _p], _int),
    "bsp_mm_mxfp4": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_gelu_tanh_bf16": ([_p, _p, _i64, _p], _int),
    "bsp_nvfp4_quantize_gelu": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], _int),
    "bsp_nvfp4_quantize_per_token": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], _int),
    "bsp_nvfp4_sf_bytes_8x4": ([_i64, _i64, ctypes.POINTER(_i64)], _int),
    "bsp_nvfp4_quantize_8x4": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], _int),
    "bsp_mm_fp4_8x4": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_nvfp4_global_sf_4over6": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], _int),
    "bsp_mm_fp4_per_token": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_mm_fp4_bias": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_mm_fp4_gelu_nvfp4": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p], _int),
    "bsp_mm_mxfp8_bias": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_mm_mxfp4_bias": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_rmsnorm_bf16": ([_p, _i64, _i64, _i64, _p, ctypes.c_float, _p, _i64, _p], _int),
    "bsp_nvfp4_quantize_rmsnorm": ([_p, _i64, _i64, _i64, _p, ctypes.c_float, _p, _p, _p, _p], _int),
    "bsp_nvfp4_frag_bytes": ([_i64, _i64, ctypes.POINTER(_i64)], _int),
    "bsp_nvfp4_quantize_frag": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], _int),
    "bsp_nvfp4_quantize_gelu_frag": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], _int),
    "bsp_mm_fp4_frag": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_mxfp4_frag_bytes": ([_i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)], _int),
    "bsp_mxfp4_quantize_frag": ([_p, _i64, _i64, _i64, _p, _p, _p], _int),
    "bsp_mm_mxfp4_frag": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
    "bsp_mxfp8_frag_bytes": ([_i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)], _int),
    "bsp_mxfp8_quantize_frag": ([_p, _i64, _i64, _i64, _p, _p, _p], _int),
    "bsp_mm_mxfp8_frag": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _int, _p], _int),
}


class BspLibraryError(RuntimeError):
    """libbsp.so could not be loaded."""


class BspError(RuntimeError):
    """A libbsp call returned a non-OK status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises BspLibraryError if it is not built or cannot be loaded)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise BspLibraryError(f"{LIB_PATH} not found; build it with "
                                  "`python -m block_scaled_precision_nvfp4_amd._build`")
        try:
            h = ctypes.CDLL(LIB_PATH)
        except OSError as e:
            raise BspLibraryError(f"cannot load {LIB_PATH}: {e}") from e
        for name, (args, res) in SIGNATURES.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = res
        _lib = h
    return _lib


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise BspError(name, st, lib().bsp_last_error().decode(errors="replace"))


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, dev: Optional[torch.device] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _as_bf16_2d(x: torch.Tensor, name: str) -> torch.Tensor:
    """fp32 activations are cast to bf16 (the pages coerce fp32 to bf16 before the FP4 linear);
    non-float inputs are rejected; the last dim must be contiguous."""
    if not x.is_floating_point():
        raise TypeError(f"{name} must be floating point, got {x.dtype}")
    if x.dtype == torch.float32:
        x = x.to(torch.bfloat16)
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bf16 (or fp32, cast to bf16), got {x.dtype}")
    if x.dim() != 2:
        x = x.reshape(-1, x.shape[-1])
    if x.stride(-1) != 1:
        x = x.contiguous()
    return x


# ------------------------------------------------------------------------------------- queries
def bsp_version() -> int:
    return lib().bsp_version()


def bsp_nvfp4_sf_bytes(rows: int, k: int) -> int:
    out = ctypes.c_int64(0)
    _call("bsp_nvfp4_sf_bytes", rows, k, ctypes.byref(out))
    return out.value


# ------------------------------------------------------------------------------------- NVFP4
def bsp_nvfp4_global_sf(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(gsf, inv_gsf, amax): fp32 device scalars (shape [1]) for bf16 weight w [N, K]."""
    w = _as_bf16_2d(w, "w")
    _need(w, "w", torch.bfloat16)
    sc = torch.empty(3, dtype=torch.float32, device=w.device)
    gsf, inv, amax = sc[0:1], sc[1:2], sc[2:3]
    _call("bsp_nvfp4_global_sf", w.data_ptr(), w.shape[0], w.shape[1], w.stride(0),
          gsf.data_ptr(), inv.data_ptr(), amax.data_ptr(), _stream(w.device))
    return gsf, inv, amax


def bsp_nvfp4_quantize(x: torch.Tensor, gsf: torch.Tensor,
                       packed: Optional[torch.Tensor] = None,
                       sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(packed uint8 [M, K/2], sf uint8 [ceil(M/128)*128, ceil(K/64)*4] in the 128x4 layout)."""
    return _nvfp4_quantize("bsp_nvfp4_quantize", x, gsf, packed, sf)


def bsp_nvfp4_quantize_gelu(y: torch.Tensor, gsf: torch.Tensor,
                            packed: Optional[torch.Tensor] = None,
                            sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """NVFP4 quantize of bf16(gelu_tanh(y)) in one pass; outputs as bsp_nvfp4_quantize."""
    return _nvfp4_quantize("bsp_nvfp4_quantize_gelu", y, gsf, packed, sf)


def bsp_nvfp4_quantize_8x4(x: torch.Tensor, gsf: torch.Tensor,
                           packed: Optional[torch.Tensor] = None,
                           sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """NVFP4 quantize with layout_8x4 scales: sf uint8 [ceil(M/8)*8, ceil(K/64)*4]."""
    return _nvfp4_quantize("bsp_nvfp4_quantize_8x4", x, gsf, packed, sf, row_tile=8)


def _nvfp4_quantize(fn: str, x: torch.Tensor, gsf: torch.Tensor, packed: Optional[torch.Tensor],
                    sf: Optional[torch.Tensor], row_tile: int = 128) -> Tuple[torch.Tensor, torch.Tensor]:
    x = _as_bf16_2d(x, "x")
    _need(gsf, "gsf", torch.float32, x.device)
    m, k = x.shape
    rp = -(-m // row_tile) * row_tile
    kp = -(-(k // 16) // 4) * 4
    if packed is None:
        packed = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((rp, kp), dtype=torch.uint8, device=x.device)
    _need(packed, "packed", torch.uint8, x.device)
    _need(sf, "sf", torch.uint8, x.device)
    if packed.numel() < m * (k // 2) or not packed.is_contiguous():
        raise ValueError("packed must be contiguous with M*K/2 bytes")
    if sf.numel() < rp * kp or not sf.is_contiguous():
        raise ValueError("sf must be contiguous with rows padded to the scale tile x ceil(K/64)*4 bytes")
    _call(fn, x.data_ptr(), m, k, x.stride(0), gsf.data_ptr(),
          packed.data_ptr(), sf.data_ptr(), _stream(x.device))
    return packed, sf


def bsp_nvfp4_quantize_per_token(x: torch.Tensor, packed: Optional[torch.Tensor] = None,
                                 sf: Optional[torch.Tensor] = None,
                                 gsf_rows: Optional[torch.Tensor] = None):
    """NVFP4 quantize with one encode scale per row: (packed, sf, gsf_rows fp32 [M])."""
    x = _as_bf16_2d(x, "x")
    m, k = x.shape
    rp = -(-m // 128) * 128
    kp = -(-(k // 16) // 4) * 4
    if packed is None:
        packed = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((rp, kp), dtype=torch.uint8, device=x.device)
    if gsf_rows is None:
        gsf_rows = torch.empty((m,), dtype=torch.float32, device=x.device)
    _need(packed, "packed", torch.uint8, x.device)
    _need(sf, "sf", torch.uint8, x.device)
    _need(gsf_rows, "gsf_rows", torch.float32, x.device)
    if packed.numel() < m * (k // 2) or not packed.is_contiguous():
        raise ValueError("packed must be contiguous with M*K/2 bytes")
    if sf.numel() < rp * kp or not sf.is_contiguous():
        raise ValueError("sf must be contiguous with bsp_nvfp4_sf_bytes(M, K) bytes")
    if gsf_rows.numel() < m or not gsf_rows.is_contiguous():
        raise ValueError("gsf_rows must be a contiguous fp32 vector of M scales")
    _call("bsp_nvfp4_quantize_per_token", x.data_ptr(), m, k, x.stride(0), packed.data_ptr(),
          sf.data_ptr(), gsf_rows.data_ptr(), _stream(x.device))
    return packed, sf, gsf_rows


def bsp_nvfp4_prequantize_weight(w: torch.Tensor):
    """Load-time: (packed, sf, gsf, inv_gsf, amax) for bf16 weight w [N, K]."""
    w = _as_bf16_2d(w, "w")
    n, k = w.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    sf = torch.empty((-(-n // 128) * 128, -(-(k // 16) // 4) * 4), dtype=torch.uint8, device=w.device)
    sc = torch.empty(3, dtype=torch.float32, device=w.device)
    gsf, inv, amax = sc[0:1], sc[1:2], sc[2:3]
    _call("bsp_nvfp4_prequantize_weight", w.data_ptr(), n, k, w.stride(0), packed.data_ptr(),
          sf.data_ptr(), gsf.data_ptr(), inv.data_ptr(), amax.data_ptr(), _stream(w.device))
    return packed, sf, gsf, inv, amax


def bsp_nvfp4_alpha(x_gsf: torch.Tensor, w_gsf: torch.Tensor) -> torch.Tensor:
    _need(x_gsf, "x_gsf", torch.float32)
    _need(w_gsf, "w_gsf", torch.float32, x_gsf.device)
    out = torch.empty(1, dtype=torch.float32, device=x_gsf.device)
    _call("bsp_nvfp4_alpha", x_gsf.data_ptr(), w_gsf.data_ptr(), out.data_ptr(), _stream(x_gsf.device))
    return out


def bsp_mm_fp4(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
               alpha: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C [M, N] = alpha * A . B^T. a: packed [M, K/2], b: packed weight [N, K/2] (K-major)."""
    m, n, k, code, out = _mm_fp4_args(a, a_sf, b, b_sf, out_dtype, out)
    _need(alpha, "alpha", torch.float32, a.device)
    _call("bsp_mm_fp4", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          alpha.data_ptr(), m, n, k, out.data_ptr(), out.stride(0), code, _stream(a.device))
    return out


def _bias_vector(bias: torch.Tensor, n: int, dtype: torch.dtype, dev) -> None:
    _need(bias, "bias", dtype, dev)
    if bias.dim() != 1 or bias.numel() != n or not bias.is_contiguous():
        raise ValueError(f"bias must be a contiguous vector of N = {n} elements")


def bsp_mm_fp4_bias(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                    alpha: torch.Tensor, bias: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsp_mm_fp4 with the bf16 bias [N] added to its output in the epilogue (the pages' out + bias)."""
    m, n, k, code, out = _mm_fp4_args(a, a_sf, b, b_sf, out_dtype, out)
    _need(alpha, "alpha", torch.float32, a.device)
    _bias_vector(bias, n, torch.bfloat16, a.device)
    _call("bsp_mm_fp4_bias", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          alpha.data_ptr(), bias.data_ptr(), m, n, k, out.data_ptr(), out.stride(0), code,
          _stream(a.device))
    return out


def bsp_mm_fp4_gelu_nvfp4(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                          alpha: torch.Tensor, out_gsf: torch.Tensor,
                          packed: Optional[torch.Tensor] = None,
                          sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """NVFP4 of gelu_tanh(alpha * A . B^T) with global scale out_gsf, straight from the GEMM: the
    same bytes as bsp_nvfp4_quantize_gelu(bsp_mm_fp4(...), out_gsf) without the bf16 product in
    memory. packed [M, N/2], sf [ceil(M/128)*128, N/16] (128x4); N must be a multiple of 128."""
    m, n, k = _mm_fp4_shapes(a, a_sf, b, b_sf)
    _need(alpha, "alpha", torch.float32, a.device)
    _need(out_gsf, "out_gsf", torch.float32, a.device)
    rp, kp = -(-m // 128) * 128, n // 16
    if packed is None:
        packed = torch.empty((m, n // 2), dtype=torch.uint8, device=a.device)
    if sf is None:
        sf = torch.empty((rp, kp), dtype=torch.uint8, device=a.device)
    _need(packed, "packed", torch.uint8, a.device)
    _need(sf, "sf", torch.uint8, a.device)
    if packed.numel() < m * (n // 2) or not packed.is_contiguous():
        raise ValueError("packed must be contiguous with M*N/2 bytes")
    if sf.numel() < rp * kp or not sf.is_contiguous():
        raise ValueError("sf must be contiguous with ceil(M/128)*128 x N/16 bytes")
    _call("bsp_mm_fp4_gelu_nvfp4", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          alpha.data_ptr(), out_gsf.data_ptr(), m, n, k, packed.data_ptr(), sf.data_ptr(),
          _stream(a.device))
    return packed, sf


def bsp_mm_fp4_per_token(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                         x_gsf_rows: torch.Tensor, w_gsf: torch.Tensor,
                         out_dtype: torch.dtype = torch.bfloat16,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C [M, N] = alpha_m * A . B^T with alpha_m = 1/(x_gsf_rows[m] * w_gsf) (per-token scales)."""
    m, n, k, code, out = _mm_fp4_args(a, a_sf, b, b_sf, out_dtype, out)
    _need(x_gsf_rows, "x_gsf_rows", torch.float32, a.device)
    _need(w_gsf, "w_gsf", torch.float32, a.device)
    if x_gsf_rows.numel() < m or not x_gsf_rows.is_contiguous():
        raise ValueError("x_gsf_rows must be a contiguous fp32 vector of M scales")
    _call("bsp_mm_fp4_per_token", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          x_gsf_rows.data_ptr(), w_gsf.data_ptr(), m, n, k, out.data_ptr(), out.stride(0), code,
          _stream(a.device))
    return out


def bsp_mm_fp4_8x4(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                   alpha: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsp_mm_fp4 with A's scales in layout_8x4 (from bsp_nvfp4_quantize_8x4)."""
    m, n, k, code, out = _mm_fp4_args(a, a_sf, b, b_sf, out_dtype, out, a_row_tile=8)
    _need(alpha, "alpha", torch.float32, a.device)
    _call("bsp_mm_fp4_8x4", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          alpha.data_ptr(), m, n, k, out.data_ptr(), out.stride(0), code, _stream(a.device))
    return out


def bsp_nvfp4_global_sf_4over6(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(gsf, inv_gsf, amax) of the 4over6 variant (block scales capped at 256), device fp32."""
    w = _as_bf16_2d(w, "w")
    gsf, inv, amax = (torch.empty(1, dtype=torch.float32, device=w.device) for _ in range(3))
    _call("bsp_nvfp4_global_sf_4over6", w.data_ptr(), w.shape[0], w.shape[1], w.stride(0),
          gsf.data_ptr(), inv.data_ptr(), amax.data_ptr(), _stream(w.device))
    return gsf, inv, amax


def _mm_fp4_shapes(a, a_sf, b, b_sf, a_row_tile: int = 128):
    """(M, N, K) of an NVFP4 GEMM after checking the operands and their scale buffers."""
    _need(a, "a", torch.uint8)
    dev = a.device
    for t, nm in ((a_sf, "a_sf"), (b, "b"), (b_sf, "b_sf")):
        _need(t, nm, torch.uint8, dev)
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"a {tuple(a.shape)} and b {tuple(b.shape)} must be [M, K/2] and [N, K/2]")
    if not (a.is_contiguous() and b.is_contiguous() and a_sf.is_contiguous() and b_sf.is_contiguous()):
        raise ValueError("operands and scales must be contiguous")
    m, n, k = a.shape[0], b.shape[0], a.shape[1] * 2
    a_need = bsp_nvfp4_sf_bytes(m, k) if a_row_tile == 128 else bsp_nvfp4_sf_bytes_8x4(m, k)
    if a_sf.numel() < a_need or b_sf.numel() < bsp_nvfp4_sf_bytes(n, k):
        raise ValueError("scale buffers are smaller than the layout needs")
    return m, n, k


def _mm_fp4_args(a, a_sf, b, b_sf, out_dtype, out, a_row_tile: int = 128):
    m, n, k = _mm_fp4_shapes(a, a_sf, b, b_sf, a_row_tile)
    dev = a.device
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out_dtype must be bf16 or fp32, got {out_dtype}")
    code = BSP_OUT_BF16 if out_dtype == torch.bfloat16 else BSP_OUT_F32
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, dev)
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError(f"out must be [{m}, {n}] with unit column stride")
    return m, n, k, code, out


# ------------------------------------------------------------------------------------- MXFP8
def bsp_mxfp8_quantize(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                       sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(q uint8 e4m3 [M, K], sf uint8 e8m0 [M, K/32])."""
    x = _as_bf16_2d(x, "x")
    m, k = x.shape
    if q is None:
        q = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((m, k // 32), dtype=torch.uint8, device=x.device)
    _need(q, "q", torch.uint8, x.device)
    _need(sf, "sf", torch.uint8, x.device)
    if tuple(q.shape) != (m, k) or tuple(sf.shape) != (m, k // 32) or not (q.is_contiguous() and sf.is_contiguous()):
        raise ValueError("q must be contiguous [M, K] and sf contiguous [M, K/32]")
    _call("bsp_mxfp8_quantize", x.data_ptr(), m, k, x.stride(0), q.data_ptr(), sf.data_ptr(),
          _stream(x.device))
    return q, sf


def _mm_mxfp8_args(a, a_sf, b, b_sf, out_dtype, out):
    _need(a, "a", torch.uint8)
    dev = a.device
    for t, nm in ((a_sf, "a_sf"), (b, "b"), (b_sf, "b_sf")):
        _need(t, nm, torch.uint8, dev)
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"a {tuple(a.shape)} and b {tuple(b.shape)} must be [M, K] and [N, K]")
    m, n, k = a.shape[0], b.shape[0], a.shape[1]
    if tuple(a_sf.shape) != (m, k // 32) or tuple(b_sf.shape) != (n, k // 32):
        raise ValueError("scales must be [rows, K/32]")
    if not (a.is_contiguous() and b.is_contiguous() and a_sf.is_contiguous() and b_sf.is_contiguous()):
        raise ValueError("operands and scales must be contiguous")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out_dtype must be bf16 or fp32, got {out_dtype}")
    code = BSP_OUT_BF16 if out_dtype == torch.bfloat16 else BSP_OUT_F32
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, dev)
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError(f"out must be [{m}, {n}] with unit column stride")
    return m, n, k, code, out


def bsp_mm_mxfp8(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                 out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C [M, N] = A . B^T for MXFP8 a [M, K] / a_sf [M, K/32] and b [N, K] / b_sf [N, K/32]."""
    m, n, k, code, out = _mm_mxfp8_args(a, a_sf, b, b_sf, out_dtype, out)
    _call("bsp_mm_mxfp8", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(), m, n, k,
          out.data_ptr(), out.stride(0), code, _stream(a.device))
    return out


def bsp_mm_mxfp8_bias(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                      bias: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsp_mm_mxfp8 with the fp32 bias [N] added to the fp32 product before its rounding."""
    m, n, k, code, out = _mm_mxfp8_args(a, a_sf, b, b_sf, out_dtype, out)
    _bias_vector(bias, n, torch.float32, a.device)
    _call("bsp_mm_mxfp8_bias", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          bias.data_ptr(), m, n, k, out.data_ptr(), out.stride(0), code, _stream(a.device))
    return out


# ------------------------------------------------------------------------------------- MXFP4
def bsp_nvfp4_sf_bytes_8x4(rows: int, k: int) -> int:
    out = ctypes.c_int64(0)
    _call("bsp_nvfp4_sf_bytes_8x4", rows, k, ctypes.byref(out))
    return out.value


def bsp_mxfp4_sf_bytes(rows: int, k: int) -> int:
    out = ctypes.c_int64(0)
    _call("bsp_mxfp4_sf_bytes", rows, k, ctypes.byref(out))
    return out.value


def bsp_mxfp4_quantize(x: torch.Tensor, packed: Optional[torch.Tensor] = None,
                       sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(packed uint8 [M, K/2], sf uint8 [ceil(M/128)*128, ceil(K/128)*4] in the 128x4 layout)."""
    x = _as_bf16_2d(x, "x")
    m, k = x.shape
    rp, kp = -(-m // 128) * 128, -(-k // 128) * 4
    if packed is None:
        packed = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((rp, kp), dtype=torch.uint8, device=x.device)
    _need(packed, "packed", torch.uint8, x.device)
    _need(sf, "sf", torch.uint8, x.device)
    if packed.numel() < m * (k // 2) or not packed.is_contiguous():
        raise ValueError("packed must be contiguous with M*K/2 bytes")
    if sf.numel() < rp * kp or not sf.is_contiguous():
        raise ValueError("sf must be contiguous with bsp_mxfp4_sf_bytes(M, K) bytes")
    _call("bsp_mxfp4_quantize", x.data_ptr(), m, k, x.stride(0), packed.data_ptr(), sf.data_ptr(),
          _stream(x.device))
    return packed, sf


def _mm_mxfp4_args(a, a_sf, b, b_sf, alpha, out_dtype, out):
    _need(a, "a", torch.uint8)
    dev = a.device
    for t, nm in ((a_sf, "a_sf"), (b, "b"), (b_sf, "b_sf")):
        _need(t, nm, torch.uint8, dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, dev)
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"a {tuple(a.shape)} and b {tuple(b.shape)} must be [M, K/2] and [N, K/2]")
    if not (a.is_contiguous() and b.is_contiguous() and a_sf.is_contiguous() and b_sf.is_contiguous()):
        raise ValueError("operands and scales must be contiguous")
    m, n, k = a.shape[0], b.shape[0], a.shape[1] * 2
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out_dtype must be bf16 or fp32, got {out_dtype}")
    code = BSP_OUT_BF16 if out_dtype == torch.bfloat16 else BSP_OUT_F32
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, dev)
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError(f"out must be [{m}, {n}] with unit column stride")
    if a_sf.numel() < bsp_mxfp4_sf_bytes(m, k) or b_sf.numel() < bsp_mxfp4_sf_bytes(n, k):
        raise ValueError("scale buffers are smaller than bsp_mxfp4_sf_bytes")
    return m, n, k, code, out


def bsp_mm_mxfp4(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                 alpha: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C [M, N] = alpha * A . B^T for MXFP4 a [M, K/2] and weight b [N, K/2] (128x4 scales)."""
    m, n, k, code, out = _mm_mxfp4_args(a, a_sf, b, b_sf, alpha, out_dtype, out)
    _call("bsp_mm_mxfp4", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          _ptr(alpha), m, n, k, out.data_ptr(), out.stride(0), code, _stream(a.device))
    return out


def bsp_mm_mxfp4_bias(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                      bias: torch.Tensor, alpha: Optional[torch.Tensor] = None,
                      out_dtype: torch.dtype = torch.bfloat16,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsp_mm_mxfp4 with the bf16 bias [N] added to its output (as bsp_mm_fp4_bias)."""
    m, n, k, code, out = _mm_mxfp4_args(a, a_sf, b, b_sf, alpha, out_dtype, out)
    _bias_vector(bias, n, torch.bfloat16, a.device)
    _call("bsp_mm_mxfp4_bias", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          _ptr(alpha), bias.data_ptr(), m, n, k, out.data_ptr(), out.stride(0), code,
          _stream(a.device))
    return out


# ---------------------------------------------------------------- NVFP4, MFMA fragment layout
def bsp_nvfp4_frag_bytes(rows: int, k: int) -> int:
    """Packed bytes of a [rows, K] operand with its values in the fragment layout (K % 64 == 0)."""
    pb = ctypes.c_int64(0)
    _call("bsp_nvfp4_frag_bytes", rows, k, ctypes.byref(pb))
    return pb.value


def bsp_nvfp4_quantize_frag(x: torch.Tensor, gsf: torch.Tensor,
                            packed: Optional[torch.Tensor] = None,
                            sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """NVFP4 of x [M, K] with the packed values in the fragment layout: (packed uint8
    [ceil(M/32), K/64, 1024] -- one 1 KB fragment per 32-row tile and 64-K step --, sf in the 128x4
    layout as bsp_nvfp4_quantize's)."""
    return _nvfp4_quantize_frag("bsp_nvfp4_quantize_frag", x, gsf, packed, sf)


def bsp_nvfp4_quantize_gelu_frag(y: torch.Tensor, gsf: torch.Tensor,
                                 packed: Optional[torch.Tensor] = None,
                                 sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bsp_nvfp4_quantize_gelu with the packed values in the fragment layout."""
    return _nvfp4_quantize_frag("bsp_nvfp4_quantize_gelu_frag", y, gsf, packed, sf)


def _nvfp4_quantize_frag(fn, x, gsf, packed, sf):
    x = _as_bf16_2d(x, "x")
    _need(gsf, "gsf", torch.float32, x.device)
    m, k = x.shape
    pb = bsp_nvfp4_frag_bytes(m, k)
    if packed is None:
        packed = torch.empty((-(-m // 32), k // 64, 1024), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((-(-m // 128) * 128, -(-(k // 16) // 4) * 4), dtype=torch.uint8, device=x.device)
    _need(packed, "packed", torch.uint8, x.device)
    _need(sf, "sf", torch.uint8, x.device)
    if packed.numel() < pb or not packed.is_contiguous():
        raise ValueError("packed must be contiguous with bsp_nvfp4_frag_bytes(M, K) bytes")
    if sf.numel() < bsp_nvfp4_sf_bytes(m, k) or not sf.is_contiguous():
        raise ValueError("sf must be contiguous with bsp_nvfp4_sf_bytes(M, K) bytes")
    _call(fn, x.data_ptr(), m, k, x.stride(0), gsf.data_ptr(), packed.data_ptr(), sf.data_ptr(),
          _stream(x.device))
    return packed, sf


def bsp_nvfp4_prequantize_weight_frag(w: torch.Tensor):
    """Load-time, fragment layout: (packed [ceil(N/32), K/64, 1024], sf (128x4), gsf, inv_gsf, amax)
    for bf16 weight w [N, K], K % 64 == 0."""
    w = _as_bf16_2d(w, "w")
    n, k = w.shape
    packed = torch.empty((-(-n // 32), k // 64, 1024), dtype=torch.uint8, device=w.device)
    sf = torch.empty((-(-n // 128) * 128, -(-(k // 16) // 4) * 4), dtype=torch.uint8, device=w.device)
    sc = torch.empty(3, dtype=torch.float32, device=w.device)
    gsf, inv, amax = sc[0:1], sc[1:2], sc[2:3]
    _call("bsp_nvfp4_prequantize_weight_frag", w.data_ptr(), n, k, w.stride(0), packed.data_ptr(),
          sf.data_ptr(), gsf.data_ptr(), inv.data_ptr(), amax.data_ptr(), _stream(w.device))
    return packed, sf, gsf, inv, amax


def bsp_mm_fp4_frag(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                    m: int, n: int, alpha: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.bfloat16,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C [m, n] = alpha * A . B^T (+ bias) for operands A [m, K] and B [n, K] whose packed values are
    in the fragment layout (as written by bsp_nvfp4_quantize_frag), scales in 128x4."""
    _need(a, "a", torch.uint8)
    dev = a.device
    for t, nm in ((a_sf, "a_sf"), (b, "b"), (b_sf, "b_sf")):
        _need(t, nm, torch.uint8, dev)
    _need(alpha, "alpha", torch.float32, dev)
    if a.dim() != 3 or b.dim() != 3 or a.shape[1:] != b.shape[1:] or a.shape[2] != 1024:
        raise ValueError(f"a {tuple(a.shape)} and b {tuple(b.shape)} must be fragment tensors "
                         "[ceil(rows/32), K/64, 1024] with the same K")
    k = a.shape[1] * 64
    if not (-(-m // 32) == a.shape[0] and -(-n // 32) == b.shape[0]):
        raise ValueError(f"m={m}, n={n} do not match the fragment tensors' row tiles "
                         f"({a.shape[0]}, {b.shape[0]})")
    if not all(t.is_contiguous() for t in (a, a_sf, b, b_sf)):
        raise ValueError("operands and scales must be contiguous")
    if a_sf.numel() < bsp_nvfp4_sf_bytes(m, k) or b_sf.numel() < bsp_nvfp4_sf_bytes(n, k):
        raise ValueError("scale buffers are smaller than bsp_nvfp4_sf_bytes")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out_dtype must be bf16 or fp32, got {out_dtype}")
    code = BSP_OUT_BF16 if out_dtype == torch.bfloat16 else BSP_OUT_F32
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, dev)
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError(f"out must be [{m}, {n}] with unit column stride")
    if bias is not None:
        _bias_vector(bias, n, torch.bfloat16, dev)
    _call("bsp_mm_fp4_frag", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          alpha.data_ptr(), _ptr(bias), m, n, k, out.data_ptr(), out.stride(0), code, _stream(dev))
    return out


# ----------------------------------------------------------------- MXFP4, MFMA fragment layout
def bsp_mxfp4_frag_bytes(rows: int, k: int) -> Tuple[int, int]:
    """(packed bytes, scale bytes) of a [rows, K] operand in the fragment layout (K % 256 == 0)."""
    pb, sb = ctypes.c_int64(0), ctypes.c_int64(0)
    _call("bsp_mxfp4_frag_bytes", rows, k, ctypes.byref(pb), ctypes.byref(sb))
    return pb.value, sb.value


def _frag_shapes(rows: int, k: int):
    rt = -(-rows // 32)
    return (rt, k // 64, 1024), (rt, k // 256, 256)


def bsp_mxfp4_quantize_frag(x: torch.Tensor, packed: Optional[torch.Tensor] = None,
                            sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MXFP4 of x [M, K] in the fragment layout: (packed uint8 [ceil(M/32), K/64, 1024] -- one 1 KB
    MFMA fragment per 32-row tile and 64-K step --, sf uint8 [ceil(M/32), K/256, 256])."""
    x = _as_bf16_2d(x, "x")
    m, k = x.shape
    pshape, sshape = _frag_shapes(m, k)
    pb, sb = bsp_mxfp4_frag_bytes(m, k)
    if packed is None:
        packed = torch.empty(pshape, dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    _need(packed, "packed", torch.uint8, x.device)
    _need(sf, "sf", torch.uint8, x.device)
    if packed.numel() < pb or not packed.is_contiguous():
        raise ValueError("packed must be contiguous with bsp_mxfp4_frag_bytes(M, K)[0] bytes")
    if sf.numel() < sb or not sf.is_contiguous():
        raise ValueError("sf must be contiguous with bsp_mxfp4_frag_bytes(M, K)[1] bytes")
    _call("bsp_mxfp4_quantize_frag", x.data_ptr(), m, k, x.stride(0), packed.data_ptr(),
          sf.data_ptr(), _stream(x.device))
    return packed, sf


def bsp_mm_mxfp4_frag(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                      m: int, n: int, alpha: Optional[torch.Tensor] = None,
                      bias: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C [m, n] = alpha * A . B^T (+ bias) for fragment-layout operands A [m, K] and B [n, K] (as
    written by bsp_mxfp4_quantize_frag); bit-identical to bsp_mm_mxfp4 on the same values."""
    _need(a, "a", torch.uint8)
    dev = a.device
    for t, nm in ((a_sf, "a_sf"), (b, "b"), (b_sf, "b_sf")):
        _need(t, nm, torch.uint8, dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, dev)
    if a.dim() != 3 or b.dim() != 3 or a.shape[1:] != b.shape[1:] or a.shape[2] != 1024:
        raise ValueError(f"a {tuple(a.shape)} and b {tuple(b.shape)} must be fragment tensors "
                         "[ceil(rows/32), K/64, 1024] with the same K")
    k = a.shape[1] * 64
    if not (-(-m // 32) == a.shape[0] and -(-n // 32) == b.shape[0]):
        raise ValueError(f"m={m}, n={n} do not match the fragment tensors' row tiles "
                         f"({a.shape[0]}, {b.shape[0]})")
    if not all(t.is_contiguous() for t in (a, a_sf, b, b_sf)):
        raise ValueError("operands and scales must be contiguous")
    if a_sf.numel() < bsp_mxfp4_frag_bytes(m, k)[1] or b_sf.numel() < bsp_mxfp4_frag_bytes(n, k)[1]:
        raise ValueError("scale buffers are smaller than bsp_mxfp4_frag_bytes")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out_dtype must be bf16 or fp32, got {out_dtype}")
    code = BSP_OUT_BF16 if out_dtype == torch.bfloat16 else BSP_OUT_F32
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, dev)
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError(f"out must be [{m}, {n}] with unit column stride")
    if bias is not None:
        _bias_vector(bias, n, torch.bfloat16, dev)
    _call("bsp_mm_mxfp4_frag", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          _ptr(alpha), _ptr(bias), m, n, k, out.data_ptr(), out.stride(0), code, _stream(dev))
    return out


# ----------------------------------------------------------------- MXFP8, MFMA fragment layout
def bsp_mxfp8_frag_bytes(rows: int, k: int) -> Tuple[int, int]:
    """(element bytes, scale bytes) of a [rows, K] operand in the fragment layout (K % 256 == 0)."""
    qb, sb = ctypes.c_int64(0), ctypes.c_int64(0)
    _call("bsp_mxfp8_frag_bytes", rows, k, ctypes.byref(qb), ctypes.byref(sb))
    return qb.value, sb.value


def bsp_mxfp8_quantize_frag(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                            sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MXFP8 of x [M, K] in the fragment layout: (q uint8 [ceil(M/32), K/64, 2048] -- one 2 KB MFMA
    fragment per 32-row tile and 64-K step --, sf uint8 [ceil(M/32), K/256, 256])."""
    x = _as_bf16_2d(x, "x")
    m, k = x.shape
    qbytes, sbytes = bsp_mxfp8_frag_bytes(m, k)
    rt = -(-m // 32)
    if q is None:
        q = torch.empty((rt, k // 64, 2048), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((rt, k // 256, 256), dtype=torch.uint8, device=x.device)
    _need(q, "q", torch.uint8, x.device)
    _need(sf, "sf", torch.uint8, x.device)
    if q.numel() < qbytes or not q.is_contiguous():
        raise ValueError("q must be contiguous with bsp_mxfp8_frag_bytes(M, K)[0] bytes")
    if sf.numel() < sbytes or not sf.is_contiguous():
        raise ValueError("sf must be contiguous with bsp_mxfp8_frag_bytes(M, K)[1] bytes")
    _call("bsp_mxfp8_quantize_frag", x.data_ptr(), m, k, x.stride(0), q.data_ptr(), sf.data_ptr(),
          _stream(x.device))
    return q, sf


def bsp_mm_mxfp8_frag(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                      m: int, n: int, bias: Optional[torch.Tensor] = None,
                      out_dtype: torch.dtype = torch.bfloat16,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C [m, n] = A . B^T (+ fp32 bias) for fragment-layout operands A [m, K] and B [n, K] (as
    written by bsp_mxfp8_quantize_frag); bit-identical to bsp_mm_mxfp8 on the same values."""
    _need(a, "a", torch.uint8)
    dev = a.device
    for t, nm in ((a_sf, "a_sf"), (b, "b"), (b_sf, "b_sf")):
        _need(t, nm, torch.uint8, dev)
    if a.dim() != 3 or b.dim() != 3 or a.shape[1:] != b.shape[1:] or a.shape[2] != 2048:
        raise ValueError(f"a {tuple(a.shape)} and b {tuple(b.shape)} must be fragment tensors "
                         "[ceil(rows/32), K/64, 2048] with the same K")
    k = a.shape[1] * 64
    if not (-(-m // 32) == a.shape[0] and -(-n // 32) == b.shape[0]):
        raise ValueError(f"m={m}, n={n} do not match the fragment tensors' row tiles "
                         f"({a.shape[0]}, {b.shape[0]})")
    if not all(t.is_contiguous() for t in (a, a_sf, b, b_sf)):
        raise ValueError("operands and scales must be contiguous")
    if a_sf.numel() < bsp_mxfp8_frag_bytes(m, k)[1] or b_sf.numel() < bsp_mxfp8_frag_bytes(n, k)[1]:
        raise ValueError("scale buffers are smaller than bsp_mxfp8_frag_bytes")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out_dtype must be bf16 or fp32, got {out_dtype}")
    code = BSP_OUT_BF16 if out_dtype == torch.bfloat16 else BSP_OUT_F32
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, dev)
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError(f"out must be [{m}, {n}] with unit column stride")
    if bias is not None:
        _bias_vector(bias, n, torch.float32, dev)
    _call("bsp_mm_mxfp8_frag", a.data_ptr(), a_sf.data_ptr(), b.data_ptr(), b_sf.data_ptr(),
          _ptr(bias), m, n, k, out.data_ptr(), out.stride(0), code, _stream(dev))
    return out


def bsp_gelu_tanh_bf16(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(x, "x", torch.bfloat16)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.bfloat16, x.device)
    _call("bsp_gelu_tanh_bf16", x.data_ptr(), out.data_ptr(), x.numel(), _stream(x.device))
    return out


def _rmsnorm_args(x: torch.Tensor, weight: Optional[torch.Tensor]):
    x = _as_bf16_2d(x, "x")
    if weight is not None:
        _need(weight, "weight", torch.bfloat16, x.device)
        if weight.numel() != x.shape[1] or not weight.is_contiguous():
            raise ValueError("weight must be a contiguous bf16 vector of K elements")
    return x


def bsp_rmsnorm_bf16(x: torch.Tensor, weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """RMSNorm of each row of x over K (optional bf16 gain), bf16 out [M, K]."""
    x = _rmsnorm_args(x, weight)
    m, k = x.shape
    if out is None:
        out = torch.empty((m, k), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, x.device)
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != k or out.stride(1) != 1:
        raise ValueError("out must be bf16 [M, K] with unit column stride")
    _call("bsp_rmsnorm_bf16", x.data_ptr(), m, k, x.stride(0), _ptr(weight), float(eps),
          out.data_ptr(), out.stride(0), _stream(x.device))
    return out


def bsp_nvfp4_quantize_rmsnorm(x: torch.Tensor, gsf: torch.Tensor,
                               weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                               packed: Optional[torch.Tensor] = None,
                               sf: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """NVFP4 quantize of bsp_rmsnorm_bf16(x, weight, eps) in one pass; outputs as bsp_nvfp4_quantize."""
    x = _rmsnorm_args(x, weight)
    _need(gsf, "gsf", torch.float32, x.device)
    m, k = x.shape
    mp, kp = -(-m // 128) * 128, -(-(k // 16) // 4) * 4
    if packed is None:
        packed = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((mp, kp), dtype=torch.uint8, device=x.device)
    _need(packed, "packed", torch.uint8, x.device)
    _need(sf, "sf", torch.uint8, x.device)
    if packed.numel() < m * (k // 2) or not packed.is_contiguous():
        raise ValueError("packed must be contiguous with M*K/2 bytes")
    if sf.numel() < mp * kp or not sf.is_contiguous():
        raise ValueError("sf must be contiguous with ceil(M/128)*128 x ceil(K/64)*4 bytes")
    _call("bsp_nvfp4_quantize_rmsnorm", x.data_ptr(), m, k, x.stride(0), _ptr(weight), float(eps),
          gsf.data_ptr(), packed.data_ptr(), sf.data_ptr(), _stream(x.device))
    return packed, sf


__all__ = [n for n in SIGNATURES if n not in ("bsp_last_error",)] + [
    "BspError", "BspLibraryError", "BSP_OUT_BF16", "BSP_OUT_F32", "lib"]
