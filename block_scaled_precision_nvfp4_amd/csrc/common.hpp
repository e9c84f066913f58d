// Shared helpers of libbsp: error reporting, launch checks and the small scalar codecs the
// kernels use. gfx950 (CDNA4) only; compiled with -ffp-contract=off and IEEE fp32 division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdlib>
#include <cstring>
#include <cstdio>
#include <string>

#include "../../include/bsp.h"

namespace bsp {

// ---------------------------------------------------------------------------------------------
// host: errors
// ---------------------------------------------------------------------------------------------
std::string& last_error_slot();

inline int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error_slot() = buf;
  return status;
}

inline int ok() { return BSP_OK; }

// Verifies that the current device is gfx950 (cached per device).
int check_device();

inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BSP_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return BSP_OK;
}

#define BSP_REQUIRE(cond, status, ...) \
  do {                                 \
    if (!(cond)) return ::bsp::fail(status, __VA_ARGS__); \
  } while (0)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------------------------
// device: bf16 and the 8-bit / 4-bit scalar codecs
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even, with gfx950's v_cvt_pk_bf16_f32 (two values per instruction,
// NaN kept quiet). bf16x2_rne packs lo into bits 0-15 and hi into bits 16-31.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// e4m3 (fn) encode of a non-negative fp32: nearest even, saturating at 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode_pos(float s) {
  if (s >= 448.0f) return 0x7Eu;
  if (s < 0.015625f) return (uint32_t)__builtin_rintf(s * 512.0f);  // subnormals: m * 2^-9, m = 0..8
  uint32_t u = __float_as_uint(s);
  uint32_t c = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - 960u;    // (exp-120) << 3 | mantissa, RNE
  return c > 0x7Eu ? 0x7Eu : c;
}

// e4m3 decode of a non-negative code 0..0x7E (exact, branch-free). Placing the 7 code bits at
// the top of an fp32 exponent/mantissa field gives 2^(e-127) * (1 + m/8) for e >= 1 and the fp32
// denormal m * 2^-129 for e == 0; one exact multiply by 2^120 rebias both to the e4m3 values
// 2^(e-7) * (1 + m/8) and m * 2^-9. Needs fp32 denormals enabled (the HIP default, no
// flush-to-zero flags are used).
__device__ __forceinline__ float e4m3_decode_pos(uint32_t c) {
  return __uint_as_float(c << 20) * 1.329227995784916e36f;  // 2^120
}

// e4m3 encode with sign (nearest even, saturating at +-448, sign of zero kept).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  return ((__float_as_uint(v) >> 24) & 0x80u) | e4m3_encode_pos(__builtin_fabsf(v));
}

// e2m1 encode (nearest even, saturating at +-6, sign of zero kept); returns the 4-bit code.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t ua = u & 0x7FFFFFFFu;
  float a = __uint_as_float(ua);
  uint32_t code;
  if (a < 1.0f) {
    code = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u);          // 0, 0.5, 1.0 (ties even)
  } else {
    uint32_t c = ((ua + 0x1FFFFFu + ((ua >> 22) & 1u)) >> 22) - 252u;  // exponent/mantissa, RNE
    code = c > 7u ? 7u : c;
  }
  return code | ((u >> 28) & 8u);
}

// Max across the two lanes of each even/odd lane pair (DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ float pair_max(float x) {
  int y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false);
  return fmaxf(x, __int_as_float(y));
}

// Max across each quad of lanes (DPP quad_perm [1,0,3,2] then [2,3,0,1]).
__device__ __forceinline__ float quad_max(float x) {
  x = pair_max(x);
  int y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false);
  return fmaxf(x, __int_as_float(y));
}

}  // namespace bsp
