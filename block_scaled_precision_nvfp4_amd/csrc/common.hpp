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
// Compute units of the current device (cached per device; 256 on MI355X); 0 if unknown.
int device_cu_count();

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
// The hardware hands a launch's workgroups to the 8 XCDs round-robin by linear id, and each XCD has
// its own L2. xcd_blocked maps linear id b of n to an order in which consecutive ids run on one
// XCD (a bijection on [0, n)), so that workgroups that write neighbouring bytes of one memory sector
// do so through the same L2, which merges them, instead of each XCD writing back a partial sector.
__device__ __forceinline__ int64_t xcd_blocked(int64_t b, int64_t n) {
  const int64_t per = n / 8, r = n % 8, xcd = b % 8, local = b / 8;
  return (xcd < r ? xcd * (per + 1) : r * (per + 1) + (xcd - r) * per) + local;
}

// A milder regrouping: within each complete block of 32 ids, ids 4x .. 4x + 3 (in the returned
// order) are the four the hardware gives XCD x, so runs of four consecutive ids share one L2 while
// the XCDs still work side by side (a bijection on [0, n); an incomplete last block is unchanged).
__device__ __forceinline__ int64_t xcd_quads(int64_t b, int64_t n) {
  const int64_t blk = b >> 5, w = b & 31;
  return (blk * 32 + 32 <= n) ? blk * 32 + (w & 7) * 4 + (w >> 3) : b;
}

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

// ---------------------------------------------------------------------------------------------
// device: NVFP4 encoding pieces shared by the quantize kernels and the GEMM epilogue that emits
// NVFP4
// ---------------------------------------------------------------------------------------------
constexpr float kSixth = 0.16666667163372040f;  // fl32(1/6) = 0x3E2AAAAB

// gelu(x) = 0.5 x (1 + tanh(z)), z = sqrt(2/pi) (x + 0.044715 x^3), in fp32, rounded once to bf16
// by the caller. 0.5 (1 + tanh z) is the logistic function of 2z, evaluated with t = 2^(-2|z| log2 e)
// <= 1 as x / (1 + t) for x >= 0 and x t / (1 + t) for x < 0 (z has the sign of x): no cancellation
// and no overflow. -2|z| log2 e = |x| (c0 + c2 x^2) with c0 = -2 log2(e) sqrt(2/pi) and
// c2 = 0.044715 c0, one fused multiply-add. t is always formed as 2^64 t = 2^(that + 64) (the
// exponent is at most 64, so no overflow) and negative outputs are scaled back by 2^-64 at the end,
// so tiny negative outputs keep their bits down to where bf16 underflows too. v_exp_f32 and
// v_rcp_f32 (about 1 ulp each) keep the whole function at a dozen instructions; the result is
// within a few fp32 ulps, far inside one bf16 ulp except next to a rounding boundary.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float c0 = -2.302208198144325f;    // -2 log2(e) sqrt(2/pi)
  const float c2 = -0.1029432395800235f;   // 0.044715 c0
  const float x2 = x * x;
  const float p64 = __builtin_fmaf(__builtin_fmaf(c2, x2, c0), __builtin_fabsf(x), 64.0f);
  const float ts = __builtin_amdgcn_exp2f(p64);                       // t * 2^64
  const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(ts, 5.421010862427522e-20f, 1.0f));  // 1/(1+t)
  const bool neg = x < 0.0f;                                  // branch-free: selects, no exec masks
  const float m = neg ? ts : 1.0f;
  const float sc = neg ? 5.421010862427522e-20f : 1.0f;       // 2^-64
  return ((x * m) * r) * sc;
}

// GELU of bf16 values by table. A bf16 input has 2^16 values, so gelu rounded to bf16 is a
// function of 16 bits. The table (gelu_table.inc, written by gen_gelu_table.py in exact arithmetic)
// holds the correctly rounded bf16 of gelu(x) for |x| in [2^-12, 2^6) -- 18 binades x 128 mantissas
// x 2 signs, 9 KB -- which holds nearly all activations of a linear layer; a workgroup copies it into
// LDS with a few 16-byte loads. Lookups replace a dozen VALU instructions and two quarter-rate
// transcendentals per value with about six instructions and an LDS read; values outside the table
// (zeros, tiny or huge magnitudes, inf, NaN) take gelu_tanh above, whose bf16 rounding is within
// one ulp of the correctly rounded value.
constexpr int kGeluTabE0 = 115;                    // bf16 exponent field of 2^-12
constexpr int kGeluTabHalf = 18 * 128;             // entries per sign
constexpr int kGeluTabSize = 2 * kGeluTabHalf;     // uint16 entries

#include "gelu_table.inc"

// tab: LDS, kGeluTabSize entries, 16-byte aligned; threads t = 0 .. nt-1 of the workgroup copy it
// (the caller synchronises before the first lookup)
__device__ __forceinline__ void gelu_table_load(uint16_t* tab, int t, int nt) {
  const uint4* src = reinterpret_cast<const uint4*>(kGeluTable);
  uint4* dst = reinterpret_cast<uint4*>(tab);
  for (int i = t; i < kGeluTabSize / 8; i += nt) dst[i] = src[i];
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------------
// device: the values a quantizer encodes. Non-finite inputs are encoded as nan_to_num gives them
// (NaN -> +0, +-inf -> +-largest finite bf16), the substitution the pages apply before a weight's
// amax, so a block's scale and its elements come from the same finite values.
// ---------------------------------------------------------------------------------------------
// Largest magnitude among 8 bf16 values, as bf16 bits: magnitude bit patterns of non-negative
// bf16 values order like the values, so this is an integer max (packed 16-bit maxes). At least
// 0x7F80 exactly when one of the values is an infinity or a NaN.
__device__ __forceinline__ uint32_t mag_bits8(const uint4& v) {
  const u16x2_t a = __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu);
  const u16x2_t b = __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu);
  const u16x2_t c = __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu);
  const u16x2_t d = __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu);
  const u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                              __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

__device__ __forceinline__ uint32_t bf16_nan_to_num(uint32_t h) {
  const uint32_t m = h & 0x7FFFu;
  return m > 0x7F80u ? 0u : (m == 0x7F80u ? (h & 0x8000u) | 0x7F7Fu : h);
}

__device__ __forceinline__ uint32_t bf16x2_nan_to_num(uint32_t w) {
  return bf16_nan_to_num(w & 0xFFFFu) | (bf16_nan_to_num(w >> 16) << 16);
}

__device__ __forceinline__ uint4 nan_to_num8(const uint4& v) {
  return make_uint4(bf16x2_nan_to_num(v.x), bf16x2_nan_to_num(v.y), bf16x2_nan_to_num(v.z),
                    bf16x2_nan_to_num(v.w));
}

// Replaces N segments of 8 bf16 values by their nan_to_num when any of them holds an infinity or a
// NaN: one running integer max over all segments and one branch, rarely taken, so that the loads
// before and the encoding after stay branch-free (the encoder takes each segment's magnitude bits
// again, which costs a few integer instructions and no registers held across the loop).
template <int N>
__device__ __forceinline__ void nan_to_num_segments(uint4 (&v)[N]) {
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) mx = max(mx, mag_bits8(v[i]));
  if (mx >= 0x7F80u) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = nan_to_num8(v[i]);
  }
}

// The fp32 value (exact) of magnitude bits from mag_bits8
__device__ __forceinline__ float mag_value(uint32_t mb) { return __uint_as_float(mb << 16); }

// gelu of the two bf16 values in w (bits 0-15 and 16-31) from the table; sets bits of miss when
// either lies outside it (its result is then meaningless)
__device__ __forceinline__ uint32_t gelu2_tab(uint32_t w, const uint16_t* tab, uint32_t& miss) {
  const u16x2_t mag = __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
  const u16x2_t d = mag - (u16x2_t){kGeluTabE0 << 7, kGeluTabE0 << 7};   // wraps below the table
  const u16x2_t c = __builtin_elementwise_min(d, (u16x2_t){kGeluTabHalf - 1, kGeluTabHalf - 1});
  const uint32_t c32 = __builtin_bit_cast(uint32_t, c);
  miss |= c32 ^ __builtin_bit_cast(uint32_t, d);
  const uint32_t idx = ((w >> 15) & 0x10001u) * kGeluTabHalf + c32;      // sign picks the half
  return (uint32_t)tab[idx & 0xFFFFu] | ((uint32_t)tab[idx >> 16] << 16);
}

// gelu of 8 bf16 values, rounded to bf16, by the arithmetic (for inputs outside the table)
__device__ __forceinline__ uint4 gelu8_bf16_arith(const uint4& v) {
  return make_uint4(bf16x2_rne(gelu_tanh(bf16_lo(v.x)), gelu_tanh(bf16_hi(v.x))),
                    bf16x2_rne(gelu_tanh(bf16_lo(v.y)), gelu_tanh(bf16_hi(v.y))),
                    bf16x2_rne(gelu_tanh(bf16_lo(v.z)), gelu_tanh(bf16_hi(v.z))),
                    bf16x2_rne(gelu_tanh(bf16_lo(v.w)), gelu_tanh(bf16_hi(v.w))));
}

// gelu (bf16 in, bf16 out) of NSEG segments of 8 values: all by table first, then one branch,
// rarely taken, that computes the segments holding a value outside the table arithmetically. Keeping the
// common path free of branches lets the LDS latencies of all segments overlap. FINITE: the
// recomputed segments also get nan_to_num (for an encoder's input: the table holds only finite
// values, and gelu of a finite bf16 is finite, so only inputs outside the table can give an
// infinity or a NaN).
template <int NSEG, bool FINITE = false>
__device__ __forceinline__ void gelu_segments_tab(const uint4 (&in)[NSEG], uint4 (&out)[NSEG],
                                                  const uint16_t* tab) {
  uint32_t missbits = 0;
#pragma unroll
  for (int i = 0; i < NSEG; ++i) {
    uint32_t m = 0;
    out[i].x = gelu2_tab(in[i].x, tab, m);
    out[i].y = gelu2_tab(in[i].y, tab, m);
    out[i].z = gelu2_tab(in[i].z, tab, m);
    out[i].w = gelu2_tab(in[i].w, tab, m);
    missbits |= (m != 0 ? 1u : 0u) << i;
  }
  if (missbits) {
#pragma unroll
    for (int i = 0; i < NSEG; ++i)
      if ((missbits >> i) & 1u)
        out[i] = FINITE ? nan_to_num8(gelu8_bf16_arith(in[i])) : gelu8_bf16_arith(in[i]);
  }
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}



}  // namespace bsp
