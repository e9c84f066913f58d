// Pieces shared by the GEMM kernels: vector types, the XCD-aware tile order and the epilogue.
#pragma once

#include "common.hpp"

namespace bsp {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kXcds = 8;     // MI355X: 8 XCDs, each with its own L2; workgroups go round-robin
constexpr int kGroupM = 4;   // M tiles per group in the grouped (L2-friendly) tile order

// Tile (tm, tn) of workgroup `bid`. The hardware hands workgroup ids to the XCDs round-robin, so
// XCD x runs ids x, x+8, x+16, ...; those are mapped to one contiguous range of the tile order,
// which is itself grouped: kGroupM tile-rows are swept together across all tile-columns, so the
// tiles an XCD runs at the same time share A row-blocks and B column-blocks in its L2.
// The map is a bijection on [0, ntm*ntn) whatever the dispatch order is.
__device__ __forceinline__ void tile_coords(int bid, int ntm, int ntn, int& tm, int& tn) {
  const int total = ntm * ntn;
  const int q = total / kXcds, r = total % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int t = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
  const int group = kGroupM * ntn;
  const int g = t / group;
  const int first = g * kGroupM;
  const int gm = ntm - first < kGroupM ? ntm - first : kGroupM;
  const int in = t - g * group;
  tm = first + in % gm;
  tn = in / gm;
}

// Bias of the linear layer, added in the epilogue:
//  kBiasNone;
//  kBiasBf16After: a bf16 [N] vector added to the bf16-rounded product, the sum rounded to bf16
//    again (the pages add the bias to mm_fp4's bf16 output); with fp32 output, product + bias;
//  kBiasF32Before: an fp32 [N] vector added to the fp32 product before its one rounding (the MXFP8
//    matmul that takes an fp32 bias).
enum { kBiasNone = 0, kBiasBf16After = 1, kBiasF32Before = 2 };

// Epilogue of a 128x128 wave tile made of 4x4 MFMA 32x32 tiles acc[n][m] holding D[n][m] (the
// MFMA's A operand is the B (weight) fragment): a lane holds output column gm = m0w + 32m + (lane%32)
// (a row of C) and, per group b, the four consecutive C columns n0w + 32n + 8b + 4*(lane/32) + 0..3.
// alpha[m] multiplies the lane's row of sub-tile m (the same value four times for a tensor alpha).
template <bool OUT_F32, int BIAS = kBiasNone>
__device__ __forceinline__ void store_wave_tile(const f32x16 (&acc)[4][4], const float (&alpha)[4],
                                                int64_t m0w, int64_t n0w, int64_t M, int64_t N,
                                                void* out, int64_t ldc, bool vec_store, int li, int h,
                                                const void* bias = nullptr) {
  constexpr int bias_kind = BIAS;
  // the lane's 64 bias values (they depend on the column only), zero past N
  float bq[4][4][4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t gn = n0w + n * 32 + 8 * b + 4 * h + i;
        float v = 0.0f;
        if (bias_kind == kBiasBf16After && gn < N)
          v = __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t*>(bias)[gn] << 16);
        else if (bias_kind == kBiasF32Before && gn < N)
          v = static_cast<const float*>(bias)[gn];
        bq[n][b][i] = v;
      }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t gm = m0w + m * 32 + li;
    if (gm >= M) continue;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t gn = n0w + n * 32 + 8 * b + 4 * h;
        float v0 = alpha[m] * acc[n][m][4 * b + 0];
        float v1 = alpha[m] * acc[n][m][4 * b + 1];
        float v2 = alpha[m] * acc[n][m][4 * b + 2];
        float v3 = alpha[m] * acc[n][m][4 * b + 3];
        if (bias_kind != kBiasNone && (OUT_F32 || bias_kind == kBiasF32Before)) {
          v0 += bq[n][b][0]; v1 += bq[n][b][1]; v2 += bq[n][b][2]; v3 += bq[n][b][3];
        }
        if (OUT_F32) {
          float* o = static_cast<float*>(out) + gm * ldc + gn;
          if (vec_store && gn + 3 < N) {
            *reinterpret_cast<float4*>(o) = make_float4(v0, v1, v2, v3);
          } else {
            if (gn + 0 < N) o[0] = v0;
            if (gn + 1 < N) o[1] = v1;
            if (gn + 2 < N) o[2] = v2;
            if (gn + 3 < N) o[3] = v3;
          }
        } else {
          uint16_t* o = static_cast<uint16_t*>(out) + gm * ldc + gn;
          uint32_t p01 = bf16x2_rne(v0, v1), p23 = bf16x2_rne(v2, v3);
          if (bias_kind == kBiasBf16After) {
            const float t0 = __builtin_bit_cast(float, p01 << 16) + bq[n][b][0];
            const float t1 = __builtin_bit_cast(float, p01 & 0xFFFF0000u) + bq[n][b][1];
            const float t2 = __builtin_bit_cast(float, p23 << 16) + bq[n][b][2];
            const float t3 = __builtin_bit_cast(float, p23 & 0xFFFF0000u) + bq[n][b][3];
            p01 = bf16x2_rne(t0, t1);
            p23 = bf16x2_rne(t2, t3);
          }
          if (vec_store && gn + 3 < N) {
            *reinterpret_cast<uint2*>(o) = make_uint2(p01, p23);
          } else {
            if (gn + 0 < N) o[0] = (uint16_t)p01;
            if (gn + 1 < N) o[1] = (uint16_t)(p01 >> 16);
            if (gn + 2 < N) o[2] = (uint16_t)p23;
            if (gn + 3 < N) o[3] = (uint16_t)(p23 >> 16);
          }
        }
      }
    }
  }
}

}  // namespace bsp
