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

// Epilogue of a 128x128 wave tile made of 4x4 MFMA 32x32 tiles acc[n][m] holding D[n][m] (the
// MFMA's A operand is the B (weight) fragment): a lane holds output column gm = m0w + 32m + (lane%32)
// (a row of C) and, per group b, the four consecutive C columns n0w + 32n + 8b + 4*(lane/32) + 0..3.
// alpha[m] multiplies the lane's row of sub-tile m (the same value four times for a tensor alpha).
template <bool OUT_F32>
__device__ __forceinline__ void store_wave_tile(const f32x16 (&acc)[4][4], const float (&alpha)[4],
                                                int64_t m0w,
                                                int64_t n0w, int64_t M, int64_t N, void* out,
                                                int64_t ldc, bool vec_store, int li, int h) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t gm = m0w + m * 32 + li;
    if (gm >= M) continue;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t gn = n0w + n * 32 + 8 * b + 4 * h;
        const float v0 = alpha[m] * acc[n][m][4 * b + 0];
        const float v1 = alpha[m] * acc[n][m][4 * b + 1];
        const float v2 = alpha[m] * acc[n][m][4 * b + 2];
        const float v3 = alpha[m] * acc[n][m][4 * b + 3];
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
          const uint32_t p01 = bf16x2_rne(v0, v1), p23 = bf16x2_rne(v2, v3);
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
