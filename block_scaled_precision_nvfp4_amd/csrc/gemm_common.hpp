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

// Raw buffer loads for operands read straight into registers: one resource (base, size) per row
// tile held in scalar registers, the K step's byte offset in a scalar register and the lane's
// offset in one vector register, instead of a 64-bit vector address per load. The resource's last
// word, 0x00020000, is the plain raw-buffer format of this GPU family (32-bit data format, no
// swizzle); the stride is 0, so the byte offsets are used as given.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const uint8_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t ld4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t ld2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

// Bias of the linear layer, added in the epilogue:
//  kBiasNone;
//  kBiasBf16After: a bf16 [N] vector added to the bf16-rounded product, the sum rounded to bf16
//    again (the pages add the bias to mm_fp4's bf16 output); with fp32 output, product + bias;
//  kBiasF32Before: an fp32 [N] vector added to the fp32 product before its one rounding (the MXFP8
//    matmul that takes an fp32 bias).
// kGeluNvfp4 is no bias but a different output: NVFP4 of gelu(C) (store_tile_gelu_nvfp4 below).
enum { kBiasNone = 0, kBiasBf16After = 1, kBiasF32Before = 2, kGeluNvfp4 = 3 };

// Epilogue of a 128x128 wave tile made of 4x4 MFMA 32x32 tiles acc[n][m] holding D[n][m] (the
// MFMA's A operand is the B (weight) fragment): a lane holds output column gm = m0w + 32m + (lane%32)
// (a row of C) and, per group b, the four consecutive C columns n0w + 32n + 8b + 4*(lane/32) + 0..3.
// alpha[m] multiplies the lane's row of sub-tile m (the same value four times for a tensor alpha).

// The lane's 64 bias values (they depend on the column only), zero past N.
template <int BIAS>
__device__ __forceinline__ void load_bias(float (&bq)[4][4][4], int64_t n0w, int64_t N, int h,
                                          const void* bias) {
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t gn = n0w + n * 32 + 8 * b + 4 * h + i;
        float v = 0.0f;
        if (BIAS == kBiasBf16After && gn < N)
          v = __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t*>(bias)[gn] << 16);
        else if (BIAS == kBiasF32Before && gn < N)
          v = static_cast<const float*>(bias)[gn];
        bq[n][b][i] = v;
      }
}

// ACC16: the accumulators hold 2^-16 times the products (mm_fp4's f16 operands each carry 2^-8).
// The 2^16 goes onto the accumulator, alpha * (acc * 2^16): acc * 2^16 is exact and far below
// fp32's range (|acc| <= 2^31 for K <= 2^24), so the one rounding is that of the exact
// alpha * sum, for every finite alpha (2^16 folded into alpha instead would overflow above 2^112).
template <bool ACC16>
__device__ __forceinline__ float acc_value(float a) {
  return ACC16 ? a * 65536.0f : a;
}

// The four fp32 results of piece (m, n, b), bias of kind kBiasF32Before (or any kind for fp32
// output) included.
template <bool OUT_F32, int BIAS, bool ACC16>
__device__ __forceinline__ void piece_f32(const f32x16 (&acc)[4][4], const float (&alpha)[4],
                                          const float (&bq)[4][4][4], int m, int n, int b,
                                          float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = alpha[m] * acc_value<ACC16>(acc[n][m][4 * b + i]);
    if (BIAS != kBiasNone && (OUT_F32 || BIAS == kBiasF32Before)) v[i] += bq[n][b][i];
  }
}

// The four bf16 results of piece (m, n, b) as two packed pairs (nearest even; a kBiasBf16After
// bias is added to the rounded product and the sum rounded again).
template <int BIAS, bool ACC16>
__device__ __forceinline__ void piece_bf16(const f32x16 (&acc)[4][4], const float (&alpha)[4],
                                           const float (&bq)[4][4][4], int m, int n, int b,
                                           uint32_t& p01, uint32_t& p23) {
  float v[4];
  piece_f32<false, BIAS, ACC16>(acc, alpha, bq, m, n, b, v);
  p01 = bf16x2_rne(v[0], v[1]);
  p23 = bf16x2_rne(v[2], v[3]);
  if (BIAS == kBiasBf16After) {
    const float t0 = __builtin_bit_cast(float, p01 << 16) + bq[n][b][0];
    const float t1 = __builtin_bit_cast(float, p01 & 0xFFFF0000u) + bq[n][b][1];
    const float t2 = __builtin_bit_cast(float, p23 << 16) + bq[n][b][2];
    const float t3 = __builtin_bit_cast(float, p23 & 0xFFFF0000u) + bq[n][b][3];
    p01 = bf16x2_rne(t0, t1);
    p23 = bf16x2_rne(t2, t3);
  }
}

// Direct epilogue: each lane stores its 8-byte (bf16) or 16-byte (fp32) pieces, with bounds checks.
template <bool OUT_F32, int BIAS, bool ACC16>
__device__ __forceinline__ void store_wave_tile(const f32x16 (&acc)[4][4], const float (&alpha)[4],
                                                int64_t m0w, int64_t n0w, int64_t M, int64_t N,
                                                void* out, int64_t ldc, bool vec_store, int li, int h,
                                                const void* bias = nullptr) {
  float bq[4][4][4];
  load_bias<BIAS>(bq, n0w, N, h, bias);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t gm = m0w + m * 32 + li;
    if (gm >= M) continue;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t gn = n0w + n * 32 + 8 * b + 4 * h;
        if (OUT_F32) {
          float v[4];
          piece_f32<true, BIAS, ACC16>(acc, alpha, bq, m, n, b, v);
          float* o = static_cast<float*>(out) + gm * ldc + gn;
          if (vec_store && gn + 3 < N) {
            *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            if (gn + 0 < N) o[0] = v[0];
            if (gn + 1 < N) o[1] = v[1];
            if (gn + 2 < N) o[2] = v[2];
            if (gn + 3 < N) o[3] = v[3];
          }
        } else {
          uint32_t p01, p23;
          piece_bf16<BIAS, ACC16>(acc, alpha, bq, m, n, b, p01, p23);
          uint16_t* o = static_cast<uint16_t*>(out) + gm * ldc + gn;
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

// Staged epilogue for a bf16 wave tile that lies wholly inside C (rows 16-byte aligned): the
// 8-byte pieces go to a row-major image of 64 rows at a time in this wave's LDS area
// (kEpiWaveBytes), and come back as 16-byte row segments, so each store instruction writes four
// whole 256-byte rows instead of 32 rows x 16 bytes; the rows are not read again by this
// computation, so the stores are nontemporal. Image rows are 272 bytes apart: 16-byte aligned
// reads, and a 64-bit write of lanes li and li + 16 shares banks at most pairwise.
constexpr int kEpiRowBytes = 272;
constexpr int kEpiWaveBytes = 64 * kEpiRowBytes;

template <int BIAS, bool ACC16>
__device__ __forceinline__ void store_wave_tile_staged(const f32x16 (&acc)[4][4],
                                                       const float (&alpha)[4], int64_t m0w,
                                                       int64_t n0w, int64_t N, void* out,
                                                       int64_t ldc, uint8_t* lds, int lane, int li,
                                                       int h, const void* bias = nullptr) {
  float bq[4][4][4];
  load_bias<BIAS>(bq, n0w, N, h, bias);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          uint32_t p01, p23;
          piece_bf16<BIAS, ACC16>(acc, alpha, bq, 2 * half + mm, n, b, p01, p23);
          *reinterpret_cast<uint2*>(lds + (mm * 32 + li) * kEpiRowBytes + (n * 32 + 8 * b + 4 * h) * 2) =
              make_uint2(p01, p23);
        }
    }
    // the same wave reads back what it wrote: LDS executes one wave's operations in order
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = it * 4 + (lane >> 4), c16 = lane & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * kEpiRowBytes + c16 * 16);
      uint16_t* o = static_cast<uint16_t*>(out) + (m0w + half * 64 + row) * ldc + n0w + c16 * 8;
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(o));
    }
  }
}

// The workgroup's epilogue (4 waves, 2x2 wave tiles of a 256x256 C tile). `lds` is the
// workgroup's stage memory, at least 4 * kEpiWaveBytes bytes, which no wave reads or loads into
// any more (every global -> LDS load has completed). The choice of path is uniform across the
// workgroup, so the barrier is reached by all waves or none.
template <bool OUT_F32, int BIAS, bool ACC16>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], const float (&alpha)[4],
                                           int64_t m0, int64_t n0, int wm, int wn, int64_t M,
                                           int64_t N, void* out, int64_t ldc, bool vec_store,
                                           uint8_t* lds, int wave, int lane, int li, int h,
                                           const void* bias = nullptr) {
  const bool whole = !OUT_F32 && m0 + 256 <= M && n0 + 256 <= N && ldc % 8 == 0 &&
                     (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  if (whole) {
    __syncthreads();   // every wave is done reading the stage buffers the images overlay
    store_wave_tile_staged<BIAS, ACC16>(acc, alpha, m0 + wm * 128, n0 + wn * 128, N, out, ldc,
                                 lds + wave * kEpiWaveBytes, lane, li, h, bias);
  } else {
    store_wave_tile<OUT_F32, BIAS, ACC16>(acc, alpha, m0 + wm * 128, n0 + wn * 128, M, N, out, ldc,
                                   vec_store, li, h, bias);
  }
}

// Deferred epilogue of the persistent kernels. A wave's finished bf16 128x128 tile that lies wholly
// inside C (rows 16-byte aligned) is written as a row-major image into the wave's own LDS area
// (kImgWaveBytes; rows kImgRowBytes apart, as in the staged epilogue) and leaves later as
// kImgStores row-segment stores, each four whole 256-byte rows, issued one at a time between the
// MFMAs of the next tile's first K steps. The stores of all the workgroups then do not leave in
// one burst at the end of each round of tiles, and a K step's loads queue behind at most one of
// them (vector memory completes loads and stores in issue order). Only the wave that wrote an
// image reads it, so no workgroup barrier is needed: LDS executes one wave's operations in order.
constexpr int kImgRowBytes = kEpiRowBytes;

// x, hidden from the optimizer: values computed from it are computed where it is used.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
constexpr int kImgWaveBytes = 128 * kImgRowBytes;
constexpr int kImgStores = 32;

template <int BIAS, bool ACC16>
__device__ __forceinline__ void img_write(const f32x16 (&acc)[4][4], const float (&alpha)[4],
                                          int64_t n0w, int64_t N, uint8_t* img, int li, int h,
                                          const void* bias = nullptr) {
  float bq[4][4][4];
  load_bias<BIAS>(bq, n0w, N, h, bias);
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t p01, p23;
        piece_bf16<BIAS, ACC16>(acc, alpha, bq, m, n, b, p01, p23);
        *reinterpret_cast<uint2*>(img + (m * 32 + li) * kImgRowBytes + (n * 32 + 8 * b + 4 * h) * 2) =
            make_uint2(p01, p23);
      }
}

// Row-segment load s (0 .. kImgStores-1) of a wave's image: rows 4s .. 4s+3, 16 bytes per lane.
__device__ __forceinline__ u32x4 img_load(const uint8_t* img, int s, int lane) {
  return *reinterpret_cast<const u32x4*>(img + (4 * s + (lane >> 4)) * kImgRowBytes + (lane & 15) * 16);
}
// ... and its store to C, `base` pointing at the wave tile's first element. The pointer is
// marked global: a store through a generic pointer might write LDS, and the compiler would then
// drain every outstanding load before the next LDS read.
typedef __attribute__((address_space(1))) u32x4 global_u32x4;
__device__ __forceinline__ void img_put(const u32x4& v, int s, uint16_t* base, int64_t ldc, int lane) {
  uint16_t* o = base + (int64_t)(4 * s + (lane >> 4)) * ldc + (lane & 15) * 8;
  __builtin_nontemporal_store(v, (global_u32x4*)(o));
}

// GELU + NVFP4 epilogue: instead of C, the NVFP4 encoding of gelu(C) (the input of the next
// linear layer, quantized with the static global scale *gsf): packed e2m1 [M, N/2] (row stride N/2
// bytes) and e4m3 scales in the 128x4 layout over [ceil(M/128)*128, N/16], rows M.. of the last
// 128-row tile zero. Each value is what the separate kernels give: C rounded to bf16, gelu in fp32
// rounded to bf16, then nvfp4 quantize. Needs N % 128 == 0, so a wave's 128 columns are all inside
// or all outside C and its scale columns fill two whole 128x4 tiles.
// The bf16 image of 64 rows is built as in the staged epilogue; each lane then takes one 16-byte
// segment (8 values, half a 16-value block, the other half in the neighbouring lane), encodes it
// and writes 4 bytes; the scale bytes gather in a 1 KB image of the wave's two 512-byte scale
// tiles, stored whole at the end. rtab[c] = fl32(g / e4m3(c)) for the 127 scale codes.
// One 64-row half of the GELU + NVFP4 wave epilogue, from its bf16 image in `lds`. ROWS_IN: all
// 64 rows lie below M (no per-row checks, so that the loop has no branches and the LDS latencies
// of its iterations overlap).
template <bool ROWS_IN>
__device__ __forceinline__ void gelu_nvfp4_half(const uint8_t* lds, int half, int64_t m0w,
                                                int64_t n0w, int64_t M, int64_t half_n,
                                                uint8_t* packed, float g, const float* rtab,
                                                const uint16_t* gtab, uint8_t* sfimg, int lane) {
  const int c16 = lane & 15;
  uint4 seg[16], gv[16];
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (it * 4 + (lane >> 4)) * kEpiRowBytes + c16 * 16);
    seg[it] = make_uint4(v.x, v.y, v.z, v.w);
  }
  gelu_segments_tab<16, true>(seg, gv, gtab);
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int rr = half * 64 + it * 4 + (lane >> 4);  // row inside the wave's 128 rows
    const int64_t gm = m0w + rr;
    const float a = pair_max(mag_value(mag_bits8(gv[it])));
    float f[8];
    unpack8(gv[it], f);
    const uint32_t S = (ROWS_IN || gm < M) ? e4m3_encode_pos(g * (a * kSixth)) : 0u;
    const float r = rtab[S];
    uint32_t o = 0;
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[0] * r, f[1] * r, 1.0f, 0);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[2] * r, f[3] * r, 1.0f, 1);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[4] * r, f[5] * r, 1.0f, 2);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[6] * r, f[7] * r, 1.0f, 3);
    if (ROWS_IN || gm < M)
      __builtin_nontemporal_store(o, reinterpret_cast<uint32_t*>(packed + gm * half_n + n0w / 2 + c16 * 4));
    // both lanes of a block hold its scale code: both store it, to the same byte
    const int cb = c16 >> 1;  // scale column inside the wave's 8
    sfimg[(cb >> 2) * 512 + (rr & 31) * 16 + (rr >> 5) * 4 + (cb & 3)] = (uint8_t)S;
  }
}

__device__ __forceinline__ void store_wave_tile_gelu_nvfp4(const f32x16 (&acc)[4][4],
                                                           const float (&alpha)[4], int64_t m0w,
                                                           int64_t n0w, int64_t M, int64_t N,
                                                           uint8_t* packed, uint8_t* sf, float g,
                                                           const float* rtab, const uint16_t* gtab,
                                                           uint8_t* lds, uint8_t* sfimg, int lane,
                                                           int li, int h) {
  if (n0w >= N) return;
  const float bq[4][4][4] = {};
  const int64_t half_n = N / 2;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          uint32_t p01, p23;
          piece_bf16<kBiasNone, true>(acc, alpha, bq, 2 * half + mm, n, b, p01, p23);
          *reinterpret_cast<uint2*>(lds + (mm * 32 + li) * kEpiRowBytes + (n * 32 + 8 * b + 4 * h) * 2) =
              make_uint2(p01, p23);
        }
    }
    // the same wave reads back what it wrote: LDS executes one wave's operations in order
    if (m0w + half * 64 + 64 <= M)
      gelu_nvfp4_half<true>(lds, half, m0w, n0w, M, half_n, packed, g, rtab, gtab, sfimg, lane);
    else
      gelu_nvfp4_half<false>(lds, half, m0w, n0w, M, half_n, packed, g, rtab, gtab, sfimg, lane);
  }
  // the wave's two 512-byte scale tiles: row tile m0w / 128, column groups n0w / 64 and + 1
  if (m0w < M) {
    const int64_t groups = N / 64;
    const int64_t tile = (m0w / 128) * groups + n0w / 64 + (lane >> 5);
    const u32x4 v = reinterpret_cast<const u32x4*>(sfimg)[lane];
    *reinterpret_cast<u32x4*>(sf + tile * 512 + (lane & 31) * 16) = v;
  }
}

// Workgroup epilogue for the GELU + NVFP4 output. The images overlay the stage memory `lds`
// (at least 4 * (kEpiWaveBytes + 1024) bytes); rtab (128 floats) and gtab (kGeluTabSize) are the
// workgroup's scale-reciprocal and GELU tables, filled here.
__device__ __forceinline__ void store_tile_gelu_nvfp4(const f32x16 (&acc)[4][4],
                                                      const float (&alpha)[4], int64_t m0,
                                                      int64_t n0, int wm, int wn, int64_t M,
                                                      int64_t N, uint8_t* packed, uint8_t* sf,
                                                      const float* gsf, float* rtab, uint16_t* gtab,
                                                      uint8_t* lds, int t, int wave, int lane,
                                                      int li, int h) {
  const float g = *gsf;
  if (t < 128) rtab[t] = (t == 0 || t > 0x7E) ? 0.0f : g / e4m3_decode_pos((uint32_t)t);
  gelu_table_load(gtab, t, 256);
  __syncthreads();   // the tables; every wave is done reading the stage buffers the images overlay
  store_wave_tile_gelu_nvfp4(acc, alpha, m0 + wm * 128, n0 + wn * 128, M, N, packed, sf, g, rtab,
                             gtab, lds + wave * kEpiWaveBytes, lds + 4 * kEpiWaveBytes + wave * 1024,
                             lane, li, h);
}

}  // namespace bsp
