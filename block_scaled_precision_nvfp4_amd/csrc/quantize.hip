// HBM-bound kernels of the NVFP4 / MXFP8 linear layer on gfx950:
//   the weight global scale (amax reduction + scalar finish), NVFP4 quantize (per tensor, per
//   token, layout_8x4, fused with GELU or with RMSNorm), alpha, MXFP8 and MXFP4 quantize, the bf16
//   GELU between the FFN projections and the standalone RMSNorm.
//
// Pages (by title, section): FastVideo nvfp4_qat_config.py (convert_model_to_fp4, apply),
// FastVideo nvfp4_config.py (module docstring, _nvfp4_quantize and its shape kernel,
// convert_model_to_nvfp4), SGLang nvfp4_online.py (_quantize_weight_nvfp4),
// vLLM-Omni mxfp8_config.py (DiffusionMXFP8Config, NPUMxfp8LinearMethod).
#include <cfloat>

#include "common.hpp"

namespace bsp {

// =============================================================================================
// Weight global scale
// =============================================================================================
// |bf16| magnitude bits after nan_to_num: NaN -> 0, inf -> largest finite (0x7F7F). Magnitude
// bit patterns of non-negative bf16 values order like the values, so the max is an integer max.
__device__ __forceinline__ uint32_t mag_nan_to_num(uint32_t b16) {
  uint32_t m = b16 & 0x7FFFu;
  return m > 0x7F80u ? 0u : (m == 0x7F80u ? 0x7F7Fu : m);
}

// The quantizers read each input byte once and write each output byte once: their global loads and
// stores are nontemporal (they do not displace other data in the caches; measured 20-30 % faster
// when the caches hold another kernel's dirty output).
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const nt_u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store4_nt(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

__global__ void amax_init_kernel(float* amax) { *reinterpret_cast<uint32_t*>(amax) = 0u; }

__device__ __forceinline__ uint32_t mag_max8(uint32_t m, const uint4& v) {
  const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m = max(m, mag_nan_to_num(q[j] & 0xFFFFu));
    m = max(m, mag_nan_to_num(q[j] >> 16));
  }
  return m;
}

// MODE 0: contiguous rows (ld == K, K % 8 == 0, 16-byte aligned): the matrix is one run of
//   16-byte chunks, four loads in flight per thread per step, no index division;
// MODE 1: strided rows with K % 8 == 0, ld % 8 == 0, 16-byte aligned: workgroups stride over rows,
//   threads over a row's chunks;
// MODE 2: anything else, element by element.
template <int MODE>
__global__ __launch_bounds__(256) void amax_reduce_kernel(const uint16_t* __restrict__ w, int64_t rows,
                                                          int64_t K, int64_t ld, float* amax) {
  uint32_t m = 0;
  if (MODE == 0) {
    const uint4* c = reinterpret_cast<const uint4*>(w);
    const int64_t total = rows * (K / 8);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // plain (not nontemporal) loads: the quantize that follows at load time reads W again
    for (; i + 7 * stride < total; i += 8 * stride) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c[i + u * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) m = mag_max8(m, v[u]);
    }
    for (; i < total; i += stride) m = mag_max8(m, c[i]);
  } else if (MODE == 1) {
    const int64_t cpr = K / 8;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
      const uint4* c = reinterpret_cast<const uint4*>(w + r * ld);
      for (int64_t j = threadIdx.x; j < cpr; j += blockDim.x) m = mag_max8(m, c[j]);
    }
  } else {
    const int64_t total = rows * K;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
      int64_t r = i / K, c = i - r * K;
      m = max(m, mag_nan_to_num(w[r * ld + c]));
    }
  }
  // wave max, then across the 4 waves through LDS, then one atomic per block
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = max(max(part[0], part[1]), max(part[2], part[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), b << 16);  // non-negative fp32 bits order as uint
  }
}

__global__ void gsf_finish_kernel(float* amax, float* gsf, float* inv_gsf) {
  float a = *amax;
  float g = (a == 0.0f) ? 1.0f : 2688.0f / a;  // 448 * 6 / amax, one IEEE division
  *gsf = g;
  *inv_gsf = 1.0f / g;
}

// 4over6 variant (SGLang nvfp4_online.py, _quantize_weight_nvfp4): the largest block scale is taken
// as 256, the decode scale is fl32(amax / 1536) (1 when amax == 0) and the encode scale its fl32
// reciprocal, computed in that order.
__global__ void gsf_finish_4over6_kernel(float* amax, float* gsf, float* inv_gsf) {
  float a = *amax;
  float dec = (a == 0.0f) ? 1.0f : a / 1536.0f;
  float g = 1.0f / dec;
  *gsf = g;
  *inv_gsf = 1.0f / g;
}

// =============================================================================================
// alpha = fl32(1 / fl32(x_gsf * w_gsf))
// =============================================================================================
__global__ void alpha_kernel(const float* xg, const float* wg, float* alpha) {
  float p = (*xg) * (*wg);
  *alpha = 1.0f / p;
}

// =============================================================================================
// NVFP4 quantize
// =============================================================================================
// One workgroup quantizes a 128-row x 256-K tile (16 scale columns = 4 column groups of the
// 128x4 scale layout, i.e. four whole 512-byte scale tiles). 256 threads = 8 rows x 32 lanes;
// each lane owns 8 consecutive K elements (one 16-byte load), so a 16-element block is a lane
// pair and its amax is a DPP pair max. The tile is walked in 16 steps of 8 rows; all 16 loads
// are issued before any arithmetic. Scale bytes are staged in LDS at their 128x4 positions and
// leave as coalesced 16-byte stores of whole 512-byte tiles. Rows M..Mp-1 and columns past K
// read as zeros (no copy of the input is made), which yields the 0x00 padding scales. Interior
// tiles (the common case) take a path without per-row bounds checks.
//
// The element scale r = fl32(g / e4m3(S)) depends only on the 7-bit code S, so each workgroup
// first tabulates it for all 127 codes (the same IEEE division, once per code) and blocks look it
// up. Elements are encoded with v_cvt_scalef32_pk_fp4_f32 (unit scale): round to nearest even,
// saturating at +-6, sign of zero kept -- checked against the software encoder on every fp32
// input class (ties, denormals, huge values) on gfx950; BSP_QUANT_SW_CVT=1 selects that software
// encoder instead.
//
// FRAG: the packed values in the fragment layout (K % 64 == 0; described at
// bsp_nvfp4_quantize_frag), the scales still in 128x4. The workgroup's 128 rows x 256 K are 4 row
// tiles x 4 K steps, sixteen 1 KB fragments staged in LDS and stored as four contiguous 4 KB runs
// (steps past K are not stored). A thread's 4 bytes for row rr lie in 16-byte chunk
// p = (rr/32)*256 + cb*32 + rr%32 of the staging area (cb = (t % 32) / 4 = 2 * K step + lane half),
// placed at chunk p ^ 2cb: the eight 32-element blocks of a row otherwise sit 512 bytes apart, all
// in one LDS bank.
template <bool VEC>
__device__ __forceinline__ uint4 load8(const uint16_t* p) {
  if (VEC) return load16_nt(p);
  uint4 v;
  v.x = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
  v.y = (uint32_t)p[2] | ((uint32_t)p[3] << 16);
  v.z = (uint32_t)p[4] | ((uint32_t)p[5] << 16);
  v.w = (uint32_t)p[6] | ((uint32_t)p[7] << 16);
  return v;
}

template <bool HWCVT, bool VEC, bool GELU, bool WIDE, bool FRAG = false>
__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(const uint16_t* __restrict__ x,
                                                             int64_t M, int64_t K, int64_t ld,
                                                             const float* __restrict__ gsf,
                                                             uint8_t* __restrict__ packed,
                                                             uint8_t* __restrict__ sf, int64_t Kp,
                                                             int64_t rows8) {
  __shared__ uint4 sf_tile[128];  // 2 KB = 4 scale tiles of 512 B
  // WIDE: the tile's packed bytes (128 rows x 128 B), stored as 16-byte pieces; FRAG: its 16
  // fragments
  __shared__ __attribute__((aligned(16))) uint32_t pimg[WIDE || FRAG ? 128 * 32 : 1];
  __shared__ float rtab[128];     // fl32(g / e4m3(c)) for code c (0 for c == 0)
  __shared__ __attribute__((aligned(16))) uint16_t gtab[GELU ? kGeluTabSize : 8];
  uint8_t* sfb = reinterpret_cast<uint8_t*>(sf_tile);
  const int t = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * 128;
  const int64_t kk = (int64_t)blockIdx.x * 256 + (t & 31) * 8;
  const int rsub = t >> 5;
  const bool kin = kk < K;  // K % 16 == 0: a lane's 8 elements are all in range or all out
  const bool full = row0 + 128 <= M && (int64_t)blockIdx.x * 256 + 256 <= K;  // uniform
  const float g = *gsf;
  if (t < 128) rtab[t] = (t == 0 || t > 0x7E) ? 0.0f : g / e4m3_decode_pos((uint32_t)t);

  const uint16_t* xp = x + (row0 + rsub) * ld + kk;
  const int64_t xstep = 8 * ld;
  uint4 v[16];
  if (full) {
#pragma unroll
    for (int s = 0; s < 16; ++s) v[s] = load8<VEC>(xp + s * xstep);
  } else {
#pragma unroll
    for (int s = 0; s < 16; ++s)
      v[s] = (kin && row0 + s * 8 + rsub < M) ? load8<VEC>(xp + s * xstep) : make_uint4(0u, 0u, 0u, 0u);
  }
  if (GELU) gelu_table_load(gtab, t, 256);   // while the loads are in flight
  __syncthreads();  // rtab, gtab
  if (!GELU) nan_to_num_segments(v);   // the GELU path substitutes in its table-miss branch

  const int64_t half_k = K / 2;
  const bool wide = WIDE && full;   // uniform: interior tiles
  uint8_t* pp = packed + (row0 + rsub) * half_k + kk / 2;
  const int64_t pstep = 8 * half_k;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    uint4 xv[1] = {v[s]};
    if (GELU) gelu_segments_tab<1, true>({v[s]}, xv, gtab);  // gelu(0) = 0 keeps the padding zero
    const float a = pair_max(mag_value(mag_bits8(xv[0])));
    float f[8];
    unpack8(xv[0], f);
    const float sc = g * (a * kSixth);
    const uint32_t S = e4m3_encode_pos(sc);
    const float r = rtab[S];
    uint32_t out = 0;
    if (HWCVT) {
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[0] * r, f[1] * r, 1.0f, 0);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[2] * r, f[3] * r, 1.0f, 1);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[4] * r, f[5] * r, 1.0f, 2);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[6] * r, f[7] * r, 1.0f, 3);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out |= e2m1_encode(f[i] * r) << (4 * i);
    }
    const int rr = s * 8 + rsub;  // row inside the 128-row tile
    if (FRAG) {
      const int cb = (t & 31) >> 2;
      const int p = (rr >> 5) * 256 + cb * 32 + (rr & 31);
      pimg[(p ^ (cb << 1)) * 4 + (t & 3)] = out;
    } else if (wide) pimg[rr * 32 + (t & 31)] = out;
    else if (full || (kin && row0 + rr < M)) store4_nt(pp + s * pstep, out);
    if ((t & 1) == 0) {
      const int cb = (t & 31) >> 1;  // scale column inside the 16-column tile
      sfb[(cb >> 2) * 512 + (rr & 31) * 16 + (rr >> 5) * 4 + (cb & 3)] = (uint8_t)S;
    }
  }
  __syncthreads();
  if (FRAG) {
    // row tiles past ceil(M / 32) are not part of the buffer; padded rows inside the last one were
    // encoded from zeros
    const int64_t row_tiles = (M + 31) / 32, rt0 = (int64_t)blockIdx.y * 4;
    const int64_t ks = K / 64, ks0 = (int64_t)blockIdx.x * 4;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int p = it * 256 + t;   // chunk (p & 255) of row tile it: K step (p >> 6) & 3, lane p & 63
      if (rt0 + it < row_tiles && ks0 + ((p >> 6) & 3) < ks) {
        const uint4 w = reinterpret_cast<const uint4*>(pimg)[p ^ (((p >> 5) & 7) << 1)];
        __builtin_nontemporal_store(
            (nt_u32x4){w.x, w.y, w.z, w.w},
            reinterpret_cast<nt_u32x4*>(packed + ((rt0 + it) * ks + ks0) * 1024) + (p & 255));
      }
    }
  } else if (wide) {   // each row's 128 bytes as eight 16-byte pieces
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = t + 256 * i, rr = p >> 3, part = p & 7;
      const uint4 w = *reinterpret_cast<const uint4*>(&pimg[rr * 32 + part * 4]);
      __builtin_nontemporal_store(
          (nt_u32x4){w.x, w.y, w.z, w.w},
          reinterpret_cast<nt_u32x4*>(packed + (row0 + rr) * half_k + (int64_t)blockIdx.x * 128 + part * 16));
    }
  }
  const int64_t groups = Kp / 4;                       // 4-column groups in the matrix
  const int64_t g0 = (int64_t)blockIdx.x * 4;
  const int64_t ng = groups - g0 < 4 ? groups - g0 : 4;
  if (rows8 == 0) {                                    // 128x4: four whole 512-byte tiles
    if (t < ng * 32) {
      const int cg = t >> 5;
      const int64_t tile = (int64_t)blockIdx.y * groups + g0 + cg;
      reinterpret_cast<uint4*>(sf + tile * 512)[t & 31] = sf_tile[cg * 32 + (t & 31)];
    }
  } else {
    // 8x4 (rows padded to rows8, a multiple of 8): 32-byte tiles of 8 rows x 4 columns, row-tile
    // major. A row's 4 scales of a column group are one dword in both layouts; 8 consecutive
    // threads write one tile and 32 threads four neighbouring tiles (128 contiguous bytes).
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(sf_tile);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = t + 256 * i;
      const int rr = (idx >> 5) * 8 + (idx & 7), cg = (idx >> 3) & 3;
      const int64_t r = row0 + rr;
      if (cg < ng && r < rows8)
        reinterpret_cast<uint32_t*>(sf)[((r >> 3) * groups + g0 + cg) * 8 + (r & 7)] =
            sw[cg * 128 + (rr & 31) * 4 + (rr >> 5)];
    }
  }
}

// =============================================================================================
// NVFP4 quantize with per-token (per-row) activation scales
// =============================================================================================
// One wave owns one row. The row is read in segments of 64 lanes x C chunks of 8 elements (lane l
// holds elements (64 j + l) * 8 .. + 7 of chunk j); its amax is a wave max and its encode scale is
// gsf_m = 2688 / amax (one IEEE division; 1 for an all-zero row), the tensor-scale rule applied to
// the row. The wave tabulates fl32(gsf_m / e4m3(c)) for the 127 codes in LDS, then quantizes the
// blocks (lane pairs) exactly as the per-tensor kernel does. When the padded row fits one segment
// (K <= 64 * 8 * C) it stays in registers between the two phases (one pass over HBM); longer rows
// are read twice. Rows M..Mp-1 run as zero rows, which writes their 0x00 padding scales. The four
// waves of a workgroup own rows q, q+32, q+64, q+96 of one 128-row tile, whose scales of a column
// group form one 16-byte run of the 128x4 layout: they are gathered in LDS and leave as 16-byte
// stores.
constexpr int kTokMaxCols = 1024;  // scale columns per row staged in LDS (K <= 16384 per segment set)

// The row's registers, hidden from the optimizer between a kernel's two passes over them: the
// second pass then unpacks them again instead of keeping the first pass's unpacked values live
// (eight registers per chunk, which lowered the RMSNorm kernel's occupancy from 7 to 5 waves).
template <int C>
__device__ __forceinline__ void rows_opaque(uint4 (&v)[C]) {
#pragma unroll
  for (int j = 0; j < C; ++j) asm volatile("" : "+v"(v[j].x), "+v"(v[j].y), "+v"(v[j].z), "+v"(v[j].w));
}

// A per-row kernel's packed bytes of one segment leave from an LDS image of the wave's row,
// 16 bytes per lane (1 KB per store instruction): the four-byte-per-lane stores of the encode loop
// measured about 12 % slower for the whole per-token kernel at K = 5120. WIDE needs K % 32 == 0 and
// a 16-byte aligned packed matrix (every row then starts 16-byte aligned); otherwise each lane's
// four bytes are stored from the encode loop. nb: the segment's packed bytes (a multiple of 16).
__device__ __forceinline__ void store_row_wide(const uint32_t* img, uint8_t* __restrict__ dst,
                                               int64_t nb, int lane) {
  for (int64_t o = (int64_t)lane * 16; o < nb; o += 64 * 16) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(img) + o);
    __builtin_nontemporal_store((nt_u32x4){w.x, w.y, w.z, w.w}, reinterpret_cast<nt_u32x4*>(dst + o));
  }
}

template <int C, bool VEC, bool WIDE>
__global__ __launch_bounds__(256) void nvfp4_quantize_token_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ld, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ sf, float* __restrict__ gsf_rows, int64_t Kp) {
  __shared__ float rtab[4][128];
  __shared__ uint32_t srow[4][kTokMaxCols / 4];
  __shared__ __attribute__((aligned(16))) uint32_t pimg[WIDE ? 4 : 1][WIDE ? C * 64 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // workgroups q and q + 1 of a tile write neighbouring 16-byte runs of each scale tile: one XCD
  const int64_t wg = xcd_blocked(blockIdx.x, gridDim.x);
  const int64_t tile = wg >> 5, q = wg & 31;
  const int64_t row = tile * 128 + q + 32 * wave;
  const bool live = row < M;
  const int64_t seg_elems = 64 * 8 * C;
  const int64_t kpad = Kp * 16;                     // elements incl. the padding scale columns
  const int nseg = (int)((kpad + seg_elems - 1) / seg_elems);
  const uint16_t* xr = x + (live ? row : 0) * ld;

  uint4 v[C];
  uint32_t mrow = 0;   // the row's largest magnitude, as bf16 bits (mag_bits8)
  for (int sg = 0; sg < nseg; ++sg) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int64_t e = sg * seg_elems + (int64_t)(j * 64 + lane) * 8;
      v[j] = (live && e < K) ? load8<VEC>(xr + e) : make_uint4(0u, 0u, 0u, 0u);
      mrow = max(mrow, mag_bits8(v[j]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mrow = max(mrow, (uint32_t)__shfl_xor((int)mrow, off));
  // a row holding an inf or a NaN (wave-uniform, rare): its amax after nan_to_num, with the
  // registers of a one-segment row replaced in place
  const bool nonfinite = mrow >= 0x7F80u;
  if (nonfinite) {
    mrow = 0;
    for (int sg = 0; sg < nseg; ++sg) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int64_t e = sg * seg_elems + (int64_t)(j * 64 + lane) * 8;
        if (nseg > 1) v[j] = (live && e < K) ? load8<VEC>(xr + e) : make_uint4(0u, 0u, 0u, 0u);
        v[j] = nan_to_num8(v[j]);
        mrow = max(mrow, mag_bits8(v[j]));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mrow = max(mrow, (uint32_t)__shfl_xor((int)mrow, off));
  }
  const float amax = mag_value(mrow);
  const float g = (amax == 0.0f) ? 1.0f : 2688.0f / amax;  // 448 * 6 / amax, one IEEE division
  if (live && lane == 0) gsf_rows[row] = g;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = lane + 64 * h;
    rtab[wave][c] = (c == 0 || c > 0x7E) ? 0.0f : g / e4m3_decode_pos((uint32_t)c);
  }
  __syncthreads();

  const int64_t half_k = K / 2;
  uint8_t* prow = packed + (live ? row : 0) * half_k;
  uint8_t* sb = reinterpret_cast<uint8_t*>(srow[wave]);
  for (int sg = 0; sg < nseg; ++sg) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int64_t e = sg * seg_elems + (int64_t)(j * 64 + lane) * 8;
      if (nseg > 1) {
        v[j] = (live && e < K) ? load8<VEC>(xr + e) : make_uint4(0u, 0u, 0u, 0u);
        if (nonfinite) v[j] = nan_to_num8(v[j]);
      }
      const float a = pair_max(mag_value(mag_bits8(v[j])));
      float f[8];
      unpack8(v[j], f);
      const uint32_t S = e4m3_encode_pos(g * (a * kSixth));
      const float r = rtab[wave][S];
      uint32_t out = 0;
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[0] * r, f[1] * r, 1.0f, 0);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[2] * r, f[3] * r, 1.0f, 1);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[4] * r, f[5] * r, 1.0f, 2);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[6] * r, f[7] * r, 1.0f, 3);
      if (WIDE) pimg[wave][j * 64 + lane] = out;
      else if (live && e < K) store4_nt(prow + e / 2, out);
      const int64_t col = e / 16;                         // scale column of this lane pair
      if ((lane & 1) == 0 && col < Kp) sb[col % kTokMaxCols] = (uint8_t)S;
    }
    if (WIDE && live) {
      const int64_t e0 = sg * seg_elems;
      store_row_wide(pimg[wave], prow + e0 / 2, (e0 + seg_elems < K ? seg_elems : K - e0) / 2, lane);
    }
    // this segment's scale columns [sg * seg_elems / 16, ...): per column group, the dwords of
    // the four waves' rows are one 16-byte run at (q * 16) of the group's 512-byte tile
    __syncthreads();
    const int64_t c0 = sg * seg_elems / 16;
    const int64_t c1 = c0 + seg_elems / 16 < Kp ? c0 + seg_elems / 16 : Kp;
    const int64_t groups = Kp / 4;
    for (int64_t cg = c0 / 4 + threadIdx.x; cg < c1 / 4; cg += 256) {
      const int i = (int)(cg % (kTokMaxCols / 4));
      *reinterpret_cast<uint4*>(sf + (tile * groups + cg) * 512 + q * 16) =
          make_uint4(srow[0][i], srow[1][i], srow[2][i], srow[3][i]);
    }
    __syncthreads();
  }
}

// =============================================================================================
// RMSNorm, alone (bf16 out) or followed by the NVFP4 quantize of its bf16 output
// =============================================================================================
// The norm whose fused quantize hands mm_fp4 a pre-quantized activation (FastVideo
// nvfp4_config.py, NVFP4QuantizeMethod.apply: FlashInfer's fused norm + quantize producers; the
// page does not name the norm, RMSNorm is the norm of the LTX-2 blocks it quantizes):
//   y = bf16( fl32( fl32(x * r) * w ) ),  r = fl32( 1 / sqrt(ss / K + eps) ),
// w the optional bf16 gain (no multiply without one). ss, the sum of the row's squares, and r are
// evaluated in fp64 (a bf16 square is exact there and the sums of up to 2^24 of them stay within
// about 2^-29 relative), so r is the fp32 rounding of the exact value up to a few fp64 ulps; the
// two products and the bf16 rounding are fp32. Each lane adds its own squares in element order,
// then a butterfly over the wave. Row placement is
// the per-token kernel's: one wave per row, rows q, q+32, q+64, q+96 of a 128-row tile per
// workgroup, the row held in registers between the two phases when it fits one segment. QUANT
// then encodes y exactly as nvfp4_quantize_kernel does (element scales tabulated once per
// workgroup from the device global scale); otherwise y is stored. The same arithmetic in both
// forms, so the fused bytes equal the NVFP4 quantize of the standalone output. Padding rows
// (M..Mp-1) run with r = 0, which writes their 0x00 scales.
template <int C, bool VEC, bool QUANT, bool GAIN, bool WIDE>
__global__ __launch_bounds__(256) void rmsnorm_token_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ld,
    const uint16_t* __restrict__ wgain, float eps, const float* __restrict__ gsf,
    uint16_t* __restrict__ out, int64_t ldo, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ sf, int64_t Kp) {
  __shared__ float rtab[QUANT ? 128 : 1];
  __shared__ uint32_t srow[QUANT ? 4 : 1][QUANT ? kTokMaxCols / 4 : 1];
  __shared__ __attribute__((aligned(16))) uint32_t pimg[QUANT && WIDE ? 4 : 1][QUANT && WIDE ? C * 64 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // workgroups q and q + 1 of a tile write neighbouring 16-byte runs of each scale tile: one XCD
  const int64_t wg = xcd_blocked(blockIdx.x, gridDim.x);
  const int64_t tile = wg >> 5, q = wg & 31;
  const int64_t row = tile * 128 + q + 32 * wave;
  const bool live = row < M;
  const int64_t seg_elems = 64 * 8 * C;
  const int64_t kpad = QUANT ? Kp * 16 : K;        // elements incl. the padding scale columns
  const int nseg = (int)((kpad + seg_elems - 1) / seg_elems);
  const uint16_t* xr = x + (live ? row : 0) * ld;
  float g = 1.0f;
  if (QUANT) {
    g = *gsf;
    if (threadIdx.x < 128) {
      const int c = threadIdx.x;
      rtab[c] = (c == 0 || c > 0x7E) ? 0.0f : g / e4m3_decode_pos((uint32_t)c);
    }
    // the table, before any load: the waves start together, while a barrier after the loads would
    // hold each wave until the slowest one's row has arrived
    __syncthreads();
  }

  uint4 v[C];
  double ss = 0.0;
  for (int sg = 0; sg < nseg; ++sg) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int64_t e = sg * seg_elems + (int64_t)(j * 64 + lane) * 8;
      v[j] = (live && e < K) ? load8<VEC>(xr + e) : make_uint4(0u, 0u, 0u, 0u);
      float f[8];
      unpack8(v[j], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double d = (double)f[i];
        ss = __builtin_fma(d, d, ss);  // d * d is exact in fp64, so this is the rounded sum
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = live ? (float)(1.0 / sqrt(ss / (double)K + (double)eps)) : 0.0f;
  // y can only be infinite or NaN when the row is (ss, a sum of squares, is then infinite or NaN)
  // or when a gain multiplies it: only then does the encoder need its input substituted
  const bool maybe_nonfinite = GAIN || !(ss <= DBL_MAX);
  rows_opaque<C>(v);

  const int64_t half_k = K / 2;
  uint8_t* prow = QUANT ? packed + (live ? row : 0) * half_k : nullptr;
  uint16_t* orow = QUANT ? nullptr : out + (live ? row : 0) * ldo;
  uint8_t* sb = reinterpret_cast<uint8_t*>(srow[QUANT ? wave : 0]);
  for (int sg = 0; sg < nseg; ++sg) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int64_t e = sg * seg_elems + (int64_t)(j * 64 + lane) * 8;
      const bool in = live && e < K;
      if (nseg > 1) v[j] = in ? load8<VEC>(xr + e) : make_uint4(0u, 0u, 0u, 0u);
      float f[8];
      unpack8(v[j], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] * r;
      if (GAIN) {
        float w[8];
        unpack8(e < K ? load8<VEC>(wgain + e) : make_uint4(0u, 0u, 0u, 0u), w);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = f[i] * w[i];
      }
      uint4 y = make_uint4(bf16x2_rne(f[0], f[1]), bf16x2_rne(f[2], f[3]),
                           bf16x2_rne(f[4], f[5]), bf16x2_rne(f[6], f[7]));
      if (!QUANT) {
        if (in) {
          if (VEC) {
            __builtin_nontemporal_store((nt_u32x4){y.x, y.y, y.z, y.w},
                                        reinterpret_cast<nt_u32x4*>(orow + e));
          } else {
            const uint32_t yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              orow[e + 2 * i] = (uint16_t)(yw[i] & 0xFFFFu);
              orow[e + 2 * i + 1] = (uint16_t)(yw[i] >> 16);
            }
          }
        }
        continue;
      }
      if (maybe_nonfinite) y = nan_to_num8(y);   // wave-uniform
      const float a = pair_max(mag_value(mag_bits8(y)));
      unpack8(y, f);
      const uint32_t S = e4m3_encode_pos(g * (a * kSixth));
      const float rs = rtab[S];
      uint32_t o = 0;
      o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[0] * rs, f[1] * rs, 1.0f, 0);
      o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[2] * rs, f[3] * rs, 1.0f, 1);
      o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[4] * rs, f[5] * rs, 1.0f, 2);
      o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[6] * rs, f[7] * rs, 1.0f, 3);
      if (WIDE) pimg[wave][j * 64 + lane] = o;
      else if (in) store4_nt(prow + e / 2, o);
      const int64_t col = e / 16;
      if ((lane & 1) == 0 && col < Kp) sb[col % kTokMaxCols] = (uint8_t)S;
    }
    if (QUANT && WIDE && live) {
      const int64_t e0 = sg * seg_elems;
      store_row_wide(pimg[wave], prow + e0 / 2, (e0 + seg_elems < K ? seg_elems : K - e0) / 2, lane);
    }
    if (QUANT) {
      __syncthreads();
      const int64_t c0 = sg * seg_elems / 16;
      const int64_t c1 = c0 + seg_elems / 16 < Kp ? c0 + seg_elems / 16 : Kp;
      const int64_t groups = Kp / 4;
      for (int64_t cg = c0 / 4 + threadIdx.x; cg < c1 / 4; cg += 256) {
        const int i = (int)(cg % (kTokMaxCols / 4));
        *reinterpret_cast<uint4*>(sf + (tile * groups + cg) * 512 + q * 16) =
            make_uint4(srow[0][i], srow[1][i], srow[2][i], srow[3][i]);
      }
      __syncthreads();
    }
  }
}

// =============================================================================================
// MXFP8 quantize
// =============================================================================================
// One workgroup covers 64 rows x 256 K (8 steps of 8 rows x 32 lanes x 8 elements). A 32-element
// group is a lane quad; its amax is a DPP quad max. Scale byte = max(biased exponent of amax - 8, 0)
// (that is Es + 127 with Es = clamp(floor(log2 amax) - 8, -127, 127), and 0x00 for amax == 0).
// Elements: x * 2^-Es (exact), clamped to +-448 (saturation), then v_cvt_pk_fp8_f32, which
// rounds to nearest even with the sign of zero kept (its only difference from the software
// encoder on gfx950 is that it does not saturate, hence the clamp); BSP_QUANT_SW_CVT=1 selects
// the software encoder.
//
// FRAG: both outputs in the MFMA fragment layout (K % 256 == 0; described at
// bsp_mxfp8_quantize_frag). The workgroup's 64 rows x 256 K are 2 row tiles x 4 K steps, eight 2 KB
// fragments and two 256-byte scale groups, staged in LDS and stored as two contiguous 8 KB runs
// and two 256-byte runs. A thread's 8 output bytes for row rr and K offset 8 (t % 32) within the
// 256 are half (t & 1) of 16-byte chunk p = (rr/32)*512 + g*32 + rr%32 of the staging area, with
// g = (t % 32) / 2 = 4 * K step + 2 * block + lane half; it is placed at chunk p ^ 2g, as the
// sixteen g of a row otherwise sit 512 bytes apart, in one set of LDS banks.
template <bool HWCVT, bool VEC, bool FRAG = false, bool WIDE = false>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint16_t* __restrict__ x,
                                                             int64_t M, int64_t K, int64_t ld,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ sf) {
  // FRAG: the workgroup's 16 KB of fragments; WIDE: its 64 rows x 256 bytes of codes
  __shared__ uint4 frag_tile[FRAG || WIDE ? 1024 : 1];
  __shared__ uint4 sf_stage[FRAG || WIDE ? 32 : 1];  // FRAG: two 256-byte scale groups; WIDE: 64 x 8
  const int t = threadIdx.x;
  // row-major scales: the 8 scale bytes a workgroup writes per row are a quarter of a 32-byte sector,
  // whose other quarters come from the next three K tiles; those four run on one XCD (one L2)
  const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t wg = FRAG ? lin : xcd_quads(lin, (int64_t)gridDim.x * gridDim.y);
  const int64_t bx = wg % gridDim.x, by = wg / gridDim.x;
  const int64_t row0 = by * 64;
  const int64_t kk = bx * 256 + (t & 31) * 8;
  const int rsub = t >> 5;
  const bool kin = kk < K;  // K % 32 == 0: a quad is entirely in or out
  const bool full = row0 + 64 <= M && bx * 256 + 256 <= K;
  const uint16_t* xp = x + (row0 + rsub) * ld + kk;
  const int64_t xstep = 8 * ld;
  uint4 v[8];
  if (full) {
#pragma unroll
    for (int s = 0; s < 8; ++s) v[s] = load8<VEC>(xp + s * xstep);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      v[s] = (kin && row0 + s * 8 + rsub < M) ? load8<VEC>(xp + s * xstep) : make_uint4(0u, 0u, 0u, 0u);
  }
  nan_to_num_segments(v);
  const int64_t ng = K / 32;
  uint8_t* qp = q + (row0 + rsub) * K + kk;
  uint8_t* sp = sf + (row0 + rsub) * ng + kk / 32;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float a = quad_max(mag_value(mag_bits8(v[s])));
    float f[8];
    unpack8(v[s], f);
    const uint32_t ef = __float_as_uint(a) >> 23;            // biased exponent (a >= 0, finite)
    const uint32_t byte = ef > 8u ? ef - 8u : 0u;            // Es + 127
    const float inv = __uint_as_float((254u - byte) << 23);  // 2^-Es = 2^(127 - byte), exact
    uint32_t lo = 0, hi = 0;
    if (HWCVT) {
      float c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_fmed3f(f[i] * inv, -448.0f, 448.0f);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], lo, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], hi, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) lo |= e4m3_encode(f[i] * inv) << (8 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) hi |= e4m3_encode(f[4 + i] * inv) << (8 * i);
    }
    if constexpr (FRAG) {
      const int rr = s * 8 + rsub, g = (t & 31) >> 1;
      const int p = (rr >> 5) * 512 + g * 32 + (rr & 31);
      uint32_t* d = reinterpret_cast<uint32_t*>(frag_tile) + (p ^ (g << 1)) * 4 + (t & 1) * 2;
      d[0] = lo;
      d[1] = hi;
      if ((t & 3) == 0) {  // block cb = (t % 32) / 4 of the 256 K: K step cb / 2, lane half cb % 2
        const int cb = (t & 31) >> 2;
        reinterpret_cast<uint8_t*>(sf_stage)[(rr >> 5) * 256 + ((cb & 1) * 32 + (rr & 31)) * 4 + (cb >> 1)] =
            (uint8_t)byte;
      }
    } else if (WIDE && full) {
      // row rr's 256 code bytes at rr * 256 of the image; its 8 scale bytes at rr * 8
      const int rr = s * 8 + rsub;
      reinterpret_cast<uint2*>(frag_tile)[rr * 32 + (t & 31)] = make_uint2(lo, hi);
      if ((t & 3) == 0) reinterpret_cast<uint8_t*>(sf_stage)[rr * 8 + ((t & 31) >> 2)] = (uint8_t)byte;
    } else if (full || (kin && row0 + s * 8 + rsub < M)) {
      typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
      __builtin_nontemporal_store((u32x2_nt){lo, hi}, reinterpret_cast<u32x2_nt*>(qp + s * 8 * K));
      if ((t & 3) == 0) sp[s * 8 * ng] = (uint8_t)byte;
    }
  }
  if (WIDE && full) {   // uniform: interior tiles leave as 16-byte pieces, 4 rows per instruction
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int p = it * 256 + t, rr = p >> 4, part = p & 15;
      const uint4 w = frag_tile[p];
      __builtin_nontemporal_store((nt_u32x4){w.x, w.y, w.z, w.w},
                                  reinterpret_cast<nt_u32x4*>(q + (row0 + rr) * K + bx * 256 + part * 16));
    }
    // each row's 8 scale bytes of this K range: one 8-byte store when the row offsets allow it
    if (t < 64) {
      const int64_t off = (row0 + t) * ng + bx * 8;
      const uint2 w = reinterpret_cast<const uint2*>(sf_stage)[t];
      if (((reinterpret_cast<uintptr_t>(sf) + off) & 7) == 0) {
        *reinterpret_cast<uint2*>(sf + off) = w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) sf[off + i] = (uint8_t)((i < 4 ? w.x : w.y) >> (8 * (i & 3)));
      }
    }
  }
  if constexpr (FRAG) {
    __syncthreads();
    // row tiles past ceil(M / 32) are not part of the buffers; padded rows inside the last one
    // were encoded from zeros (code 0, scale 0x00)
    const int64_t row_tiles = (M + 31) / 32, rt0 = by * 2;
    const int64_t ks_steps = K / 64, k_groups = K / 256;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int p = it * 256 + t;
      if (rt0 + (p >> 9) < row_tiles) {
        const uint4 v = frag_tile[p ^ (((p >> 5) & 15) << 1)];
        __builtin_nontemporal_store((nt_u32x4){v.x, v.y, v.z, v.w},
                                    reinterpret_cast<nt_u32x4*>(q + ((rt0 + (p >> 9)) * ks_steps + bx * 4) * 2048) + (p & 511));
      }
    }
    if (t < 32 && rt0 + (t >> 4) < row_tiles)
      reinterpret_cast<uint4*>(sf + ((rt0 + (t >> 4)) * k_groups + bx) * 256)[t & 15] = sf_stage[t];
  }
}

// =============================================================================================
// MXFP4 quantize (mm_fp4's MX operands)
// =============================================================================================
// As the NVFP4 kernel (128 rows x 256 K per workgroup, 8 elements per lane), with OCP MX scales:
// a 32-element group is a lane quad; scale byte = max(biased exponent of amax - 2, 0), i.e.
// Es + 127 with Es = clamp(floor(log2 amax) - 2, -127, 127) (0x00 for amax == 0); elements
// e2m1(x * 2^-Es) (exact scaling, nearest even, saturating at 6). The 8 scale columns of a
// workgroup are two 128x4 column groups, staged in LDS and stored as whole 512-byte tiles.
//
// FRAG: both outputs in the MFMA fragment layout instead (K % 256 == 0; the layout is described at
// bsp_mxfp4_quantize_frag). The workgroup's 128 rows x 256 K are 4 row tiles x 4 K steps, sixteen
// 1 KB fragments and four 256-byte scale groups: all staged in LDS and stored as four contiguous
// 4 KB runs and four 256-byte runs. A thread's 4 output bytes for row rr and block cb are 16-byte
// chunk p = (rr/32)*256 + cb*32 + rr%32 of the staging area (cb = 2 * K step + lane half), placed
// at chunk p ^ 2cb: the eight blocks of a row otherwise sit 512 bytes apart, all in one LDS bank.
template <bool HWCVT, bool VEC, bool FRAG = false, bool WIDE = false>
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const uint16_t* __restrict__ x,
                                                             int64_t M, int64_t K, int64_t ld,
                                                             uint8_t* __restrict__ packed,
                                                             uint8_t* __restrict__ sf, int64_t Kp) {
  __shared__ uint4 sf_tile[64];  // 1 KB = 2 scale tiles of 512 B (FRAG: 4 scale groups of 256 B)
  // FRAG: the workgroup's 16 KB of packed fragments; WIDE: its 128 rows x 128 packed bytes
  __shared__ uint4 frag_tile[FRAG || WIDE ? 1024 : 1];
  uint8_t* sfb = reinterpret_cast<uint8_t*>(sf_tile);
  const int t = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * 128;
  const int64_t kk = (int64_t)blockIdx.x * 256 + (t & 31) * 8;
  const int rsub = t >> 5;
  const bool kin = kk < K;  // K % 32 == 0: a quad is entirely in or out
  const bool full = row0 + 128 <= M && (int64_t)blockIdx.x * 256 + 256 <= K;
  const uint16_t* xp = x + (row0 + rsub) * ld + kk;
  const int64_t xstep = 8 * ld;
  uint4 v[16];
  if (full) {
#pragma unroll
    for (int s = 0; s < 16; ++s) v[s] = load8<VEC>(xp + s * xstep);
  } else {
#pragma unroll
    for (int s = 0; s < 16; ++s)
      v[s] = (kin && row0 + s * 8 + rsub < M) ? load8<VEC>(xp + s * xstep) : make_uint4(0u, 0u, 0u, 0u);
  }
  nan_to_num_segments(v);
  const int64_t half_k = K / 2;
  uint8_t* pp = packed + (row0 + rsub) * half_k + kk / 2;
  const int64_t pstep = 8 * half_k;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const float a = quad_max(mag_value(mag_bits8(v[s])));
    float f[8];
    unpack8(v[s], f);
    const uint32_t ef = __float_as_uint(a) >> 23;
    const uint32_t byte = ef > 2u ? ef - 2u : 0u;            // Es + 127
    const float inv = __uint_as_float((254u - byte) << 23);  // 2^-Es, exact
    uint32_t out = 0;
    if (HWCVT) {
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[0] * inv, f[1] * inv, 1.0f, 0);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[2] * inv, f[3] * inv, 1.0f, 1);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[4] * inv, f[5] * inv, 1.0f, 2);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[6] * inv, f[7] * inv, 1.0f, 3);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out |= e2m1_encode(f[i] * inv) << (4 * i);
    }
    const int rr = s * 8 + rsub;
    const int cb = (t & 31) >> 2;  // the lane quad's 32-element block inside the workgroup's 256 K
    if constexpr (FRAG) {
      const int p = (rr >> 5) * 256 + cb * 32 + (rr & 31);
      reinterpret_cast<uint32_t*>(frag_tile)[(p ^ (cb << 1)) * 4 + (t & 3)] = out;
      if ((t & 3) == 0) sfb[(rr >> 5) * 256 + ((cb & 1) * 32 + (rr & 31)) * 4 + (cb >> 1)] = (uint8_t)byte;
    } else {
      if (WIDE && full) reinterpret_cast<uint32_t*>(frag_tile)[rr * 32 + (t & 31)] = out;
      else if (full || (kin && row0 + rr < M)) store4_nt(pp + s * pstep, out);
      if ((t & 3) == 0)  // cb: scale column inside the 8-column tile
        sfb[(cb >> 2) * 512 + (rr & 31) * 16 + (rr >> 5) * 4 + (cb & 3)] = (uint8_t)byte;
    }
  }
  __syncthreads();
  if constexpr (FRAG) {
    // row tiles past ceil(M / 32) are not part of the buffers; padded rows inside the last one
    // were encoded from zeros (code 0, scale 0x00)
    const int64_t row_tiles = (M + 31) / 32, rt0 = (int64_t)blockIdx.y * 4;
    const int64_t ks_steps = K / 64, k_groups = K / 256;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int p = it * 256 + t;
      if (rt0 + it < row_tiles) {
        const uint4 v = frag_tile[p ^ (((p >> 5) & 7) << 1)];
        __builtin_nontemporal_store((nt_u32x4){v.x, v.y, v.z, v.w},
                                    reinterpret_cast<nt_u32x4*>(packed + ((rt0 + it) * ks_steps + blockIdx.x * 4) * 1024) + (p & 255));
      }
    }
    if (t < 64 && rt0 + (t >> 4) < row_tiles)
      reinterpret_cast<uint4*>(sf + ((rt0 + (t >> 4)) * k_groups + blockIdx.x) * 256)[t & 15] = sf_tile[t];
    return;
  }
  if (WIDE && full) {   // uniform: interior tiles leave as 16-byte pieces, 8 rows per instruction
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int p = it * 256 + t, rr = p >> 3, part = p & 7;
      const uint4 w = frag_tile[p];
      __builtin_nontemporal_store(
          (nt_u32x4){w.x, w.y, w.z, w.w},
          reinterpret_cast<nt_u32x4*>(packed + (row0 + rr) * half_k + (int64_t)blockIdx.x * 128 + part * 16));
    }
  }
  const int64_t groups = Kp / 4;
  const int64_t g0 = (int64_t)blockIdx.x * 2;
  const int64_t ng = groups - g0 < 2 ? groups - g0 : 2;
  if (t < ng * 32) {
    const int cg = t >> 5;
    const int64_t tile = (int64_t)blockIdx.y * groups + g0 + cg;
    reinterpret_cast<uint4*>(sf + tile * 512)[t & 31] = sf_tile[cg * 32 + (t & 31)];
  }
}

// =============================================================================================
// GELU (tanh form), bf16 in/out
// =============================================================================================
// Grid-stride over 8-value segments, GELU by the workgroup's LDS table (gelu_segments_tab).
__global__ __launch_bounds__(256) void gelu_kernel(const uint16_t* x, uint16_t* y, int64_t n) {
  __shared__ __attribute__((aligned(16))) uint16_t gtab[kGeluTabSize];
  gelu_table_load(gtab, threadIdx.x, 256);
  __syncthreads();
  const int64_t n8 = n / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint4 v[1] = {load16_nt(reinterpret_cast<const uint4*>(x) + i)}, w[1];
    gelu_segments_tab(v, w, gtab);
    __builtin_nontemporal_store((nt_u32x4){w[0].x, w[0].y, w[0].z, w[0].w}, reinterpret_cast<nt_u32x4*>(y) + i);
  }
  // tail (n % 8 elements)
  int64_t i = n8 * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = (uint16_t)f32_to_bf16_rne(gelu_tanh(__uint_as_float((uint32_t)x[i] << 16)));
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int hw_cvt_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("BSP_QUANT_SW_CVT");
    v = (e && e[0] == '1') ? 0 : BSP_DEFAULT_HW_CVT;
  }
  return v;
}

int launch_global_sf(const void* w, int64_t rows, int64_t K, int64_t ld, float* gsf, float* inv,
                     float* amax, hipStream_t s, bool four_over_six) {
  hipLaunchKernelGGL(amax_init_kernel, dim3(1), dim3(1), 0, s, amax);
  if (rows > 0 && K > 0) {
    const uint16_t* wp = static_cast<const uint16_t*>(w);
    const bool vec = (K % 8 == 0) && (ld % 8 == 0) && aligned16(w);
    if (vec && (ld == K || rows == 1)) {
      int64_t blocks = ceil_div(rows * (K / 8), 256 * 8);
      if (blocks > 1024) blocks = 1024;
      hipLaunchKernelGGL(amax_reduce_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, wp, rows,
                         K, K, amax);
    } else if (vec) {
      const int64_t blocks = rows < 4096 ? rows : 4096;
      hipLaunchKernelGGL(amax_reduce_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, wp, rows,
                         K, ld, amax);
    } else {
      int64_t blocks = ceil_div(rows * K, 256);
      if (blocks > 4096) blocks = 4096;
      hipLaunchKernelGGL(amax_reduce_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, wp, rows,
                         K, ld, amax);
    }
  }
  if (four_over_six)
    hipLaunchKernelGGL(gsf_finish_4over6_kernel, dim3(1), dim3(1), 0, s, amax, gsf, inv);
  else
    hipLaunchKernelGGL(gsf_finish_kernel, dim3(1), dim3(1), 0, s, amax, gsf, inv);
  return check_launch(four_over_six ? "bsp_nvfp4_global_sf_4over6" : "bsp_nvfp4_global_sf");
}

// wide: 16-byte stores of the packed tile (K % 32 == 0 and a 16-byte aligned packed matrix):
// 3.9 % faster for X[32760, 5120]. The GELU-fused kernel keeps the four-byte stores: with its 9 KB
// GELU table in LDS the 16 KB image measured 1 % slower. The software-encoder path (a test
// switch) keeps them too.
template <bool GELU>
static void launch_nvfp4_quantize_t(dim3 grid, const uint16_t* xp, int64_t M, int64_t K, int64_t ld,
                                    const float* gsf, uint8_t* packed, uint8_t* sf, int64_t Kp,
                                    int64_t rows8, bool hw, bool vec, bool wide, bool frag,
                                    hipStream_t s) {
  if (frag) {
    if (hw && vec)
      hipLaunchKernelGGL((nvfp4_quantize_kernel<true, true, GELU, false, true>), grid, dim3(256), 0, s, xp,
                         M, K, ld, gsf, packed, sf, Kp, rows8);
    else if (hw)
      hipLaunchKernelGGL((nvfp4_quantize_kernel<true, false, GELU, false, true>), grid, dim3(256), 0, s, xp,
                         M, K, ld, gsf, packed, sf, Kp, rows8);
    else if (vec)
      hipLaunchKernelGGL((nvfp4_quantize_kernel<false, true, GELU, false, true>), grid, dim3(256), 0, s, xp,
                         M, K, ld, gsf, packed, sf, Kp, rows8);
    else
      hipLaunchKernelGGL((nvfp4_quantize_kernel<false, false, GELU, false, true>), grid, dim3(256), 0, s,
                         xp, M, K, ld, gsf, packed, sf, Kp, rows8);
    return;
  }
  wide = wide && !GELU;
  if (hw && vec && wide)
    hipLaunchKernelGGL((nvfp4_quantize_kernel<true, true, GELU, true>), grid, dim3(256), 0, s, xp, M, K,
                       ld, gsf, packed, sf, Kp, rows8);
  else if (hw && wide)
    hipLaunchKernelGGL((nvfp4_quantize_kernel<true, false, GELU, true>), grid, dim3(256), 0, s, xp, M, K,
                       ld, gsf, packed, sf, Kp, rows8);
  else if (hw && vec)
    hipLaunchKernelGGL((nvfp4_quantize_kernel<true, true, GELU, false>), grid, dim3(256), 0, s, xp, M, K,
                       ld, gsf, packed, sf, Kp, rows8);
  else if (hw)
    hipLaunchKernelGGL((nvfp4_quantize_kernel<true, false, GELU, false>), grid, dim3(256), 0, s, xp, M, K,
                       ld, gsf, packed, sf, Kp, rows8);
  else if (vec)
    hipLaunchKernelGGL((nvfp4_quantize_kernel<false, true, GELU, false>), grid, dim3(256), 0, s, xp, M, K,
                       ld, gsf, packed, sf, Kp, rows8);
  else
    hipLaunchKernelGGL((nvfp4_quantize_kernel<false, false, GELU, false>), grid, dim3(256), 0, s, xp, M,
                       K, ld, gsf, packed, sf, Kp, rows8);
}

// layout8: scales in layout_8x4 (rows padded to 8) instead of 128x4; frag: packed values in the
// fragment layout (K % 64 == 0, scales in 128x4)
int launch_nvfp4_quantize(const void* x, int64_t M, int64_t K, int64_t ld, const float* gsf,
                          uint8_t* packed, uint8_t* sf, hipStream_t s, bool gelu, bool layout8,
                          bool frag) {
  const int64_t Mp = ceil_div(M, 128) * 128;
  const int64_t Kp = ceil_div(K / 16, 4) * 4;
  dim3 grid((unsigned)ceil_div(Kp, 16), (unsigned)(Mp / 128));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const bool vec = (ld % 8 == 0) && aligned16(x);
  const bool hw = hw_cvt_enabled();
  const int64_t rows8 = layout8 ? ceil_div(M, 8) * 8 : 0;
  const bool wide = K % 32 == 0 && aligned16(packed);
  if (gelu)
    launch_nvfp4_quantize_t<true>(grid, xp, M, K, ld, gsf, packed, sf, Kp, rows8, hw, vec, wide, frag, s);
  else
    launch_nvfp4_quantize_t<false>(grid, xp, M, K, ld, gsf, packed, sf, Kp, rows8, hw, vec, wide, frag, s);
  if (frag) return check_launch(gelu ? "bsp_nvfp4_quantize_gelu_frag" : "bsp_nvfp4_quantize_frag");
  return check_launch(gelu ? "bsp_nvfp4_quantize_gelu"
                           : (layout8 ? "bsp_nvfp4_quantize_8x4" : "bsp_nvfp4_quantize"));
}

}  // namespace bsp

using namespace bsp;

extern "C" int bsp_nvfp4_global_sf(const void* w, int64_t rows, int64_t K, int64_t ld, float* gsf,
                                   float* inv_gsf, float* amax, void* stream) {
  BSP_REQUIRE(gsf && inv_gsf && amax, BSP_EINVAL, "bsp_nvfp4_global_sf: null scalar pointer");
  BSP_REQUIRE(rows >= 0 && K >= 0, BSP_EINVAL, "bsp_nvfp4_global_sf: negative size");
  BSP_REQUIRE(rows * K == 0 || w, BSP_EINVAL, "bsp_nvfp4_global_sf: null weight pointer");
  BSP_REQUIRE(rows <= 1 || ld >= K, BSP_ESHAPE, "bsp_nvfp4_global_sf: ld (%lld) < K (%lld)",
              (long long)ld, (long long)K);
  if (int e = check_device()) return e;
  return launch_global_sf(w, rows, K, ld, gsf, inv_gsf, amax, (hipStream_t)stream, false);
}

template <int C>
static void launch_token_c(const uint16_t* xp, int64_t M, int64_t K, int64_t ld, uint8_t* packed,
                           uint8_t* sf, float* gsf_rows, int64_t Kp, bool vec, hipStream_t s) {
  const int64_t Mp = ceil_div(M, 128) * 128;
  dim3 grid((unsigned)(Mp / 4));
  const bool wide = K % 32 == 0 && aligned16(packed);   // 16-byte row stores (store_row_wide)
  if (vec && wide)
    hipLaunchKernelGGL((nvfp4_quantize_token_kernel<C, true, true>), grid, dim3(256), 0, s, xp, M, K,
                       ld, packed, sf, gsf_rows, Kp);
  else if (vec)
    hipLaunchKernelGGL((nvfp4_quantize_token_kernel<C, true, false>), grid, dim3(256), 0, s, xp, M, K,
                       ld, packed, sf, gsf_rows, Kp);
  else if (wide)
    hipLaunchKernelGGL((nvfp4_quantize_token_kernel<C, false, true>), grid, dim3(256), 0, s, xp, M, K,
                       ld, packed, sf, gsf_rows, Kp);
  else
    hipLaunchKernelGGL((nvfp4_quantize_token_kernel<C, false, false>), grid, dim3(256), 0, s, xp, M, K,
                       ld, packed, sf, gsf_rows, Kp);
}

int launch_nvfp4_quantize_per_token(const void* x, int64_t M, int64_t K, int64_t ld, uint8_t* packed,
                                    uint8_t* sf, float* gsf_rows, hipStream_t s) {
  const int64_t Kp = ceil_div(K / 16, 4) * 4;
  const int64_t kpad = Kp * 16;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const bool vec = (ld % 8 == 0) && aligned16(x);
  // smallest register segment that holds the padded row (one HBM pass), else 16384-element segments
  if (kpad <= 64 * 8 * 4)
    launch_token_c<4>(xp, M, K, ld, packed, sf, gsf_rows, Kp, vec, s);
  else if (kpad <= 64 * 8 * 8)
    launch_token_c<8>(xp, M, K, ld, packed, sf, gsf_rows, Kp, vec, s);
  else if (kpad <= 64 * 8 * 10)   // K <= 5120 (fewer registers, more rows in flight per CU)
    launch_token_c<10>(xp, M, K, ld, packed, sf, gsf_rows, Kp, vec, s);
  else if (kpad <= 64 * 8 * 16)
    launch_token_c<16>(xp, M, K, ld, packed, sf, gsf_rows, Kp, vec, s);
  else
    launch_token_c<32>(xp, M, K, ld, packed, sf, gsf_rows, Kp, vec, s);
  return check_launch("bsp_nvfp4_quantize_per_token");
}

template <int C, bool QUANT, bool WIDE>
static void launch_rmsnorm_g(dim3 grid, const uint16_t* xp, int64_t M, int64_t K, int64_t ld,
                             const uint16_t* wg, float eps, const float* gsf, uint16_t* out,
                             int64_t ldo, uint8_t* packed, uint8_t* sf, int64_t Kp, bool vec,
                             hipStream_t s) {
  if (vec && wg)
    hipLaunchKernelGGL((rmsnorm_token_kernel<C, true, QUANT, true, WIDE>), grid, dim3(256), 0, s, xp, M,
                       K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp);
  else if (vec)
    hipLaunchKernelGGL((rmsnorm_token_kernel<C, true, QUANT, false, WIDE>), grid, dim3(256), 0, s, xp, M,
                       K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp);
  else if (wg)
    hipLaunchKernelGGL((rmsnorm_token_kernel<C, false, QUANT, true, WIDE>), grid, dim3(256), 0, s, xp, M,
                       K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp);
  else
    hipLaunchKernelGGL((rmsnorm_token_kernel<C, false, QUANT, false, WIDE>), grid, dim3(256), 0, s, xp, M,
                       K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp);
}

template <int C, bool QUANT>
static void launch_rmsnorm_c(const uint16_t* xp, int64_t M, int64_t K, int64_t ld,
                             const uint16_t* wg, float eps, const float* gsf, uint16_t* out,
                             int64_t ldo, uint8_t* packed, uint8_t* sf, int64_t Kp, bool vec,
                             hipStream_t s) {
  dim3 grid((unsigned)(ceil_div(M, 128) * 128 / 4));  // one wave per row of whole 128-row tiles
  // the fused quantize stores 16-byte row pieces (store_row_wide) where the packed rows allow it
  if (QUANT && K % 32 == 0 && aligned16(packed))
    launch_rmsnorm_g<C, QUANT, true>(grid, xp, M, K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp, vec, s);
  else
    launch_rmsnorm_g<C, QUANT, false>(grid, xp, M, K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp, vec, s);
}

// QUANT: the fused NVFP4 quantize; else the standalone RMSNorm into out. The register segment is
// the smallest that holds the (padded) row, as for the per-token quantize.
template <bool QUANT>
static void launch_rmsnorm_t(const uint16_t* xp, int64_t M, int64_t K, int64_t ld, const uint16_t* wg,
                             float eps, const float* gsf, uint16_t* out, int64_t ldo,
                             uint8_t* packed, uint8_t* sf, int64_t Kp, bool vec, hipStream_t s) {
  const int64_t kpad = QUANT ? Kp * 16 : K;
  if (kpad <= 64 * 8 * 4)
    launch_rmsnorm_c<4, QUANT>(xp, M, K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp, vec, s);
  else if (kpad <= 64 * 8 * 8)
    launch_rmsnorm_c<8, QUANT>(xp, M, K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp, vec, s);
  else if (kpad <= 64 * 8 * 10)
    launch_rmsnorm_c<10, QUANT>(xp, M, K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp, vec, s);
  else if (kpad <= 64 * 8 * 16)
    launch_rmsnorm_c<16, QUANT>(xp, M, K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp, vec, s);
  else
    launch_rmsnorm_c<32, QUANT>(xp, M, K, ld, wg, eps, gsf, out, ldo, packed, sf, Kp, vec, s);
}

// quant: the fused NVFP4 quantize (gsf, packed, sf); else the standalone RMSNorm into out
static int rmsnorm_entry(const char* fn, bool quant, const void* x, int64_t M, int64_t K, int64_t ld,
                         const void* weight, float eps, const float* gsf, void* out, int64_t ldo,
                         uint8_t* packed, uint8_t* sf, void* stream) {
  BSP_REQUIRE(M >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld K=%lld", fn, (long long)M, (long long)K);
  BSP_REQUIRE(eps > 0.0f && eps <= FLT_MAX, BSP_EINVAL, "%s: eps must be positive and finite", fn);
  BSP_REQUIRE(K % 16 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 16", fn, (long long)K);
  BSP_REQUIRE(M <= 1 || ld >= K, BSP_ESHAPE, "%s: ld (%lld) < K (%lld)", fn, (long long)ld, (long long)K);
  BSP_REQUIRE(quant || M <= 1 || ldo >= K, BSP_ESHAPE, "%s: ldo (%lld) < K (%lld)", fn,
              (long long)ldo, (long long)K);
  if (M == 0) return BSP_OK;
  BSP_REQUIRE(x && (quant ? (gsf && packed && sf) : out != nullptr), BSP_EINVAL, "%s: null pointer", fn);
  BSP_REQUIRE(!quant || ((reinterpret_cast<uintptr_t>(packed) & 3u) == 0 &&
                         (reinterpret_cast<uintptr_t>(sf) & 15u) == 0),
              BSP_EINVAL, "%s: packed must be 4-byte and sf 16-byte aligned", fn);
  BSP_REQUIRE(ceil_div(M, 128) * 32 < (1ll << 31), BSP_ESHAPE, "%s: M too large", fn);
  if (int e = check_device()) return e;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* wg = static_cast<const uint16_t*>(weight);
  // 16-byte loads and stores need 16-byte aligned rows of x, of the gain and (standalone) of out
  const bool vec = (ld % 8 == 0) && aligned16(x) && (!wg || aligned16(wg)) &&
                   (quant || ((ldo % 8 == 0) && aligned16(out)));
  const int64_t Kp = ceil_div(K / 16, 4) * 4;
  if (quant)
    launch_rmsnorm_t<true>(xp, M, K, ld, wg, eps, gsf, nullptr, 0, packed, sf, Kp, vec,
                           (hipStream_t)stream);
  else
    launch_rmsnorm_t<false>(xp, M, K, ld, wg, eps, nullptr, static_cast<uint16_t*>(out), ldo,
                            nullptr, nullptr, Kp, vec, (hipStream_t)stream);
  return check_launch(fn);
}

extern "C" int bsp_rmsnorm_bf16(const void* x, int64_t M, int64_t K, int64_t ld,
                                const void* weight_bf16, float eps, void* out, int64_t ldo,
                                void* stream) {
  return rmsnorm_entry("bsp_rmsnorm_bf16", false, x, M, K, ld, weight_bf16, eps, nullptr, out, ldo,
                       nullptr, nullptr, stream);
}

extern "C" int bsp_nvfp4_quantize_rmsnorm(const void* x, int64_t M, int64_t K, int64_t ld,
                                          const void* weight_bf16, float eps, const float* gsf,
                                          uint8_t* packed, uint8_t* sf, void* stream) {
  return rmsnorm_entry("bsp_nvfp4_quantize_rmsnorm", true, x, M, K, ld, weight_bf16, eps, gsf,
                       nullptr, 0, packed, sf, stream);
}

static int nvfp4_quantize_entry(const char* fn, const void* x, int64_t M, int64_t K, int64_t ld,
                                const float* gsf, uint8_t* packed, uint8_t* sf, void* stream, bool gelu,
                                bool layout8 = false, bool frag = false) {
  BSP_REQUIRE(M >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld K=%lld", fn, (long long)M, (long long)K);
  BSP_REQUIRE(K % 16 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 16", fn, (long long)K);
  BSP_REQUIRE(!frag || K % 64 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 64", fn, (long long)K);
  BSP_REQUIRE(M <= 1 || ld >= K, BSP_ESHAPE, "%s: ld (%lld) < K (%lld)", fn, (long long)ld, (long long)K);
  if (M == 0) return BSP_OK;
  BSP_REQUIRE(x && gsf && packed && sf, BSP_EINVAL, "%s: null pointer", fn);
  // 128x4 scales leave as 16-byte stores, 8x4 scales as dword stores
  const uintptr_t sf_mask = layout8 ? 3u : 15u;
  BSP_REQUIRE((reinterpret_cast<uintptr_t>(packed) & 3u) == 0 && (reinterpret_cast<uintptr_t>(sf) & sf_mask) == 0,
              BSP_EINVAL, "%s: packed must be 4-byte and sf %d-byte aligned", fn, layout8 ? 4 : 16);
  BSP_REQUIRE(!frag || aligned16(packed), BSP_EINVAL, "%s: packed must be 16-byte aligned", fn);
  BSP_REQUIRE(ceil_div(M, 128) < 65536, BSP_ESHAPE, "%s: M too large", fn);
  if (int e = check_device()) return e;
  return launch_nvfp4_quantize(x, M, K, ld, gsf, packed, sf, (hipStream_t)stream, gelu, layout8, frag);
}

extern "C" int bsp_nvfp4_frag_bytes(int64_t rows, int64_t K, int64_t* packed_bytes) {
  BSP_REQUIRE(packed_bytes, BSP_EINVAL, "bsp_nvfp4_frag_bytes: null output pointer");
  BSP_REQUIRE(rows >= 0 && K >= 0, BSP_EINVAL, "bsp_nvfp4_frag_bytes: negative size");
  BSP_REQUIRE(K % 64 == 0, BSP_ESHAPE, "bsp_nvfp4_frag_bytes: K (%lld) must be a multiple of 64",
              (long long)K);
  *packed_bytes = ceil_div(rows, 32) * 32 * (K / 2);
  return BSP_OK;
}

extern "C" int bsp_nvfp4_quantize_frag(const void* x, int64_t M, int64_t K, int64_t ld, const float* gsf,
                                       uint8_t* packed, uint8_t* sf, void* stream) {
  return nvfp4_quantize_entry("bsp_nvfp4_quantize_frag", x, M, K, ld, gsf, packed, sf, stream, false,
                              false, true);
}

extern "C" int bsp_nvfp4_quantize_gelu_frag(const void* y, int64_t M, int64_t K, int64_t ld,
                                            const float* gsf, uint8_t* packed, uint8_t* sf,
                                            void* stream) {
  return nvfp4_quantize_entry("bsp_nvfp4_quantize_gelu_frag", y, M, K, ld, gsf, packed, sf, stream, true,
                              false, true);
}

extern "C" int bsp_nvfp4_quantize(const void* x, int64_t M, int64_t K, int64_t ld, const float* gsf,
                                  uint8_t* packed, uint8_t* sf, void* stream) {
  return nvfp4_quantize_entry("bsp_nvfp4_quantize", x, M, K, ld, gsf, packed, sf, stream, false);
}

extern "C" int bsp_nvfp4_quantize_per_token(const void* x, int64_t M, int64_t K, int64_t ld,
                                            uint8_t* packed, uint8_t* sf, float* gsf_rows,
                                            void* stream) {
  const char* fn = "bsp_nvfp4_quantize_per_token";
  BSP_REQUIRE(M >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld K=%lld", fn, (long long)M, (long long)K);
  BSP_REQUIRE(K % 16 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 16", fn, (long long)K);
  BSP_REQUIRE(M <= 1 || ld >= K, BSP_ESHAPE, "%s: ld (%lld) < K (%lld)", fn, (long long)ld, (long long)K);
  if (M == 0) return BSP_OK;
  BSP_REQUIRE(x && packed && sf && gsf_rows, BSP_EINVAL, "%s: null pointer", fn);
  BSP_REQUIRE((reinterpret_cast<uintptr_t>(packed) & 3u) == 0 && (reinterpret_cast<uintptr_t>(sf) & 15u) == 0,
              BSP_EINVAL, "%s: packed must be 4-byte and sf 16-byte aligned", fn);
  BSP_REQUIRE(ceil_div(M, 128) * 32 < (1ll << 31), BSP_ESHAPE, "%s: M too large", fn);
  if (int e = check_device()) return e;
  return launch_nvfp4_quantize_per_token(x, M, K, ld, packed, sf, gsf_rows, (hipStream_t)stream);
}

extern "C" int bsp_nvfp4_quantize_8x4(const void* x, int64_t M, int64_t K, int64_t ld, const float* gsf,
                                      uint8_t* packed, uint8_t* sf, void* stream) {
  return nvfp4_quantize_entry("bsp_nvfp4_quantize_8x4", x, M, K, ld, gsf, packed, sf, stream, false, true);
}

extern "C" int bsp_nvfp4_global_sf_4over6(const void* w, int64_t rows, int64_t K, int64_t ld,
                                          float* gsf, float* inv_gsf, float* amax, void* stream) {
  BSP_REQUIRE(gsf && inv_gsf && amax, BSP_EINVAL, "bsp_nvfp4_global_sf_4over6: null scalar pointer");
  BSP_REQUIRE(rows >= 0 && K >= 0, BSP_EINVAL, "bsp_nvfp4_global_sf_4over6: negative size");
  BSP_REQUIRE(rows * K == 0 || w, BSP_EINVAL, "bsp_nvfp4_global_sf_4over6: null weight pointer");
  BSP_REQUIRE(rows <= 1 || ld >= K, BSP_ESHAPE, "bsp_nvfp4_global_sf_4over6: ld (%lld) < K (%lld)",
              (long long)ld, (long long)K);
  if (int e = check_device()) return e;
  return launch_global_sf(w, rows, K, ld, gsf, inv_gsf, amax, (hipStream_t)stream, true);
}

extern "C" int bsp_nvfp4_quantize_gelu(const void* y, int64_t M, int64_t K, int64_t ld,
                                       const float* gsf, uint8_t* packed, uint8_t* sf, void* stream) {
  return nvfp4_quantize_entry("bsp_nvfp4_quantize_gelu", y, M, K, ld, gsf, packed, sf, stream, true);
}

extern "C" int bsp_nvfp4_prequantize_weight(const void* w, int64_t N, int64_t K, int64_t ld,
                                            uint8_t* packed, uint8_t* sf, float* gsf,
                                            float* inv_gsf, float* amax, void* stream) {
  BSP_REQUIRE(N > 0 && K > 0, BSP_EINVAL, "bsp_nvfp4_prequantize_weight: bad size");
  BSP_REQUIRE(K % 16 == 0, BSP_ESHAPE, "bsp_nvfp4_prequantize_weight: K (%lld) must be a multiple of 16",
              (long long)K);
  BSP_REQUIRE(w && packed && sf && gsf && inv_gsf && amax, BSP_EINVAL,
              "bsp_nvfp4_prequantize_weight: null pointer");
  // everything the quantize step checks, before the global-scale step launches anything
  BSP_REQUIRE(N <= 1 || ld >= K, BSP_ESHAPE, "bsp_nvfp4_prequantize_weight: ld (%lld) < K (%lld)",
              (long long)ld, (long long)K);
  BSP_REQUIRE((reinterpret_cast<uintptr_t>(packed) & 3u) == 0 && (reinterpret_cast<uintptr_t>(sf) & 15u) == 0,
              BSP_EINVAL, "bsp_nvfp4_prequantize_weight: packed must be 4-byte and sf 16-byte aligned");
  BSP_REQUIRE(ceil_div(N, 128) < 65536, BSP_ESHAPE, "bsp_nvfp4_prequantize_weight: N too large");
  int e = bsp_nvfp4_global_sf(w, N, K, ld, gsf, inv_gsf, amax, stream);
  if (e) return e;
  return bsp_nvfp4_quantize(w, N, K, ld, gsf, packed, sf, stream);
}

extern "C" int bsp_nvfp4_prequantize_weight_frag(const void* w, int64_t N, int64_t K, int64_t ld,
                                                 uint8_t* packed, uint8_t* sf, float* gsf,
                                                 float* inv_gsf, float* amax, void* stream) {
  const char* fn = "bsp_nvfp4_prequantize_weight_frag";
  BSP_REQUIRE(N > 0 && K > 0, BSP_EINVAL, "%s: bad size", fn);
  BSP_REQUIRE(K % 64 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 64", fn, (long long)K);
  BSP_REQUIRE(w && packed && sf && gsf && inv_gsf && amax, BSP_EINVAL, "%s: null pointer", fn);
  // everything the quantize step checks, before the global-scale step launches anything
  BSP_REQUIRE(N <= 1 || ld >= K, BSP_ESHAPE, "%s: ld (%lld) < K (%lld)", fn, (long long)ld, (long long)K);
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(sf)) & 15u) == 0,
              BSP_EINVAL, "%s: packed and sf must be 16-byte aligned", fn);
  BSP_REQUIRE(ceil_div(N, 128) < 65536, BSP_ESHAPE, "%s: N too large", fn);
  int e = bsp_nvfp4_global_sf(w, N, K, ld, gsf, inv_gsf, amax, stream);
  if (e) return e;
  return bsp_nvfp4_quantize_frag(w, N, K, ld, gsf, packed, sf, stream);
}

extern "C" int bsp_nvfp4_alpha(const float* xg, const float* wg, float* alpha, void* stream) {
  BSP_REQUIRE(xg && wg && alpha, BSP_EINVAL, "bsp_nvfp4_alpha: null pointer");
  if (int e = check_device()) return e;
  hipLaunchKernelGGL(alpha_kernel, dim3(1), dim3(1), 0, (hipStream_t)stream, xg, wg, alpha);
  return check_launch("bsp_nvfp4_alpha");
}

extern "C" int bsp_mxfp8_quantize(const void* x, int64_t M, int64_t K, int64_t ld, uint8_t* q,
                                  uint8_t* sf, void* stream) {
  BSP_REQUIRE(M >= 0 && K > 0, BSP_EINVAL, "bsp_mxfp8_quantize: bad size M=%lld K=%lld",
              (long long)M, (long long)K);
  BSP_REQUIRE(K % 32 == 0, BSP_ESHAPE, "bsp_mxfp8_quantize: K (%lld) must be a multiple of 32",
              (long long)K);
  BSP_REQUIRE(M <= 1 || ld >= K, BSP_ESHAPE, "bsp_mxfp8_quantize: ld (%lld) < K (%lld)",
              (long long)ld, (long long)K);
  if (M == 0) return BSP_OK;
  BSP_REQUIRE(x && q && sf, BSP_EINVAL, "bsp_mxfp8_quantize: null pointer");
  BSP_REQUIRE((reinterpret_cast<uintptr_t>(q) & 7u) == 0, BSP_EINVAL,
              "bsp_mxfp8_quantize: q must be 8-byte aligned");
  BSP_REQUIRE(ceil_div(M, 64) < 65536, BSP_ESHAPE, "bsp_mxfp8_quantize: M too large");
  if (int e = check_device()) return e;
  dim3 grid((unsigned)ceil_div(K, 256), (unsigned)ceil_div(M, 64));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const bool vec = (ld % 8 == 0) && aligned16(x);
  const bool hw = hw_cvt_enabled();
  hipStream_t s = (hipStream_t)stream;
  // interior tiles of a 16-byte aligned q leave through LDS as 16-byte pieces (rows start 16-byte
  // aligned: K % 32 == 0); the software-encoder path (a test switch) keeps the direct stores
  const bool wide = aligned16(q);
  if (hw && vec && wide)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<true, true, false, true>), grid, dim3(256), 0, s, xp, M, K,
                       ld, q, sf);
  else if (hw && wide)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<true, false, false, true>), grid, dim3(256), 0, s, xp, M, K,
                       ld, q, sf);
  else if (hw && vec)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<true, true>), grid, dim3(256), 0, s, xp, M, K, ld, q, sf);
  else if (hw)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<true, false>), grid, dim3(256), 0, s, xp, M, K, ld, q, sf);
  else if (vec)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<false, true>), grid, dim3(256), 0, s, xp, M, K, ld, q, sf);
  else
    hipLaunchKernelGGL((mxfp8_quantize_kernel<false, false>), grid, dim3(256), 0, s, xp, M, K, ld, q, sf);
  return check_launch("bsp_mxfp8_quantize");
}

extern "C" int bsp_mxfp8_frag_bytes(int64_t rows, int64_t K, int64_t* q_bytes, int64_t* sf_bytes) {
  BSP_REQUIRE(q_bytes && sf_bytes, BSP_EINVAL, "bsp_mxfp8_frag_bytes: null output pointer");
  BSP_REQUIRE(rows >= 0 && K >= 0, BSP_EINVAL, "bsp_mxfp8_frag_bytes: negative size");
  BSP_REQUIRE(K % 256 == 0, BSP_ESHAPE, "bsp_mxfp8_frag_bytes: K (%lld) must be a multiple of 256",
              (long long)K);
  *q_bytes = ceil_div(rows, 32) * 32 * K;
  *sf_bytes = ceil_div(rows, 32) * 32 * (K / 32);
  return BSP_OK;
}

extern "C" int bsp_mxfp8_quantize_frag(const void* x, int64_t M, int64_t K, int64_t ld, uint8_t* q,
                                       uint8_t* sf, void* stream) {
  const char* fn = "bsp_mxfp8_quantize_frag";
  BSP_REQUIRE(M >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld K=%lld", fn, (long long)M, (long long)K);
  BSP_REQUIRE(K % 256 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 256", fn, (long long)K);
  BSP_REQUIRE(M <= 1 || ld >= K, BSP_ESHAPE, "%s: ld (%lld) < K (%lld)", fn, (long long)ld, (long long)K);
  if (M == 0) return BSP_OK;
  BSP_REQUIRE(x && q && sf, BSP_EINVAL, "%s: null pointer", fn);
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(sf)) & 15u) == 0,
              BSP_EINVAL, "%s: q and sf must be 16-byte aligned", fn);
  BSP_REQUIRE(ceil_div(M, 64) < 65536, BSP_ESHAPE, "%s: M too large", fn);
  if (int e = check_device()) return e;
  dim3 grid((unsigned)(K / 256), (unsigned)ceil_div(M, 64));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const bool vec = (ld % 8 == 0) && aligned16(x);
  const bool hw = hw_cvt_enabled();
  hipStream_t s = (hipStream_t)stream;
  if (hw && vec)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<true, true, true>), grid, dim3(256), 0, s, xp, M, K, ld, q, sf);
  else if (hw)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<true, false, true>), grid, dim3(256), 0, s, xp, M, K, ld, q, sf);
  else if (vec)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<false, true, true>), grid, dim3(256), 0, s, xp, M, K, ld, q, sf);
  else
    hipLaunchKernelGGL((mxfp8_quantize_kernel<false, false, true>), grid, dim3(256), 0, s, xp, M, K, ld, q, sf);
  return check_launch(fn);
}

extern "C" int bsp_gelu_tanh_bf16(const void* x, void* y, int64_t n, void* stream) {
  BSP_REQUIRE(n >= 0, BSP_EINVAL, "bsp_gelu_tanh_bf16: negative size");
  if (n == 0) return BSP_OK;
  BSP_REQUIRE(x && y, BSP_EINVAL, "bsp_gelu_tanh_bf16: null pointer");
  BSP_REQUIRE(aligned16(x) && aligned16(y), BSP_EINVAL, "bsp_gelu_tanh_bf16: pointers must be 16-byte aligned");
  if (int e = check_device()) return e;
  int64_t blocks = ceil_div(n / 8 > 0 ? n / 8 : 1, 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gelu_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), n);
  return check_launch("bsp_gelu_tanh_bf16");
}

extern "C" int bsp_mxfp4_sf_bytes(int64_t rows, int64_t K, int64_t* bytes) {
  BSP_REQUIRE(bytes, BSP_EINVAL, "bsp_mxfp4_sf_bytes: null output pointer");
  BSP_REQUIRE(rows >= 0 && K >= 0, BSP_EINVAL, "bsp_mxfp4_sf_bytes: negative size");
  *bytes = ceil_div(rows, 128) * 128 * ceil_div(K, 128) * 4;
  return BSP_OK;
}

extern "C" int bsp_mxfp4_frag_bytes(int64_t rows, int64_t K, int64_t* packed_bytes, int64_t* sf_bytes) {
  BSP_REQUIRE(packed_bytes && sf_bytes, BSP_EINVAL, "bsp_mxfp4_frag_bytes: null output pointer");
  BSP_REQUIRE(rows >= 0 && K >= 0, BSP_EINVAL, "bsp_mxfp4_frag_bytes: negative size");
  BSP_REQUIRE(K % 256 == 0, BSP_ESHAPE, "bsp_mxfp4_frag_bytes: K (%lld) must be a multiple of 256",
              (long long)K);
  *packed_bytes = ceil_div(rows, 32) * 32 * (K / 2);
  *sf_bytes = ceil_div(rows, 32) * 32 * (K / 32);
  return BSP_OK;
}

extern "C" int bsp_mxfp4_quantize_frag(const void* x, int64_t M, int64_t K, int64_t ld, uint8_t* packed,
                                       uint8_t* sf, void* stream) {
  const char* fn = "bsp_mxfp4_quantize_frag";
  BSP_REQUIRE(M >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld K=%lld", fn, (long long)M, (long long)K);
  BSP_REQUIRE(K % 256 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 256", fn, (long long)K);
  BSP_REQUIRE(M <= 1 || ld >= K, BSP_ESHAPE, "%s: ld (%lld) < K (%lld)", fn, (long long)ld, (long long)K);
  if (M == 0) return BSP_OK;
  BSP_REQUIRE(x && packed && sf, BSP_EINVAL, "%s: null pointer", fn);
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(sf)) & 15u) == 0,
              BSP_EINVAL, "%s: packed and sf must be 16-byte aligned", fn);
  BSP_REQUIRE(ceil_div(M, 128) < 65536, BSP_ESHAPE, "%s: M too large", fn);
  if (int e = check_device()) return e;
  dim3 grid((unsigned)(K / 256), (unsigned)ceil_div(M, 128));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const bool vec = (ld % 8 == 0) && aligned16(x);
  const bool hw = hw_cvt_enabled();
  const int64_t Kp = K / 32;
  hipStream_t s = (hipStream_t)stream;
  if (hw && vec)
    hipLaunchKernelGGL((mxfp4_quantize_kernel<true, true, true>), grid, dim3(256), 0, s, xp, M, K, ld, packed, sf, Kp);
  else if (hw)
    hipLaunchKernelGGL((mxfp4_quantize_kernel<true, false, true>), grid, dim3(256), 0, s, xp, M, K, ld, packed, sf, Kp);
  else if (vec)
    hipLaunchKernelGGL((mxfp4_quantize_kernel<false, true, true>), grid, dim3(256), 0, s, xp, M, K, ld, packed, sf, Kp);
  else
    hipLaunchKernelGGL((mxfp4_quantize_kernel<false, false, true>), grid, dim3(256), 0, s, xp, M, K, ld, packed, sf, Kp);
  return check_launch(fn);
}

extern "C" int bsp_mxfp4_quantize(const void* x, int64_t M, int64_t K, int64_t ld, uint8_t* packed,
                                  uint8_t* sf, void* stream) {
  BSP_REQUIRE(M >= 0 && K > 0, BSP_EINVAL, "bsp_mxfp4_quantize: bad size M=%lld K=%lld",
              (long long)M, (long long)K);
  BSP_REQUIRE(K % 32 == 0, BSP_ESHAPE, "bsp_mxfp4_quantize: K (%lld) must be a multiple of 32",
              (long long)K);
  BSP_REQUIRE(M <= 1 || ld >= K, BSP_ESHAPE, "bsp_mxfp4_quantize: ld (%lld) < K (%lld)",
              (long long)ld, (long long)K);
  if (M == 0) return BSP_OK;
  BSP_REQUIRE(x && packed && sf, BSP_EINVAL, "bsp_mxfp4_quantize: null pointer");
  BSP_REQUIRE((reinterpret_cast<uintptr_t>(packed) & 3u) == 0 && (reinterpret_cast<uintptr_t>(sf) & 15u) == 0,
              BSP_EINVAL, "bsp_mxfp4_quantize: packed must be 4-byte and sf 16-byte aligned");
  BSP_REQUIRE(ceil_div(M, 128) < 65536, BSP_ESHAPE, "bsp_mxfp4_quantize: M too large");
  if (int e = check_device()) return e;
  const int64_t Mp = ceil_div(M, 128) * 128;
  const int64_t Kp = ceil_div(K / 32, 4) * 4;
  dim3 grid((unsigned)ceil_div(Kp, 8), (unsigned)(Mp / 128));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const bool vec = (ld % 8 == 0) && aligned16(x);
  const bool hw = hw_cvt_enabled();
  hipStream_t s = (hipStream_t)stream;
  // interior tiles of a 16-byte aligned packed matrix leave through LDS as 16-byte pieces (rows
  // start 16-byte aligned: K % 32 == 0); the software-encoder path (a test switch) stores directly
  const bool wide = aligned16(packed);
  if (hw && vec && wide)
    hipLaunchKernelGGL((mxfp4_quantize_kernel<true, true, false, true>), grid, dim3(256), 0, s, xp, M, K,
                       ld, packed, sf, Kp);
  else if (hw && wide)
    hipLaunchKernelGGL((mxfp4_quantize_kernel<true, false, false, true>), grid, dim3(256), 0, s, xp, M, K,
                       ld, packed, sf, Kp);
  else if (hw && vec)
    hipLaunchKernelGGL((mxfp4_quantize_kernel<true, true>), grid, dim3(256), 0, s, xp, M, K, ld, packed, sf, Kp);
  else if (hw)
    hipLaunchKernelGGL((mxfp4_quantize_kernel<true, false>), grid, dim3(256), 0, s, xp, M, K, ld, packed, sf, Kp);
  else if (vec)
    hipLaunchKernelGGL((mxfp4_quantize_kernel<false, true>), grid, dim3(256), 0, s, xp, M, K, ld, packed, sf, Kp);
  else
    hipLaunchKernelGGL((mxfp4_quantize_kernel<false, false>), grid, dim3(256), 0, s, xp, M, K, ld, packed, sf, Kp);
  return check_launch("bsp_mxfp4_quantize");
}
