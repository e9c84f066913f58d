// a4 -- mm_fp4 on gfx950: C = alpha * A . B^T over NVFP4 operands (e2m1 values, one e4m3 scale
// per 16 K elements in the 128x4 layout), fp32 accumulation, bf16 or fp32 output.
// FastVideo nvfp4_config.py (_mm_fp4, module docstring) and nvfp4_qat_config.py (apply).
//
// Mapping onto CDNA4. gfx950's block-scaled MFMA applies one power-of-two (e8m0) scale per 32
// K elements, while NVFP4 carries a non-power-of-two e4m3 scale per 16; an e2m1 value times an
// e4m3 scale needs up to 6 significant bits, so no 4/6/8-bit MFMA operand can hold it exactly.
// Every such product is exact in fp16, so the packed FP4 bytes and the scale bytes are staged in
// LDS as they are (0.5 byte per element), and each wave dequantizes its own fragments in
// registers (v_cvt_scalef32_pk_f16_fp4 then a packed f16 multiply by the decoded scale) right
// before v_mfma_f32_32x32x16_f16.
//
// Tiling: a 256-thread workgroup owns a 256x256 C tile; each of its 4 waves a 128x128 quarter as
// 4x4 MFMA 32x32 tiles (256 fp32 accumulators per lane). K advances 64 per stage; one stage of
// LDS holds 256 rows x 32 bytes of packed A and of B plus the two 512-byte 128x4 scale tiles of
// each operand, double-buffered with register prefetch of the next stage. In the 128x4 layout the
// four scales of a row for a 64-K step are one dword, so the scale tiles are copied verbatim.
// The MFMA's A operand is the weight fragment and its B operand the activation fragment, so a
// lane's accumulators hold four consecutive output columns of one output row per group and the
// epilogue stores 4 bf16 (8 bytes) per lane per group.
#include "common.hpp"

namespace bsp {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace fp4 {

constexpr int BM = 256, BN = 256, BK = 64;

struct Stage {
  u32x4 a[BM * 2];  // packed A: row r holds its 32 bytes as two 16-byte halves (swizzled)
  u32x4 b[BN * 2];  // packed B (weights), same
  u32x4 sa[64];     // 2 scale tiles x 512 B (rows 0-127, 128-255 of the tile) for this K step
  u32x4 sb[64];
};

__device__ __forceinline__ int half_slot(int row, int h) { return row * 2 + (h ^ ((row >> 2) & 1)); }

// scale word (4 e4m3 bytes for the 64-K step) of tile-local row r from a staged pair of 128x4 tiles
__device__ __forceinline__ uint32_t scale_word(const u32x4* tiles, int r) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(tiles);
  return w[(r >> 7) * 128 + (r & 31) * 4 + ((r >> 5) & 3)];
}

// 8 e2m1 values (one dword) times their e4m3 scale -> 8 fp16 (exact)
__device__ __forceinline__ f16x8 dequant8(uint32_t w, uint32_t sbyte) {
  const float s = e4m3_decode_pos(sbyte);
#if BSP_CVT_FULL_SCALE
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 0);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 1);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 2);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 3);
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#else
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  const _Float16 hs = (_Float16)s;  // e4m3 values are exact in fp16
  f16x2 s2 = {hs, hs};
  p0 *= s2; p1 *= s2; p2 *= s2; p3 *= s2;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#endif
}

__device__ __forceinline__ uint32_t comp(const u32x4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Next stage's global data held in registers while the current stage computes. Named fields
// (no arrays) so that the whole struct is promoted to registers.
struct Prefetch {
  u32x4 a0, a1, b0, b1, s;  // s: one scale chunk (threads 0-63: A, 64-127: B)
};

__device__ __forceinline__ void load_stage(Prefetch& pf, const uint8_t* __restrict__ A,
                                           const uint8_t* __restrict__ B,
                                           const uint8_t* __restrict__ SA,
                                           const uint8_t* __restrict__ SB, int64_t M, int64_t N,
                                           int64_t K, int64_t m0, int64_t n0, int64_t kt,
                                           int64_t mtiles128, int64_t ntiles128, int64_t groups,
                                           int t) {
  const int64_t hk = K / 2;
  // chunk c = t (+256): row c / 2, 16-byte half c % 2 of the row's 32 bytes for this K step
  const int row = t >> 1, h = t & 1;
  int64_t ga0 = m0 + row; ga0 = ga0 < M ? ga0 : M - 1;
  int64_t ga1 = m0 + row + 128; ga1 = ga1 < M ? ga1 : M - 1;
  int64_t gb0 = n0 + row; gb0 = gb0 < N ? gb0 : N - 1;
  int64_t gb1 = n0 + row + 128; gb1 = gb1 < N ? gb1 : N - 1;
  const int64_t koff = kt * 32 + h * 16;
  pf.a0 = *reinterpret_cast<const u32x4*>(A + ga0 * hk + koff);
  pf.a1 = *reinterpret_cast<const u32x4*>(A + ga1 * hk + koff);
  pf.b0 = *reinterpret_cast<const u32x4*>(B + gb0 * hk + koff);
  pf.b1 = *reinterpret_cast<const u32x4*>(B + gb1 * hk + koff);
  // threads 0-63 fetch A's two scale tiles, 64-127 B's; threads 128-255 repeat the same
  // addresses (an unconditional load keeps the prefetch in registers) and never store them
  const int which = (t >> 6) & 1, tt = (t >> 5) & 1, q = t & 31;
  const int64_t r0 = which ? n0 / 128 : m0 / 128;
  const int64_t nt = which ? ntiles128 : mtiles128;
  int64_t rt = r0 + tt; rt = rt < nt ? rt : nt - 1;
  pf.s = *reinterpret_cast<const u32x4*>((which ? SB : SA) + (rt * groups + kt) * 512 + q * 16);
}

__device__ __forceinline__ void store_stage(Stage& st, const Prefetch& pf, int t) {
  const int row = t >> 1, h = t & 1;
  st.a[half_slot(row, h)] = pf.a0;
  st.a[half_slot(row + 128, h)] = pf.a1;
  st.b[half_slot(row, h)] = pf.b0;
  st.b[half_slot(row + 128, h)] = pf.b1;
  if (t < 64)
    st.sa[t] = pf.s;
  else if (t < 128)
    st.sb[t - 64] = pf.s;
}

template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void mm_fp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ alpha_ptr, int64_t M, int64_t N,
    int64_t K, void* __restrict__ out, int64_t ldc, int ntn, bool vec_store) {
  __shared__ Stage st[2];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  const int bid = blockIdx.x;
  const int64_t m0 = (int64_t)(bid / ntn) * BM;
  const int64_t n0 = (int64_t)(bid % ntn) * BN;
  const int64_t nk = K / BK;
  const int64_t groups = nk;  // 128x4 column groups = K/64
  const int64_t mtiles128 = (M + 127) / 128, ntiles128 = (N + 127) / 128;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  Prefetch pf;
  load_stage(pf, A, B, SA, SB, M, N, K, m0, n0, 0, mtiles128, ntiles128, groups, t);
  store_stage(st[0], pf, t);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) load_stage(pf, A, B, SA, SB, M, N, K, m0, n0, kt + 1, mtiles128, ntiles128, groups, t);

    const Stage& s = st[cur];
    u32x4 pa[4], pb[4];
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + i * 32 + li;
      const int rb = wn * 128 + i * 32 + li;
      pa[i] = s.a[half_slot(ra, h)];
      pb[i] = s.b[half_slot(rb, h)];
      wa[i] = scale_word(s.sa, ra);
      wb[i] = scale_word(s.sb, rb);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_barrier(0);  // keep each K sub-step's dequant next to its MFMAs
      const int sh = 8 * (2 * h + (j >> 1));  // scale byte of this lane's 8 elements
      f16x8 xa[4], xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xa[i] = dequant8(comp(pa[i], j), (wa[i] >> sh) & 0xFFu);
        xb[i] = dequant8(comp(pb[i], j), (wb[i] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[n][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xb[n], xa[m], acc[n][m], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(st[cur ^ 1], pf, t);
    __syncthreads();
  }

  // epilogue: D[n][m] per 32x32 tile; lane holds column m = li and rows n = 8*(r/4) + 4*h + r%4
  const float alpha = *alpha_ptr;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t gm = m0 + wm * 128 + m * 32 + li;
    if (gm >= M) continue;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t gn = n0 + wn * 128 + n * 32 + 8 * b + 4 * h;
        float v0 = alpha * acc[n][m][4 * b + 0];
        float v1 = alpha * acc[n][m][4 * b + 1];
        float v2 = alpha * acc[n][m][4 * b + 2];
        float v3 = alpha * acc[n][m][4 * b + 3];
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
          uint32_t b0 = f32_to_bf16_rne(v0), b1 = f32_to_bf16_rne(v1);
          uint32_t b2 = f32_to_bf16_rne(v2), b3 = f32_to_bf16_rne(v3);
          if (vec_store && gn + 3 < N) {
            *reinterpret_cast<uint2*>(o) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
          } else {
            if (gn + 0 < N) o[0] = (uint16_t)b0;
            if (gn + 1 < N) o[1] = (uint16_t)b1;
            if (gn + 2 < N) o[2] = (uint16_t)b2;
            if (gn + 3 < N) o[3] = (uint16_t)b3;
          }
        }
      }
    }
  }
}

}  // namespace fp4

int launch_mm_fp4(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                  const float* alpha, int64_t M, int64_t N, int64_t K, void* out, int64_t ldc,
                  int out_dtype, hipStream_t s) {
  const int64_t ntm = ceil_div(M, fp4::BM), ntn = ceil_div(N, fp4::BN);
  const int64_t tiles = ntm * ntn;
  const size_t esz = out_dtype == BSP_OUT_F32 ? 4 : 2;
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & (4 * esz - 1)) == 0);
  if (out_dtype == BSP_OUT_F32)
    hipLaunchKernelGGL(fp4::mm_fp4_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, s, a, sa, b, sb,
                       alpha, M, N, K, out, ldc, (int)ntn, vec);
  else
    hipLaunchKernelGGL(fp4::mm_fp4_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, s, a, sa, b, sb,
                       alpha, M, N, K, out, ldc, (int)ntn, vec);
  return check_launch("bsp_mm_fp4");
}

}  // namespace bsp

using namespace bsp;

extern "C" int bsp_mm_fp4(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                          const uint8_t* b_sf, const float* alpha_dev, int64_t M, int64_t N,
                          int64_t K, void* out, int64_t ldc, int out_dtype, void* stream) {
  BSP_REQUIRE(M >= 0 && N >= 0 && K > 0, BSP_EINVAL, "bsp_mm_fp4: bad size M=%lld N=%lld K=%lld",
              (long long)M, (long long)N, (long long)K);
  BSP_REQUIRE(out_dtype == BSP_OUT_BF16 || out_dtype == BSP_OUT_F32, BSP_EDTYPE,
              "bsp_mm_fp4: out_dtype must be BSP_OUT_BF16 (0) or BSP_OUT_F32 (1), got %d", out_dtype);
  BSP_REQUIRE(K % 64 == 0, BSP_ESHAPE, "bsp_mm_fp4: K (%lld) must be a multiple of 64", (long long)K);
  BSP_REQUIRE(M <= 1 || ldc >= N, BSP_ESHAPE, "bsp_mm_fp4: ldc (%lld) < N (%lld)", (long long)ldc,
              (long long)N);
  if (M == 0 || N == 0) return BSP_OK;
  BSP_REQUIRE(a_packed && a_sf && b_packed && b_sf && alpha_dev && out, BSP_EINVAL,
              "bsp_mm_fp4: null pointer");
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(a_packed) | reinterpret_cast<uintptr_t>(b_packed) |
                reinterpret_cast<uintptr_t>(a_sf) | reinterpret_cast<uintptr_t>(b_sf)) & 15u) == 0,
              BSP_EINVAL, "bsp_mm_fp4: operand and scale buffers must be 16-byte aligned");
  BSP_REQUIRE(ceil_div(M, 256) * ceil_div(N, 256) < (1ll << 31), BSP_ESHAPE, "bsp_mm_fp4: too many tiles");
  if (int e = check_device()) return e;
  return launch_mm_fp4(a_packed, a_sf, b_packed, b_sf, alpha_dev, M, N, K, out, ldc, out_dtype,
                       (hipStream_t)stream);
}
