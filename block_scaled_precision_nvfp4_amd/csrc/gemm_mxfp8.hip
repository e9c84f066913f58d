// a7 -- mm_mxfp8 on gfx950: C = A . B^T over MXFP8 operands (e4m3 values, one e8m0 scale per 32
// K elements, per row of each operand), fp32 accumulation, bf16 or fp32 output.
// vLLM-Omni mxfp8_config.py (DiffusionMXFP8Config; NPUMxfp8LinearMethod._quant_matmul).
//
// The OCP MX block scale is exactly what gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 consumes: one
// e8m0 scale per row and 32-element K block, supplied by the lane half that owns the block (lane
// i + 32*b for block b of row i), so the format maps 1:1 onto the instruction (operand format
// e4m3 for both sides, cbsz = blgp = 0). With 8-bit operands each lane holds 16 elements of each
// of the two blocks (see frag()); this placement was measured on the hardware with one-hot
// operands and distinct per-lane scales.
//
// Tiling: a 256-thread workgroup owns a 256x256 C tile, each wave a 128x128 quarter (4x4 MFMA
// 32x32 tiles). K advances 64 per stage: LDS holds 256 rows x 64 bytes of A and of B (four
// 16-byte chunks per row, XOR-swizzled by row) plus the two e8m0 bytes per row of each operand,
// double-buffered with register prefetch. The MFMA's A operand is the weight fragment, its B
// operand the activation fragment (same epilogue shape as mm_fp4).
#include "common.hpp"

namespace bsp {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace mx8 {

constexpr int BM = 256, BN = 256, BK = 64;

struct Stage {
  u32x4 a[BM * 4];
  u32x4 b[BN * 4];
  uint16_t sa[BM];
  uint16_t sb[BN];
};

__device__ __forceinline__ int chunk_slot(int row, int c) { return row * 4 + (c ^ ((row >> 1) & 3)); }

struct Prefetch {
  u32x4 a[4], b[4];
  uint16_t sa, sb;
};

__device__ __forceinline__ void load_stage(Prefetch& pf, const uint8_t* __restrict__ A,
                                           const uint8_t* __restrict__ B,
                                           const uint8_t* __restrict__ SA,
                                           const uint8_t* __restrict__ SB, int64_t M, int64_t N,
                                           int64_t K, int64_t m0, int64_t n0, int64_t kt, int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + 256 * i;
    const int row = c >> 2, part = c & 3;
    int64_t ga = m0 + row; ga = ga < M ? ga : M - 1;
    int64_t gb = n0 + row; gb = gb < N ? gb : N - 1;
    pf.a[i] = *reinterpret_cast<const u32x4*>(A + ga * K + kt * 64 + part * 16);
    pf.b[i] = *reinterpret_cast<const u32x4*>(B + gb * K + kt * 64 + part * 16);
  }
  const int64_t ng = K / 32;
  int64_t ga = m0 + t; ga = ga < M ? ga : M - 1;
  int64_t gb = n0 + t; gb = gb < N ? gb : N - 1;
  pf.sa = *reinterpret_cast<const uint16_t*>(SA + ga * ng + kt * 2);
  pf.sb = *reinterpret_cast<const uint16_t*>(SB + gb * ng + kt * 2);
}

__device__ __forceinline__ void store_stage(Stage& st, const Prefetch& pf, int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + 256 * i;
    const int row = c >> 2, part = c & 3;
    st.a[chunk_slot(row, part)] = pf.a[i];
    st.b[chunk_slot(row, part)] = pf.b[i];
  }
  st.sa[t] = pf.sa;
  st.sb[t] = pf.sb;
}

// Operand fragment of lane half h for v_mfma_scale_f32_32x32x64_f8f6f4 with 8-bit elements: the
// instruction takes bytes 0-15 of every lane as K elements of the first 32-element scale block and
// bytes 16-31 as elements of the second, lane half h supplying the 16-element half h of each block
// (and lane half h's scale applying to block h). So lane half h carries the 16-byte chunks h and
// 2 + h of the 64-byte K step.
__device__ __forceinline__ i32x8 frag(const u32x4* rows, int row, int h) {
  u32x4 lo = rows[chunk_slot(row, h)];
  u32x4 hi = rows[chunk_slot(row, 2 + h)];
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void mm_mxfp8_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, void* __restrict__ out,
    int64_t ldc, int ntn, bool vec_store) {
  __shared__ Stage st[2];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;
  const int bid = blockIdx.x;
  const int64_t m0 = (int64_t)(bid / ntn) * BM;
  const int64_t n0 = (int64_t)(bid % ntn) * BN;
  const int64_t nk = K / BK;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  Prefetch pf;
  load_stage(pf, A, B, SA, SB, M, N, K, m0, n0, 0, t);
  store_stage(st[0], pf, t);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) load_stage(pf, A, B, SA, SB, M, N, K, m0, n0, kt + 1, t);
    const Stage& s = st[cur];
    i32x8 xa[4], xb[4];
    int sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + i * 32 + li;
      const int rb = wn * 128 + i * 32 + li;
      xa[i] = frag(s.a, ra, h);
      xb[i] = frag(s.b, rb, h);
      sa[i] = (s.sa[ra] >> (8 * h)) & 0xFF;
      sb[i] = (s.sb[rb] >> (8 * h)) & 0xFF;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[n][m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xb[n], xa[m], acc[n][m], 0, 0, 0,
                                                                    sb[n], 0, sa[m]);
    if (kt + 1 < nk) store_stage(st[cur ^ 1], pf, t);
    __syncthreads();
  }

#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t gm = m0 + wm * 128 + m * 32 + li;
    if (gm >= M) continue;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t gn = n0 + wn * 128 + n * 32 + 8 * b + 4 * h;
        float v0 = acc[n][m][4 * b + 0], v1 = acc[n][m][4 * b + 1];
        float v2 = acc[n][m][4 * b + 2], v3 = acc[n][m][4 * b + 3];
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

}  // namespace mx8

}  // namespace bsp

using namespace bsp;

extern "C" int bsp_mm_mxfp8(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                            const uint8_t* b_sf, int64_t M, int64_t N, int64_t K, void* out,
                            int64_t ldc, int out_dtype, void* stream) {
  BSP_REQUIRE(M >= 0 && N >= 0 && K > 0, BSP_EINVAL, "bsp_mm_mxfp8: bad size M=%lld N=%lld K=%lld",
              (long long)M, (long long)N, (long long)K);
  BSP_REQUIRE(out_dtype == BSP_OUT_BF16 || out_dtype == BSP_OUT_F32, BSP_EDTYPE,
              "bsp_mm_mxfp8: out_dtype must be BSP_OUT_BF16 (0) or BSP_OUT_F32 (1), got %d", out_dtype);
  BSP_REQUIRE(K % 128 == 0, BSP_ESHAPE, "bsp_mm_mxfp8: K (%lld) must be a multiple of 128", (long long)K);
  BSP_REQUIRE(M <= 1 || ldc >= N, BSP_ESHAPE, "bsp_mm_mxfp8: ldc (%lld) < N (%lld)", (long long)ldc,
              (long long)N);
  if (M == 0 || N == 0) return BSP_OK;
  BSP_REQUIRE(a && a_sf && b && b_sf && out, BSP_EINVAL, "bsp_mm_mxfp8: null pointer");
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) == 0 &&
                  ((reinterpret_cast<uintptr_t>(a_sf) | reinterpret_cast<uintptr_t>(b_sf)) & 1u) == 0,
              BSP_EINVAL, "bsp_mm_mxfp8: operands must be 16-byte and scales 2-byte aligned");
  BSP_REQUIRE(ceil_div(M, 256) * ceil_div(N, 256) < (1ll << 31), BSP_ESHAPE, "bsp_mm_mxfp8: too many tiles");
  if (int e = check_device()) return e;
  const int64_t ntn = ceil_div(N, mx8::BN);
  const int64_t tiles = ceil_div(M, mx8::BM) * ntn;
  const size_t esz = out_dtype == BSP_OUT_F32 ? 4 : 2;
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & (4 * esz - 1)) == 0);
  hipStream_t s = (hipStream_t)stream;
  if (out_dtype == BSP_OUT_F32)
    hipLaunchKernelGGL(mx8::mm_mxfp8_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, s, a, a_sf, b,
                       b_sf, M, N, K, out, ldc, (int)ntn, vec);
  else
    hipLaunchKernelGGL(mx8::mm_mxfp8_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, s, a, a_sf, b,
                       b_sf, M, N, K, out, ldc, (int)ntn, vec);
  return check_launch("bsp_mm_mxfp8");
}
