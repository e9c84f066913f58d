// The MXFP4 GEMM on operands stored in the MFMA fragment layout: C = alpha * A . B^T (+ bias) with
// e2m1 elements and one e8m0 scale per 32 K elements per row (OCP MX), fp32 accumulation, bf16 or
// fp32 output. FastVideo nvfp4_config.py (_mm_fp4 with use_nvfp4=False; "MX-FP4" in the module
// docstring). Its quantize op carries a do_shuffle switch for operands pre-arranged for the matrix
// unit (always off there, the arrangement left to the library); the fragment layout is that
// arrangement for gfx950. Same products and the same K order as bsp_mm_mxfp4: the outputs are
// bit-identical for the same operand values.
//
// Fragment layout of an MXFP4 operand [R, K] (K % 256 == 0), rows in tiles of 32, K in steps of 64:
//  packed: the 1 KB fragment of row tile rt and K step ks at (rt * K/64 + ks) * 1024; lane
//          l = i + 32 h of it holds, in 16 bytes, row 32 rt + i, elements 64 ks + 32 h .. + 31
//          (even k in the low nibble) -- exactly what lane l of v_mfma_scale_f32_32x32x64_f8f6f4
//          reads for that row and K step;
//  scales: the 256 bytes of row tile rt and K-step group kg (four K steps) at
//          (rt * K/256 + kg) * 256; the dword of lane l = i + 32 h holds the e8m0 scale of row
//          32 rt + i, block 2 (4 kg + j) + h in byte j -- the MFMA's per-lane scale, byte j
//          selected by op_sel for K step 4 kg + j.
// Rows past R (to the next multiple of 32) are zero.
//
// Every wave loads the fragments of its four A and four B row tiles straight into registers, each
// a fully coalesced 1 KB read, three K steps ahead into a ring of four register buffers; no LDS and
// no workgroup barrier in the K loop (the two waves that share a row tile read it from the caches
// independently). Against the LDS-staged kernel this drops the LDS writes and reads and the
// per-stage barriers, at twice the L2 reads. Tiling and epilogue as the LDS-staged MX kernel:
// 256x256 C tile per 256-thread workgroup, 128x128 per wave, XCD-aware tile order, whole tiles
// leave through LDS as whole rows.
#include "gemm_common.hpp"

namespace bsp {
namespace mxf {

constexpr int BM = 256, BN = 256;

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

__device__ __forceinline__ i32x8 fp4_op(const u32x4& x) {
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};  // e2m1: four registers are read
}

// One K step (J = ks % 4) of a wave: its 16 MFMAs on ring buffer J, the loads of step kl (three
// ahead) into buffer (J + 3) % 4, whose step was consumed by the previous call, spread between them.
template <int J>
__device__ __forceinline__ void frag_step(f32x16 (&acc)[4][4], u32x4 (&xa)[4][4], u32x4 (&xb)[4][4],
                                          const uint32_t (&csa)[4], const uint32_t (&csb)[4],
                                          const uint8_t* const (&fa)[4], const uint8_t* const (&fb)[4],
                                          int64_t kl, uint32_t loff) {
  constexpr int NB = (J + 3) & 3;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int n = q >> 1, m = 2 * (q & 1);
    acc[n][m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        fp4_op(xb[J][n]), fp4_op(xa[J][m]), acc[n][m], 4, 4, J, (int)csb[n], J, (int)csa[m]);
    acc[n][m + 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        fp4_op(xb[J][n]), fp4_op(xa[J][m + 1]), acc[n][m + 1], 4, 4, J, (int)csb[n], J, (int)csa[m + 1]);
    if (q < 4) {
      xa[NB][q] = ld16(fa[q] + kl * 1024 + loff);
      xb[NB][q] = ld16(fb[q] + kl * 1024 + loff);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads of this step here, three steps before use
}

template <bool OUT_F32, int BIAS>
__global__ __launch_bounds__(256, 1) void mm_mxfp4_frag_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ alpha_ptr, int64_t M, int64_t N,
    int64_t K, void* __restrict__ out, int64_t ldc, int ntm, int ntn, bool vec_store,
    const void* __restrict__ bias) {
  __shared__ __attribute__((aligned(16))) uint8_t epi[4 * kEpiWaveBytes];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;
  int tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t KS = K >> 6, KG = KS >> 2;
  const int64_t ra_last = ((M + 31) >> 5) - 1, rb_last = ((N + 31) >> 5) - 1;

  // wave-uniform bases of the wave's four A and four B row tiles (rows past the operand clamp to
  // its last tile: read, never stored)
  const uint8_t* fa[4];
  const uint8_t* fb[4];
  const uint8_t* qa[4];
  const uint8_t* qb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t ra = (m0 >> 5) + wm * 4 + i;
    ra = ra < ra_last ? ra : ra_last;
    int64_t rb = (n0 >> 5) + wn * 4 + i;
    rb = rb < rb_last ? rb : rb_last;
    fa[i] = A + ra * KS * 1024;
    fb[i] = B + rb * KS * 1024;
    qa[i] = SA + ra * KG * 256;
    qb[i] = SB + rb * KG * 256;
  }
  const uint32_t loff = lane * 16, soff = lane * 4;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  u32x4 xa[4][4], xb[4][4];          // [ring buffer][row tile]
  uint32_t csa[4], csb[4], nsa[4], nsb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    csa[i] = ld4(qa[i] + soff);
    csb[i] = ld4(qb[i] + soff);
  }
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int64_t ks = b < KS ? b : KS - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xa[b][i] = ld16(fa[i] + ks * 1024 + loff);
      xb[b][i] = ld16(fb[i] + ks * 1024 + loff);
    }
  }

  for (int64_t kg = 0; kg < KG; ++kg) {
    {  // the next group's scale dwords (the last group reloads itself)
      const int64_t kn = kg + 1 < KG ? kg + 1 : KG - 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nsa[i] = ld4(qa[i] + kn * 256 + soff);
        nsb[i] = ld4(qb[i] + kn * 256 + soff);
      }
    }
    const int64_t ks = kg * 4;   // loads run three steps ahead; past the end the last step reloads
    frag_step<0>(acc, xa, xb, csa, csb, fa, fb, ks + 3 < KS ? ks + 3 : KS - 1, loff);
    frag_step<1>(acc, xa, xb, csa, csb, fa, fb, ks + 4 < KS ? ks + 4 : KS - 1, loff);
    frag_step<2>(acc, xa, xb, csa, csb, fa, fb, ks + 5 < KS ? ks + 5 : KS - 1, loff);
    frag_step<3>(acc, xa, xb, csa, csb, fa, fb, ks + 6 < KS ? ks + 6 : KS - 1, loff);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      csa[i] = nsa[i];
      csb[i] = nsb[i];
    }
  }

  const float a = alpha_ptr ? *alpha_ptr : 1.0f;
  const float alpha[4] = {a, a, a, a};
  store_tile<OUT_F32, BIAS, false>(acc, alpha, m0, n0, wm, wn, M, N, out, ldc, vec_store, epi, wave,
                                   lane, li, h, bias);
}

template <int BIAS = kBiasNone>
int launch(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, const float* alpha,
           int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype, hipStream_t s,
           const char* name, const void* bias = nullptr) {
  const int64_t ntm = ceil_div(M, BM), ntn = ceil_div(N, BN);
  const int64_t tiles = ntm * ntn;
  const size_t esz = out_dtype == BSP_OUT_F32 ? 4 : 2;
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & (4 * esz - 1)) == 0);
  if (out_dtype == BSP_OUT_F32)
    hipLaunchKernelGGL((mm_mxfp4_frag_kernel<true, BIAS>), dim3((unsigned)tiles), dim3(256), 0, s, a, sa,
                       b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  else
    hipLaunchKernelGGL((mm_mxfp4_frag_kernel<false, BIAS>), dim3((unsigned)tiles), dim3(256), 0, s, a, sa,
                       b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  return check_launch(name);
}

}  // namespace mxf
}  // namespace bsp

using namespace bsp;

extern "C" int bsp_mm_mxfp4_frag(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                                 const uint8_t* b_sf, const float* alpha_dev, const void* bias_bf16,
                                 int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
                                 void* stream) {
  const char* fn = "bsp_mm_mxfp4_frag";
  BSP_REQUIRE(M >= 0 && N >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld N=%lld K=%lld", fn,
              (long long)M, (long long)N, (long long)K);
  BSP_REQUIRE(out_dtype == BSP_OUT_BF16 || out_dtype == BSP_OUT_F32, BSP_EDTYPE,
              "%s: out_dtype must be BSP_OUT_BF16 (0) or BSP_OUT_F32 (1), got %d", fn, out_dtype);
  BSP_REQUIRE(K % 256 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 256", fn, (long long)K);
  BSP_REQUIRE(M <= 1 || ldc >= N, BSP_ESHAPE, "%s: ldc (%lld) < N (%lld)", fn, (long long)ldc, (long long)N);
  if (M == 0 || N == 0) return BSP_OK;
  BSP_REQUIRE(a && a_sf && b && b_sf && out, BSP_EINVAL, "%s: null pointer", fn);
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) == 0 &&
                  ((reinterpret_cast<uintptr_t>(a_sf) | reinterpret_cast<uintptr_t>(b_sf)) & 3u) == 0,
              BSP_EINVAL, "%s: fragments must be 16-byte and scales 4-byte aligned", fn);
  BSP_REQUIRE(!bias_bf16 || (reinterpret_cast<uintptr_t>(bias_bf16) & 1u) == 0, BSP_EINVAL,
              "%s: bias must be 2-byte aligned", fn);
  BSP_REQUIRE(ceil_div(M, 256) * ceil_div(N, 256) < (1ll << 31), BSP_ESHAPE, "%s: too many tiles", fn);
  if (int e = check_device()) return e;
  hipStream_t s = (hipStream_t)stream;
  if (bias_bf16)
    return mxf::launch<kBiasBf16After>(a, a_sf, b, b_sf, alpha_dev, M, N, K, out, ldc, out_dtype, s, fn,
                                       bias_bf16);
  return mxf::launch(a, a_sf, b, b_sf, alpha_dev, M, N, K, out, ldc, out_dtype, s, fn);
}
