// a4 -- mm_fp4 on gfx950: C = alpha * A . B^T over NVFP4 operands (e2m1 values, one e4m3 scale
// per 16 K elements in the 128x4 layout), fp32 accumulation, bf16 or fp32 output.
// FastVideo nvfp4_config.py (_mm_fp4, module docstring) and nvfp4_qat_config.py (apply).
//
// Mapping onto CDNA4. gfx950's block-scaled MFMA applies one power-of-two (e8m0) scale per 32
// K elements, while NVFP4 carries a non-power-of-two e4m3 scale per 16; an e2m1 value times an
// e4m3 scale needs up to 6 significant bits, so no 4/6/8-bit MFMA operand can hold it exactly.
// Every such product is exact in fp16, so the packed FP4 bytes and the scale bytes are staged in
// LDS as they are (0.5 byte per element), and each wave dequantizes its own fragments in
// registers (v_cvt_scalef32_pk_f16_fp4 with unit scale, then a packed f16 multiply by the decoded
// e4m3 scale; the convert's own scale operand only honours the exponent) right before
// v_mfma_f32_32x32x16_f16.
//
// Tiling: a 256-thread workgroup owns a 256x256 C tile; each of its 4 waves a 128x128 quarter as
// 4x4 MFMA 32x32 tiles (256 fp32 accumulators per lane). K advances 128 per stage: one stage of
// LDS holds 256 rows x 64 bytes of packed A and of B (four 16-byte chunks per row, XOR-swizzled
// by row for conflict-free 16-byte reads) plus the 128x4 scale tiles (two 128-row tiles x two
// 4-column groups per operand, copied verbatim: in that layout a row's four scales for 64 K are
// one dword). Two stages, register prefetch of the next stage's global data. K % 128 == 64 ends
// with a zero-filled half stage.
//
// Lane (i, h) of a wave (i = lane % 32, h = lane / 32) owns, per stage, the 32 bytes of row i at
// K [64h, 64h + 64): 8 MFMA sub-steps of K 16, sub-step j using its elements 64h + 8j .. + 7
// (both operands use the same K placement, so the MFMA pairs them correctly) with scale byte j/2
// of the row's scale dword for column group h. Dequantization of sub-step j+1 is interleaved
// between the MFMA pairs of sub-step j (explicit scheduling fences), so the VALU work issues while
// the matrix core is busy instead of in bursts that in-order issue would serialize.
//
// The MFMA's A operand is the weight fragment and its B operand the activation fragment, so a
// lane's accumulators hold four consecutive output columns of one output row per group (8-byte
// bf16 stores).
#include "gemm_common.hpp"

namespace bsp {
namespace fp4 {

constexpr int BM = 256, BN = 256, BK = 128;

struct Stage {
  u32x4 a[BM * 4];  // packed A: row r, 16-byte chunk c (K [32c, 32c+32) of the stage) at chunk_slot
  u32x4 b[BN * 4];  // packed B (weights), same
  u32x4 sa[128];    // scale tiles: (row tile rt, column group cg) at [(rt * 2 + cg) * 32 .. +32)
  u32x4 sb[128];
};

__device__ __forceinline__ int chunk_slot(int row, int c) { return row * 4 + (c ^ ((row >> 1) & 3)); }

// scale dword of tile-local row r for column group cg (K [64cg, 64cg + 64) of the stage)
__device__ __forceinline__ uint32_t scale_word(const u32x4* tiles, int r, int cg) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(tiles);
  return w[((r >> 7) * 2 + cg) * 128 + (r & 31) * 4 + ((r >> 5) & 3)];
}

__device__ __forceinline__ f16x2 scale_pair(uint32_t sbyte) {
  const _Float16 hs = (_Float16)e4m3_decode_pos(sbyte);  // e4m3 values are exact in fp16
  return f16x2{hs, hs};
}

// 8 e2m1 values (one dword) times their e4m3 scale (as an f16 pair) -> 8 fp16 (exact)
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 s2) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  p0 *= s2; p1 *= s2; p2 *= s2; p3 *= s2;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t comp(const u32x4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Next stage's global data, held in registers while the current stage computes. Named fields
// (no arrays) so that the struct is promoted to registers.
struct Prefetch {
  u32x4 a0, a1, a2, a3, b0, b1, b2, b3, s;
};

// Chunk q = t + 256 i of an operand: row q / 4, 16-byte chunk q % 4 (64 contiguous bytes per row).
__device__ __forceinline__ void load_stage(Prefetch& pf, const uint8_t* __restrict__ A,
                                           const uint8_t* __restrict__ B,
                                           const uint8_t* __restrict__ SA,
                                           const uint8_t* __restrict__ SB, int64_t M, int64_t N,
                                           int64_t K, int64_t m0, int64_t n0, int64_t kt,
                                           int64_t mtiles128, int64_t ntiles128, int64_t groups,
                                           int t) {
  const int64_t hk = K / 2;
  const int row = t >> 2, c = t & 3;
  const int64_t koff = kt * 64 + c * 16;
  // K % 128 == 64: the last stage has only its first 64 K; the rest is zero-filled (zero values
  // and zero scales contribute nothing)
  const bool tail = kt * 128 + 64 >= K;
  const bool live = !(tail && c >= 2);
  int64_t r;
#define BSP_LD(dst, base, r0, lim, rr)                                  \
  r = (r0) + (rr); r = r < (lim) ? r : (lim) - 1;                       \
  dst = live ? *reinterpret_cast<const u32x4*>((base) + r * hk + koff) : u32x4{0u, 0u, 0u, 0u};
  BSP_LD(pf.a0, A, m0, M, row)
  BSP_LD(pf.a1, A, m0, M, row + 64)
  BSP_LD(pf.a2, A, m0, M, row + 128)
  BSP_LD(pf.a3, A, m0, M, row + 192)
  BSP_LD(pf.b0, B, n0, N, row)
  BSP_LD(pf.b1, B, n0, N, row + 64)
  BSP_LD(pf.b2, B, n0, N, row + 128)
  BSP_LD(pf.b3, B, n0, N, row + 192)
#undef BSP_LD
  // threads 0-127: A's scale tiles, 128-255: B's; (row tile, column group, 16-byte piece)
  const int which = t >> 7, rt = (t >> 6) & 1, cg = (t >> 5) & 1, q = t & 31;
  const int64_t r0 = which ? n0 / 128 : m0 / 128;
  const int64_t nt = which ? ntiles128 : mtiles128;
  int64_t tr = r0 + rt; tr = tr < nt ? tr : nt - 1;
  pf.s = (tail && cg == 1)
             ? u32x4{0u, 0u, 0u, 0u}
             : *reinterpret_cast<const u32x4*>((which ? SB : SA) + (tr * groups + kt * 2 + cg) * 512 + q * 16);
}

__device__ __forceinline__ void store_stage(Stage& st, const Prefetch& pf, int t) {
  const int row = t >> 2, c = t & 3;
  st.a[chunk_slot(row, c)] = pf.a0;
  st.a[chunk_slot(row + 64, c)] = pf.a1;
  st.a[chunk_slot(row + 128, c)] = pf.a2;
  st.a[chunk_slot(row + 192, c)] = pf.a3;
  st.b[chunk_slot(row, c)] = pf.b0;
  st.b[chunk_slot(row + 64, c)] = pf.b1;
  st.b[chunk_slot(row + 128, c)] = pf.b2;
  st.b[chunk_slot(row + 192, c)] = pf.b3;
  if (t < 128)
    st.sa[t] = pf.s;
  else
    st.sb[t - 128] = pf.s;
}

template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void mm_fp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ alpha_ptr, int64_t M, int64_t N,
    int64_t K, void* __restrict__ out, int64_t ldc, int ntm, int ntn, bool vec_store) {
  __shared__ Stage st[2];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  int tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t nk = (K + BK - 1) / BK;
  const int64_t groups = K / 64;  // 128x4 column groups of the scale matrices
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

    u32x4 pa[2][4], pb[2][4];
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + i * 32 + li;
      const int rb = wn * 128 + i * 32 + li;
      pa[0][i] = s.a[chunk_slot(ra, 2 * h)];
      pa[1][i] = s.a[chunk_slot(ra, 2 * h + 1)];
      pb[0][i] = s.b[chunk_slot(rb, 2 * h)];
      pb[1][i] = s.b[chunk_slot(rb, 2 * h + 1)];
      wa[i] = scale_word(s.sa, ra, h);
      wb[i] = scale_word(s.sb, rb, h);
    }

    f16x8 xa[2][4], xb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xa[0][i] = dequant8(pa[0][i].x, scale_pair(wa[i] & 0xFFu));
      xb[0][i] = dequant8(pb[0][i].x, scale_pair(wb[i] & 0xFFu));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int cb = j & 1, nb = cb ^ 1;
      const int jn = j + 1;                        // next sub-step
      const int sh = 8 * (jn >> 1);                // its scale byte
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        const int n = q >> 1, m = 2 * (q & 1);
        acc[n][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xb[cb][n], xa[cb][m], acc[n][m], 0, 0, 0);
        acc[n][m + 1] =
            __builtin_amdgcn_mfma_f32_32x32x16_f16(xb[cb][n], xa[cb][m + 1], acc[n][m + 1], 0, 0, 0);
        if (jn < 8) {                              // dequantize one fragment of sub-step j+1
          if (q < 4)
            xa[nb][q] = dequant8(comp(pa[jn >> 2][q], jn & 3), scale_pair((wa[q] >> sh) & 0xFFu));
          else
            xb[nb][q - 4] = dequant8(comp(pb[jn >> 2][q - 4], jn & 3), scale_pair((wb[q - 4] >> sh) & 0xFFu));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) store_stage(st[cur ^ 1], pf, t);
    __syncthreads();
  }

  store_wave_tile<OUT_F32>(acc, *alpha_ptr, m0 + wm * 128, n0 + wn * 128, M, N, out, ldc, vec_store,
                           li, h);
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
                       alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec);
  else
    hipLaunchKernelGGL(fp4::mm_fp4_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, s, a, sa, b, sb,
                       alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec);
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
