// The MX GEMMs on operands stored in the MFMA fragment layout: C = alpha * A . B^T (+ bias) with
// e2m1 (MXFP4) or e4m3 (MXFP8) elements and one e8m0 scale per 32 K elements per row (OCP MX),
// fp32 accumulation, bf16 or fp32 output. FastVideo nvfp4_config.py (_mm_fp4 with use_nvfp4=False;
// "MX-FP4" in the module docstring); vLLM-Omni mxfp8_config.py (DiffusionMXFP8Config: 32-element
// e8m0 groups; NPUMxfp8LinearMethod._quant_matmul with the per-row scales of both operands and an
// fp32 bias). FastVideo's quantize op carries a do_shuffle switch for operands pre-arranged for the
// matrix unit (always off there, the arrangement left to the library); the fragment layout is that
// arrangement for gfx950. Same products and the same K order as bsp_mm_mxfp4 / bsp_mm_mxfp8: the
// outputs are bit-identical for the same operand values.
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
// (MXFP8's fragments are 2 KB, described at its kernel below; its scales are laid out as MXFP4's.)
//
// Every wave loads the fragments of its four A and four B row tiles straight into registers, each
// a fully coalesced 1 KB read, three K steps ahead into a ring of four register buffers (MXFP8: two
// steps ahead into a ring of three); no LDS and no workgroup barrier in the K loop (the two waves
// that share a row tile read it from the caches independently). Against the LDS-staged kernel this drops the LDS writes and reads and the
// per-stage barriers, at twice the L2 reads. Tiling and epilogue as the LDS-staged MX kernel:
// 256x256 C tile per 256-thread workgroup, 128x128 per wave, XCD-aware tile order, whole tiles
// leave through LDS as whole rows.
#include <stdlib.h>

#include "gemm_common.hpp"

namespace bsp {
namespace mxf {

constexpr int BM = 256, BN = 256;

// Ends a K step: the step's MFMAs stay before this point and the next step's after it. The MFMA
// builtins have no memory or side-effect ordering, so without this the scheduler may sink a step's
// MFMAs past later steps, which keeps their ring buffers live across the loop's back edge (register
// copies and a full wait on the loads every iteration).
__device__ __forceinline__ void pin_step(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) asm volatile("" : "+a"(acc[n][m]));
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ i32x8 fp4_op(const u32x4& x) {
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};  // e2m1: four registers are read
}

// One K step (J = ks % 4) of a wave: its 16 MFMAs on ring buffer J, the loads of step kl (three
// ahead) into buffer (J + 3) % 4, whose step was consumed by the previous call, spread between them.
// ST: deferred store s of the previous tile's image rides along (its LDS read before the MFMAs,
// its global store after the step's loads).
template <int J, bool ST>
__device__ __forceinline__ void frag_step(f32x16 (&acc)[4][4], u32x4 (&xa)[4][4], u32x4 (&xb)[4][4],
                                          const uint32_t (&csa)[4], const uint32_t (&csb)[4],
                                          const rsrc_t (&fa)[4], const rsrc_t (&fb)[4], uint32_t kl,
                                          uint32_t loff, const uint8_t* img, int s, uint16_t* pbase,
                                          int64_t ldc, int lane) {
  constexpr int NB = (J + 3) & 3;
  u32x4 dv;
  if (ST) dv = img_load(img, s, lane);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int n = q >> 1, m = 2 * (q & 1);
    acc[n][m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        fp4_op(xb[J][n]), fp4_op(xa[J][m]), acc[n][m], 4, 4, J, (int)csb[n], J, (int)csa[m]);
    acc[n][m + 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        fp4_op(xb[J][n]), fp4_op(xa[J][m + 1]), acc[n][m + 1], 4, 4, J, (int)csb[n], J, (int)csa[m + 1]);
    if (q < 4) {
      xa[NB][q] = ld16(fa[q], loff, kl * 1024);
      xb[NB][q] = ld16(fb[q], loff, kl * 1024);
    }
  }
  if (ST) {
    img_put(dv, s, pbase, ldc, lane);
    // the LDS read first, the store half a step later, so its wait on the read costs nothing
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
    __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);   // the step's eight loads
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // eight MFMAs
    __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);   // the store
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // eight MFMAs
  }
  pin_step(acc);  // keeps the loads of this step here, three steps before use
}

// The four K steps of scale group kg, with SPG (0, 2 or 4) deferred stores, segments s0, s0 + 1, ..
// (SPG 2: on steps 0 and 2).
template <int SPG>
__device__ __forceinline__ void frag_group(f32x16 (&acc)[4][4], u32x4 (&xa)[4][4], u32x4 (&xb)[4][4],
                                           uint32_t (&csa)[4], uint32_t (&csb)[4],
                                           const rsrc_t (&fa)[4], const rsrc_t (&fb)[4],
                                           const rsrc_t (&qa)[4], const rsrc_t (&qb)[4], int64_t kg,
                                           int64_t KS, int64_t KG, uint32_t loff, uint32_t soff,
                                           const uint8_t* img, int s0, uint16_t* pbase, int64_t ldc,
                                           int lane) {
  uint32_t nsa[4], nsb[4];
  {  // the next group's scale dwords (the last group reloads itself)
    const uint32_t kn = (uint32_t)(kg + 1 < KG ? kg + 1 : KG - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nsa[i] = ld4(qa[i], soff, kn * 256);
      nsb[i] = ld4(qb[i], soff, kn * 256);
    }
  }
  const int64_t ks = kg * 4;   // loads run three steps ahead; past the end the last step reloads
  frag_step<0, (SPG > 0)>(acc, xa, xb, csa, csb, fa, fb, (uint32_t)(ks + 3 < KS ? ks + 3 : KS - 1),
                          loff, img, s0, pbase, ldc, lane);
  frag_step<1, (SPG == 4)>(acc, xa, xb, csa, csb, fa, fb, (uint32_t)(ks + 4 < KS ? ks + 4 : KS - 1),
                           loff, img, s0 + 1, pbase, ldc, lane);
  frag_step<2, (SPG > 0)>(acc, xa, xb, csa, csb, fa, fb, (uint32_t)(ks + 5 < KS ? ks + 5 : KS - 1),
                          loff, img, s0 + SPG / 2, pbase, ldc, lane);
  frag_step<3, (SPG == 4)>(acc, xa, xb, csa, csb, fa, fb, (uint32_t)(ks + 6 < KS ? ks + 6 : KS - 1),
                           loff, img, s0 + 3, pbase, ldc, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    csa[i] = nsa[i];
    csb[i] = nsb[i];
  }
}

// The wave's remaining deferred stores, segments s .. kImgStores-1, back to back.
__device__ __forceinline__ void img_flush(const uint8_t* img, int s, uint16_t* pbase, int64_t ldc,
                                          int lane) {
  for (; s < kImgStores; ++s) img_put(img_load(img, s, lane), s, pbase, ldc, lane);
}

// Persistent: workgroup w takes tiles w, w + gridDim.x, ... of the XCD-aware order (the grid is a
// multiple of the XCD count, so every tile of a workgroup maps to the XCD it runs on). A wave's
// whole bf16 tile waits in its LDS image and leaves during the next tile's first K groups, SPG
// (2 or 4) stores per group; what a short K loop leaves is stored after it. Ragged tiles and fp32
// output are stored directly.
template <bool OUT_F32, int BIAS, int SPG>
__global__ __launch_bounds__(256, 1) void mm_mxfp4_frag_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ alpha_ptr, int64_t M, int64_t N,
    int64_t K, void* __restrict__ out, int64_t ldc, int ntm, int ntn, bool vec_store,
    const void* __restrict__ bias) {
  constexpr bool kImg = !OUT_F32;
  __shared__ __attribute__((aligned(16))) uint8_t img_all[kImg ? 4 * kImgWaveBytes : 16];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  uint8_t* img = img_all + (kImg ? wave * kImgWaveBytes : 0);
  const int64_t KS = K >> 6, KG = KS >> 2;
  const int64_t kg_st = KG < kImgStores / SPG ? KG : kImgStores / SPG;  // groups that carry stores
  const int64_t ra_last = ((M + 31) >> 5) - 1, rb_last = ((N + 31) >> 5) - 1;
  const int total = ntm * ntn;
  const bool can_img = kImg && ldc % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const float a = alpha_ptr ? *alpha_ptr : 1.0f;
  const float alpha[4] = {a, a, a, a};
  uint16_t* pbase = nullptr;   // destination of the image waiting in LDS, null if none

  for (int v = blockIdx.x; v < total; v += gridDim.x) {
    int tm, tn;
    tile_coords(v, ntm, ntn, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    // Lane-derived offsets are recomputed for each tile: hoisted out of the tile loop they would
    // stay live across the K loop and push its registers into memory.
    const int lk = opaque(lane);
    const uint32_t loff = lk * 16, soff = lk * 4;

    // wave-uniform bases of the wave's four A and four B row tiles (rows past the operand clamp
    // to its last tile: read, never stored)
    rsrc_t fa[4], fb[4], qa[4], qb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t ra = (m0 >> 5) + wm * 4 + i;
      ra = ra < ra_last ? ra : ra_last;
      int64_t rb = (n0 >> 5) + wn * 4 + i;
      rb = rb < rb_last ? rb : rb_last;
      fa[i] = make_rsrc(A + ra * KS * 1024, KS * 1024);
      fb[i] = make_rsrc(B + rb * KS * 1024, KS * 1024);
      qa[i] = make_rsrc(SA + ra * KG * 256, KG * 256);
      qb[i] = make_rsrc(SB + rb * KG * 256, KG * 256);
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    u32x4 xa[4][4], xb[4][4];          // [ring buffer][row tile]
    uint32_t csa[4], csb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      csa[i] = ld4(qa[i], soff, 0);
      csb[i] = ld4(qb[i], soff, 0);
    }
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const uint32_t ks = b < KS ? b : KS - 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xa[b][i] = ld16(fa[i], loff, ks * 1024);
        xb[b][i] = ld16(fb[i], loff, ks * 1024);
      }
    }

    int64_t kg = 0;
    if (kImg && pbase) {
      for (; kg < kg_st; ++kg)
        frag_group<SPG>(acc, xa, xb, csa, csb, fa, fb, qa, qb, kg, KS, KG, loff, soff, img,
                        (int)kg * SPG, pbase, ldc, lk);
      img_flush(img, (int)kg_st * SPG, pbase, ldc, lk);
      pbase = nullptr;
    }
    for (; kg < KG; ++kg)
      frag_group<0>(acc, xa, xb, csa, csb, fa, fb, qa, qb, kg, KS, KG, loff, soff, img, 0, pbase,
                    ldc, lk);

    const int le = opaque(lane);   // the epilogue's lane offsets, computed after the K loop
    const int64_t m0w = m0 + wm * 128, n0w = n0 + wn * 128;
    if (can_img && m0 + BM <= M && n0 + BN <= N) {
      img_write<BIAS, false>(acc, alpha, n0w, N, img, le & 31, le >> 5, bias);
      pbase = static_cast<uint16_t*>(out) + m0w * ldc + n0w;
    } else {
      store_wave_tile<OUT_F32, BIAS, false>(acc, alpha, m0w, n0w, M, N, out, ldc, vec_store, le & 31,
                                            le >> 5, bias);
    }
  }
  if (kImg && pbase) img_flush(img, 0, pbase, ldc, lane);
}

// ---------------------------------------------------------------------------------------------
// MXFP8: a fragment of row tile rt and K step ks is 2 KB at (rt * K/64 + ks) * 2048, two 1 KB halves
// b = 0, 1 (the step's two 32-element blocks); in half b, lane l = i + 32 h holds elements
// 64 ks + 32 b + 16 h .. + 15 of row 32 rt + i, so the lane's two 16-byte loads are bytes 0-15 and
// 16-31 of the MFMA's e4m3 operand. Scales as for MXFP4. The operand is 8 registers, so the ring
// is three buffers deep (loads two K steps ahead) and the K loop is unrolled over 12 steps, the
// period of both the ring and the four-step scale groups.
__device__ __forceinline__ i32x8 ld_fp8_frag(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 lo = ld16(r, voff, soff), hi = ld16(r, voff + 1024, soff);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int J, int B>
__device__ __forceinline__ void frag8_step(f32x16 (&acc)[4][4], i32x8 (&xa)[3][4], i32x8 (&xb)[3][4],
                                           const uint32_t (&csa)[4], const uint32_t (&csb)[4],
                                           const rsrc_t (&fa)[4], const rsrc_t (&fb)[4], uint32_t kl,
                                           uint32_t loff) {
  constexpr int NB = (B + 2) % 3;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int n = q >> 1, m = 2 * (q & 1);
    acc[n][m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xb[B][n], xa[B][m], acc[n][m], 0, 0, J,
                                                                (int)csb[n], J, (int)csa[m]);
    acc[n][m + 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xb[B][n], xa[B][m + 1], acc[n][m + 1],
                                                                    0, 0, J, (int)csb[n], J, (int)csa[m + 1]);
    if (q < 4) {
      xa[NB][q] = ld_fp8_frag(fa[q], loff, kl * 2048);
      xb[NB][q] = ld_fp8_frag(fb[q], loff, kl * 2048);
    }
  }
  pin_step(acc);
}

// four steps of one scale group, starting at step ks with ring buffer B0 (= ks % 3)
template <int B0>
__device__ __forceinline__ void frag8_group(f32x16 (&acc)[4][4], i32x8 (&xa)[3][4], i32x8 (&xb)[3][4],
                                            uint32_t (&csa)[4], uint32_t (&csb)[4],
                                            const rsrc_t (&fa)[4], const rsrc_t (&fb)[4],
                                            const rsrc_t (&qa)[4], const rsrc_t (&qb)[4],
                                            int64_t ks, int64_t KS, uint32_t loff, uint32_t soff) {
  uint32_t nsa[4], nsb[4];
  const uint32_t kn = (uint32_t)(ks / 4 + 1 < KS / 4 ? ks / 4 + 1 : KS / 4 - 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nsa[i] = ld4(qa[i], soff, kn * 256);
    nsb[i] = ld4(qb[i], soff, kn * 256);
  }
  frag8_step<0, B0>(acc, xa, xb, csa, csb, fa, fb, (uint32_t)(ks + 2 < KS ? ks + 2 : KS - 1), loff);
  frag8_step<1, (B0 + 1) % 3>(acc, xa, xb, csa, csb, fa, fb, (uint32_t)(ks + 3 < KS ? ks + 3 : KS - 1), loff);
  frag8_step<2, (B0 + 2) % 3>(acc, xa, xb, csa, csb, fa, fb, (uint32_t)(ks + 4 < KS ? ks + 4 : KS - 1), loff);
  frag8_step<3, B0>(acc, xa, xb, csa, csb, fa, fb, (uint32_t)(ks + 5 < KS ? ks + 5 : KS - 1), loff);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    csa[i] = nsa[i];
    csb[i] = nsb[i];
  }
}

template <bool OUT_F32, int BIAS>
__global__ __launch_bounds__(256, 1) void mm_mxfp8_frag_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, void* __restrict__ out,
    int64_t ldc, int ntm, int ntn, bool vec_store, const void* __restrict__ bias) {
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
  rsrc_t fa[4], fb[4], qa[4], qb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t ra = (m0 >> 5) + wm * 4 + i;
    ra = ra < ra_last ? ra : ra_last;
    int64_t rb = (n0 >> 5) + wn * 4 + i;
    rb = rb < rb_last ? rb : rb_last;
    fa[i] = make_rsrc(A + ra * KS * 2048, KS * 2048);
    fb[i] = make_rsrc(B + rb * KS * 2048, KS * 2048);
    qa[i] = make_rsrc(SA + ra * KG * 256, KG * 256);
    qb[i] = make_rsrc(SB + rb * KG * 256, KG * 256);
  }
  const uint32_t loff = lane * 16, soff = lane * 4;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  i32x8 xa[3][4], xb[3][4];
  uint32_t csa[4], csb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    csa[i] = ld4(qa[i], soff, 0);
    csb[i] = ld4(qb[i], soff, 0);
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t ks = b < KS ? b : KS - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xa[b][i] = ld_fp8_frag(fa[i], loff, ks * 2048);
      xb[b][i] = ld_fp8_frag(fb[i], loff, ks * 2048);
    }
  }
  int64_t ks = 0;
  for (; ks + 12 <= KS; ks += 12) {
    frag8_group<0>(acc, xa, xb, csa, csb, fa, fb, qa, qb, ks, KS, loff, soff);
    frag8_group<1>(acc, xa, xb, csa, csb, fa, fb, qa, qb, ks + 4, KS, loff, soff);
    frag8_group<2>(acc, xa, xb, csa, csb, fa, fb, qa, qb, ks + 8, KS, loff, soff);
  }
  if (ks + 4 <= KS) frag8_group<0>(acc, xa, xb, csa, csb, fa, fb, qa, qb, ks, KS, loff, soff);
  if (ks + 8 <= KS) frag8_group<1>(acc, xa, xb, csa, csb, fa, fb, qa, qb, ks + 4, KS, loff, soff);

  const float alpha[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  store_tile<OUT_F32, BIAS, false>(acc, alpha, m0, n0, wm, wn, M, N, out, ldc, vec_store, epi, wave,
                                   lane, li, h, bias);
}

template <int BIAS = kBiasNone>
int launch8(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, int64_t M,
            int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype, hipStream_t s,
            const char* name, const void* bias = nullptr) {
  const int64_t ntm = ceil_div(M, BM), ntn = ceil_div(N, BN);
  const int64_t tiles = ntm * ntn;
  const size_t esz = out_dtype == BSP_OUT_F32 ? 4 : 2;
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & (4 * esz - 1)) == 0);
  if (out_dtype == BSP_OUT_F32)
    hipLaunchKernelGGL((mm_mxfp8_frag_kernel<true, BIAS>), dim3((unsigned)tiles), dim3(256), 0, s, a, sa,
                       b, sb, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  else
    hipLaunchKernelGGL((mm_mxfp8_frag_kernel<false, BIAS>), dim3((unsigned)tiles), dim3(256), 0, s, a, sa,
                       b, sb, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  return check_launch(name);
}

// Workgroups of the launch. Up to K = 5120 a persistent grid: one workgroup per compute unit (a
// workgroup fills a CU's registers), rounded down to a multiple of the XCD count, each storing a
// tile during the next one's K loop (measured at M = 32760, N = 13824: 4-12 % faster for K <=
// 2048, even at 5120). Above it one tile per workgroup, which measured 2-4 % faster at K = 8192 and
// 13824. BSP_PERSISTENT_GRID=n sets the count (tests use small grids so that each workgroup runs
// many tiles).
inline int64_t mx_frag_grid(int64_t tiles, int64_t K) {
  int64_t g = tiles;
  if (K <= 5120) {
    g = device_cu_count();
    g = g >= kXcds ? g / kXcds * kXcds : 256;
  }
  if (const char* e = getenv("BSP_PERSISTENT_GRID")) {
    const long long n = atoll(e);
    if (n > 0) g = n;
  }
  return tiles < g ? tiles : g;
}

template <int BIAS = kBiasNone>
int launch(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, const float* alpha,
           int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype, hipStream_t s,
           const char* name, const void* bias = nullptr) {
  const int64_t ntm = ceil_div(M, BM), ntn = ceil_div(N, BN);
  const int64_t grid = mx_frag_grid(ntm * ntn, K);
  const size_t esz = out_dtype == BSP_OUT_F32 ? 4 : 2;
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & (4 * esz - 1)) == 0);
  if (out_dtype == BSP_OUT_F32)
    hipLaunchKernelGGL((mm_mxfp4_frag_kernel<true, BIAS, 2>), dim3((unsigned)grid), dim3(256), 0, s, a,
                       sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  else if (K / 256 >= kImgStores / 2)   // 16 or more scale groups: two deferred stores per group
    hipLaunchKernelGGL((mm_mxfp4_frag_kernel<false, BIAS, 2>), dim3((unsigned)grid), dim3(256), 0, s, a,
                       sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  else
    hipLaunchKernelGGL((mm_mxfp4_frag_kernel<false, BIAS, 4>), dim3((unsigned)grid), dim3(256), 0, s, a,
                       sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
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
  // a row tile's fragments are one buffer resource whose size (32 K bytes at most) is a signed
  // 32-bit field
  BSP_REQUIRE(K <= (1ll << 24), BSP_ESHAPE, "%s: K (%lld) must be at most 2^24", fn, (long long)K);
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

extern "C" int bsp_mm_mxfp8_frag(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                                 const uint8_t* b_sf, const float* bias_f32, int64_t M, int64_t N,
                                 int64_t K, void* out, int64_t ldc, int out_dtype, void* stream) {
  const char* fn = "bsp_mm_mxfp8_frag";
  BSP_REQUIRE(M >= 0 && N >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld N=%lld K=%lld", fn,
              (long long)M, (long long)N, (long long)K);
  BSP_REQUIRE(out_dtype == BSP_OUT_BF16 || out_dtype == BSP_OUT_F32, BSP_EDTYPE,
              "%s: out_dtype must be BSP_OUT_BF16 (0) or BSP_OUT_F32 (1), got %d", fn, out_dtype);
  BSP_REQUIRE(K % 256 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 256", fn, (long long)K);
  // a row tile's fragments are one buffer resource whose size (32 K bytes at most) is a signed
  // 32-bit field
  BSP_REQUIRE(K <= (1ll << 24), BSP_ESHAPE, "%s: K (%lld) must be at most 2^24", fn, (long long)K);
  BSP_REQUIRE(M <= 1 || ldc >= N, BSP_ESHAPE, "%s: ldc (%lld) < N (%lld)", fn, (long long)ldc, (long long)N);
  if (M == 0 || N == 0) return BSP_OK;
  BSP_REQUIRE(a && a_sf && b && b_sf && out, BSP_EINVAL, "%s: null pointer", fn);
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) == 0 &&
                  ((reinterpret_cast<uintptr_t>(a_sf) | reinterpret_cast<uintptr_t>(b_sf)) & 3u) == 0,
              BSP_EINVAL, "%s: fragments must be 16-byte and scales 4-byte aligned", fn);
  BSP_REQUIRE(!bias_f32 || (reinterpret_cast<uintptr_t>(bias_f32) & 3u) == 0, BSP_EINVAL,
              "%s: bias must be 4-byte aligned", fn);
  BSP_REQUIRE(ceil_div(M, 256) * ceil_div(N, 256) < (1ll << 31), BSP_ESHAPE, "%s: too many tiles", fn);
  if (int e = check_device()) return e;
  hipStream_t s = (hipStream_t)stream;
  if (bias_f32)
    return mxf::launch8<kBiasF32Before>(a, a_sf, b, b_sf, M, N, K, out, ldc, out_dtype, s, fn, bias_f32);
  return mxf::launch8(a, a_sf, b, b_sf, M, N, K, out, ldc, out_dtype, s, fn);
}
