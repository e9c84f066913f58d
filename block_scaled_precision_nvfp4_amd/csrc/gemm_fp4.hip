// mm_fp4 on gfx950: C = alpha * A . B^T over NVFP4 operands (e2m1 values, one e4m3 scale
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
// one dword). Three stages in a ring, filled by global_load_lds (global -> LDS with no register
// staging) two stages ahead, each lane's 32-bit offsets computed once (LoadPlan) and the stage's
// K offset carried in the wave-uniform base. K % 128 == 64 ends with a half stage whose other
// half's scales are zeroed. The stage barrier sits at sub-step 5, so the next stage's fragments
// are read from LDS several MFMA groups before their first use.
//
// Lane (i, h) of a wave (i = lane % 32, h = lane / 32) owns, per stage, the 32 bytes of row i at
// K [64h, 64h + 64): 8 MFMA sub-steps of K 16, sub-step j using its elements 64h + 8j .. + 7
// (both operands use the same K placement, so the MFMA pairs them correctly) with scale byte j/2
// of the row's scale dword for column group h. Dequantization of sub-step j+1 is interleaved
// between the MFMA pairs of sub-step j (explicit scheduling fences, and inside each pair a pinned
// order: MFMA, six VALU instructions, MFMA, the rest), so the VALU work issues while the matrix
// core is busy instead of in bursts that in-order issue would serialize.
//
// The MFMA's A operand is the weight fragment and its B operand the activation fragment, so a
// lane's accumulators hold four consecutive output columns of one output row per group. A tile
// wholly inside C leaves through LDS as whole 256-byte rows (store_tile in gemm_common.hpp).
#include "gemm_common.hpp"

namespace bsp {
namespace fp4 {

constexpr int BM = 256, BN = 256, BK = 128, NSTAGE = 3;
// global_load_lds instructions per wave per stage: 8 operand chunks + 1 scale half (A scales in
// the 128x4 layout), or + 2 dword gathers of A's scales + 1 of B's (A scales in layout_8x4)
template <bool SFA8> constexpr int kLoadsPerStage = SFA8 ? 11 : 9;

struct Stage {
  u32x4 a[BM * 4];  // packed A: row r, 16-byte chunk c (K [32c, 32c+32) of the stage) at chunk_slot
  u32x4 b[BN * 4];  // packed B (weights), same
  u32x4 sa[128];    // scale tiles: (row tile rt, column group cg) at [(rt * 2 + cg) * 32 .. +32)
  u32x4 sb[128];
};

typedef __attribute__((address_space(3))) void lds_t;

// 16-byte chunk c of row r. The XOR pattern makes the 16-byte reads of 8 or 16 consecutive rows
// (one LDS phase of 32 or 64 banks) hit distinct banks.
__device__ __forceinline__ int chunk_slot(int row, int c) {
  return row * 4 + (c ^ (((row >> 1) ^ (row >> 2)) & 3));
}

// f16 holding (e4m3 scale byte) * 2^-8, built from the bits alone: an e4m3 code c (non-negative)
// shifted left by 7 is an f16 with exponent field e and mantissa m, i.e. 2^(e-15) (1 + m/8) for
// e >= 1 and the f16 denormal m * 2^-17 for e == 0, which is the e4m3 value times 2^-8 in both
// cases. The 2^-8 of each operand is undone in the epilogue (alpha * (acc * 2^16)).
// A row's scale dword holds the bytes of four K blocks; two shifts and masks place bytes 0 and 2
// (shift left 7) or bytes 1 and 3 (shift right 1) at bit 7 of the low and high f16 halves, and the
// packed multiply broadcasts the half it needs. `mask` is 0x3F803F80 (sign bits dropped), or 0 to
// zero every scale of the dword.
__device__ __forceinline__ uint32_t scale_halves(uint32_t word, int byte, uint32_t mask) {
  return ((byte & 1) ? (word >> 1) : (word << 7)) & mask;
}
__device__ __forceinline__ f16x2 scale_pair(uint32_t word, int byte, uint32_t mask) {
  const f16x2 t = __builtin_bit_cast(f16x2, scale_halves(word, byte, mask));
  return (byte & 2) ? __builtin_shufflevector(t, t, 1, 1) : __builtin_shufflevector(t, t, 0, 0);
}
constexpr uint32_t kScaleMask = 0x3F803F80u;

// 8 e2m1 values (one dword) times their scale pair -> 8 fp16. Exact: every product e2m1 * e4m3 *
// 2^-8 has at most 6 significant bits and its lowest bit is >= 2^-18, within fp16's reach.
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

// Per-lane part of the global -> LDS loads, fixed for the whole K loop. Slot s = slot0 + lane of
// instruction i holds row s/4 and logical chunk (s%4) ^ ((row/2 ^ row/4) % 4); row/2 and row/4 only
// see lane bits (slot0 is a multiple of 64), so the chunk is the same for all four instructions.
// Offsets are 32-bit and relative to the tile's first row; the stage's K offset and the tile's
// row offset go into the wave-uniform base address.
struct LoadPlan {
  uint32_t offa[4], offb[4];  // (clamped local row) * K/2 + chunk * 16
  uint32_t tail_delta;        // 32 where the chunk is in the stage's second K half, else 0
  uint32_t soff, stail_delta; // scale tiles: column group * 512 + q * 16; 512 for column group 1
};

__device__ __forceinline__ LoadPlan make_load_plan(int64_t M, int64_t N, int64_t K, int64_t m0,
                                                   int64_t n0, int wave, int lane) {
  LoadPlan lp;
  const int64_t hk = K / 2;
  const int row0 = (wave * 16) * 4 + (lane >> 2);  // row of instruction 0; instruction i adds 16 i
  const int c = (lane & 3) ^ (((row0 >> 1) ^ (row0 >> 2)) & 3);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 16 * i;
    const int64_t ra = m0 + row < M ? row : M - 1 - m0;
    const int64_t rb = n0 + row < N ? row : N - 1 - n0;
    lp.offa[i] = (uint32_t)(ra * hk + c * 16);
    lp.offb[i] = (uint32_t)(rb * hk + c * 16);
  }
  lp.tail_delta = c >= 2 ? 32u : 0u;
  const int cg = lane >> 5, q = lane & 31;
  lp.soff = (uint32_t)(cg * 512 + q * 16);
  lp.stail_delta = cg == 1 ? 512u : 0u;
  return lp;
}

// Stage kt's operand and scale bytes, global -> LDS without passing through registers
// (global_load_lds_dwordx4: lane l of an instruction lands at the LDS base + 16 l). Each wave
// issues 4 instructions per operand (64 chunks each) and one for a scale half. The XOR swizzle is
// applied on the global side (LoadPlan).
// K % 128 == 64: the last stage's second half re-reads its first half (in bounds) and the compute
// zeroes that half's scales.
// PART < 0: everything; 0-3: operand chunk pair i = PART; 4: scales. The main loop issues the
// parts during sub-steps 0-4 instead of in one burst.
template <bool SFA8, int PART = -1>
__device__ __forceinline__ void issue_stage(Stage& st, const LoadPlan& lp,
                                            const uint8_t* __restrict__ A,
                                            const uint8_t* __restrict__ B,
                                            const uint8_t* __restrict__ SA,
                                            const uint8_t* __restrict__ SB, int64_t K, int64_t m0,
                                            int64_t n0, int64_t kt, int64_t mtiles128,
                                            int64_t ntiles128, int64_t groups, int64_t rows8,
                                            int wave, int lane) {
  const int64_t hk = K / 2;
  const bool tail = kt * 128 + 64 >= K;
  const uint32_t td = tail ? lp.tail_delta : 0u;
  const uint8_t* a_base = A + m0 * hk + kt * 64;
  const uint8_t* b_base = B + n0 * hk + kt * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (PART >= 0 && PART != i) continue;
    const int slot0 = (wave * 4 + i) * 64;
    __builtin_amdgcn_global_load_lds(a_base + (lp.offa[i] - td), (lds_t*)&st.a[slot0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(b_base + (lp.offb[i] - td), (lds_t*)&st.b[slot0], 16, 0, 0);
  }
  if (PART >= 0 && PART != 4) return;
  const uint32_t soff = lp.soff - (tail ? lp.stail_delta : 0u);
  if constexpr (!SFA8) {
    // waves 0-1: A's two 128-row scale tiles, waves 2-3: B's; slot = rt*64 + cg*32 + q
    const int which = wave >> 1, rt = wave & 1;
    const int64_t r0 = which ? n0 / 128 : m0 / 128;
    const int64_t nt = which ? ntiles128 : mtiles128;
    int64_t tr = r0 + rt; tr = tr < nt ? tr : nt - 1;
    const uint8_t* src = (which ? SB : SA) + (tr * groups + kt * 2) * 512 + soff;
    __builtin_amdgcn_global_load_lds(src, (lds_t*)(which ? &st.sb[rt * 64] : &st.sa[rt * 64]), 16, 0, 0);
  } else {
    // A's scales in layout_8x4: the same LDS image as the 128x4 tiles (slot rt*64 + cg*32 + q holds
    // the dwords of rows q, q+32, q+64, q+96 of half rt), gathered one dword (a row's four scales
    // of a column group) per lane: LDS dword d = 4 * slot + i, two 64-dword loads per wave.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int d = (wave * 2 + u) * 64 + lane;
      const int slot = d >> 2, i = d & 3;
      const int rt = slot >> 6, cgs = (slot >> 5) & 1, qs = slot & 31;
      const int cgd = (tail && cgs == 1) ? 0 : cgs;
      int64_t r = m0 + rt * 128 + qs + 32 * i; r = r < rows8 ? r : rows8 - 1;
      const uint8_t* src = SA + ((r >> 3) * groups + kt * 2 + cgd) * 32 + (r & 7) * 4;
      __builtin_amdgcn_global_load_lds(src, (lds_t*)(reinterpret_cast<uint32_t*>(st.sa) + (wave * 2 + u) * 64),
                                       4, 0, 0);
    }
    // B's two 128-row tiles: waves w and w+2 load the same bytes to the same place
    const int rt = wave & 1;
    int64_t tr = n0 / 128 + rt; tr = tr < ntiles128 ? tr : ntiles128 - 1;
    const uint8_t* src = SB + (tr * groups + kt * 2) * 512 + soff;
    __builtin_amdgcn_global_load_lds(src, (lds_t*)&st.sb[rt * 64], 16, 0, 0);
  }
}

// s_waitcnt vmcnt(n) (n < 16), leaving lgkmcnt and expcnt unconstrained
// s_waitcnt vmcnt(n), n < 64 (bits [3:0] and [15:14] of the immediate), leaving lgkmcnt and
// expcnt unconstrained
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// A wave's fragments of one stage: packed bytes for both 16-byte chunks of its K half and the
// scale dwords of its 4+4 rows (rows r, r+32, r+64, r+96 of a 128x4 tile are one 16-byte run).
struct Frags {
  u32x4 pa[2][4], pb[2][4];
  u32x4 wa, wb;
  uint32_t ma, mb;  // kScaleMask, or 0 where this lane half's K range is past the end
};

// Chunk `cc` (0: sub-steps 0-3, 1: sub-steps 4-7) of a wave's packed fragments of one stage.
__device__ __forceinline__ void read_chunk(Frags& f, const Stage& s, int cc, int wm, int wn, int li,
                                           int h) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + li;
    const int rb = wn * 128 + i * 32 + li;
    f.pa[cc][i] = s.a[chunk_slot(ra, 2 * h + cc)];
    f.pb[cc][i] = s.b[chunk_slot(rb, 2 * h + cc)];
  }
}

// The scale dwords and the first chunk (the second chunk is read during sub-steps 1-2, spreading
// the LDS traffic over the stage).
__device__ __forceinline__ void read_frags(Frags& f, const Stage& s, int wm, int wn, int li, int h,
                                           bool zero_half) {
  // scale dwords first: the first dequantization after the stage barrier needs them and the first
  // chunk's A fragment, and LDS reads complete in order
  f.wa = s.sa[(wm * 2 + h) * 32 + li];
  f.wb = s.sb[(wn * 2 + h) * 32 + li];
  read_chunk(f, s, 0, wm, wn, li, h);
  f.ma = f.mb = zero_half ? 0u : kScaleMask;  // K % 128 == 64 tail: zero this lane half's scales
}

// Dequantization in two halves: the converts of a fragment in one MFMA group, its scale multiplies
// in the next (so no multiply waits on a convert issued just before it).
struct Raw { f16x2 p[4]; f16x2 s; };
__device__ __forceinline__ Raw frag_cvt(const Frags& f, int q, int j) {
  const uint32_t w = q < 4 ? comp(f.pa[j >> 2][q], j & 3) : comp(f.pb[j >> 2][q - 4], j & 3);
  Raw r;
  r.s = q < 4 ? scale_pair(comp(f.wa, q), j >> 1, f.ma) : scale_pair(comp(f.wb, q - 4), j >> 1, f.mb);
  r.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  r.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  r.p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  r.p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return r;
}
__device__ __forceinline__ f16x8 raw_mul(const Raw& r) {
  f16x2 p0 = r.p[0] * r.s, p1 = r.p[1] * r.s, p2 = r.p[2] * r.s, p3 = r.p[3] * r.s;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// dequantize fragment q (0-3: A row tiles, 4-7: B row tiles) of sub-step j from f
__device__ __forceinline__ f16x8 frag_deq(const Frags& f, int q, int j) {
  if (q < 4) return dequant8(comp(f.pa[j >> 2][q], j & 3), scale_pair(comp(f.wa, q), j >> 1, f.ma));
  return dequant8(comp(f.pb[j >> 2][q - 4], j & 3), scale_pair(comp(f.wb, q - 4), j >> 1, f.mb));
}

// ROWSCALE: per-token activation scales; alpha_ptr is then the [M] array of row encode scales
// and w_gsf_ptr the weight's encode scale, alpha_m = fl32(1 / fl32(x_gsf[m] * w_gsf)).
// SFA8: A's scales are in layout_8x4 with rows8 (= ceil(M/8)*8) rows.
// BIAS: the epilogue kind (gemm_common.hpp); with kGeluNvfp4 `out` receives the packed NVFP4 of
// gelu(C), sf_out its scales and out_gsf is the device global scale it is quantized with.
template <bool OUT_F32, bool ROWSCALE, bool SFA8, int BIAS>
__global__ __launch_bounds__(256, 1) void mm_fp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ alpha_ptr,
    const float* __restrict__ w_gsf_ptr, int64_t M, int64_t N, int64_t K, void* __restrict__ out,
    int64_t ldc, int ntm, int ntn, bool vec_store, int64_t rows8, const void* __restrict__ bias,
    uint8_t* __restrict__ sf_out, const float* __restrict__ out_gsf) {
  __shared__ Stage st[NSTAGE];
  __shared__ float rtab[BIAS == kGeluNvfp4 ? 128 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t gtab[BIAS == kGeluNvfp4 ? kGeluTabSize : 8];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  int tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t nk = (K + BK - 1) / BK;
  const bool half_tail = (K % BK) != 0;     // K % 128 == 64
  const int64_t groups = K / 64;            // 128x4 column groups of the scale matrices
  const int64_t mtiles128 = (M + 127) / 128, ntiles128 = (N + 127) / 128;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Stage kt is loaded into buffer kt % 3 two stages ahead. Past the last stage the loads repeat
  // stage nk-1 into a buffer nobody reads again, so every iteration issues and waits for the same
  // number of loads and the loop body has no branches.
  const int64_t last = nk - 1;
  const LoadPlan lp = make_load_plan(M, N, K, m0, n0, wave, lane);
  issue_stage<SFA8>(st[0], lp, A, B, SA, SB, K, m0, n0, 0, mtiles128, ntiles128, groups, rows8, wave,
                    lane);
  issue_stage<SFA8>(st[1], lp, A, B, SA, SB, K, m0, n0, last < 1 ? last : 1, mtiles128, ntiles128,
                    groups, rows8, wave, lane);
  wait_vmcnt<kLoadsPerStage<SFA8>>();
  __builtin_amdgcn_s_barrier();

  Frags f;
  read_frags(f, st[0], wm, wn, li, h, half_tail && nk == 1 && h == 1);
  read_chunk(f, st[0], 1, wm, wn, li, h);
  f16x8 xa[2][4], xb[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xa[0][i] = frag_deq(f, i, 0);
    if (i < 3) xb[0][i] = frag_deq(f, 4 + i, 0);
  }
  Raw r7 = frag_cvt(f, 7, 0), rprev;

  // ring buffers of stages kt, kt+1 and kt+2 (wave-uniform, rotated each iteration)
  int b_cur = 0, b_next = 1, b_ahead = 2;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int64_t ahead = kt + 2 < last ? kt + 2 : last;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int cb = j & 1, nb = cb ^ 1;
      __builtin_amdgcn_sched_barrier(0);
      if (j == 0) issue_stage<SFA8, 0>(st[b_ahead], lp, A, B, SA, SB, K, m0, n0, ahead, mtiles128, ntiles128, groups, rows8, wave, lane);
      if (j == 1) issue_stage<SFA8, 1>(st[b_ahead], lp, A, B, SA, SB, K, m0, n0, ahead, mtiles128, ntiles128, groups, rows8, wave, lane);
      if (j == 2) issue_stage<SFA8, 2>(st[b_ahead], lp, A, B, SA, SB, K, m0, n0, ahead, mtiles128, ntiles128, groups, rows8, wave, lane);
      if (j == 3) issue_stage<SFA8, 3>(st[b_ahead], lp, A, B, SA, SB, K, m0, n0, ahead, mtiles128, ntiles128, groups, rows8, wave, lane);
      if (j == 4) issue_stage<SFA8, 4>(st[b_ahead], lp, A, B, SA, SB, K, m0, n0, ahead, mtiles128, ntiles128, groups, rows8, wave, lane);
      if (j == 5) {
        // Stage kt+1 must be in LDS for every wave: wait until only this wave's loads issued in
        // this iteration are outstanding, then a bare s_barrier (a fence would also wait for the
        // loads still in flight). Every read of the buffer that the next iteration's loads
        // overwrite (stage kt's) happened before this barrier, in sub-steps 1-2 of this iteration
        // and sub-steps 5-7 of the previous one. The next stage's first chunk goes into
        // registers that sub-steps 4-7 no longer read, so it lands well before sub-step 7
        // converts it.
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kLoadsPerStage<SFA8>>();
        __builtin_amdgcn_s_barrier();
        read_chunk(f, st[b_next], 0, wm, wn, li, h);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        // the next stage's scale dwords, each as soon as this stage's last dequantization that
        // reads the old one has issued (A's after fragment 3 of sub-step 7, B's after fragment 7)
        const bool zero_next = half_tail && kt + 2 == nk && h == 1;
        if (j == 6 && q == 4) {
          f.wa = st[b_next].sa[(wm * 2 + h) * 32 + li];
          f.ma = zero_next ? 0u : kScaleMask;
        }
        if (j == 7 && q == 0) {
          f.wb = st[b_next].sb[(wn * 2 + h) * 32 + li];
          f.mb = zero_next ? 0u : kScaleMask;
        }
        // second chunk of this stage: half of it during sub-step 1, half during sub-step 2 (it is
        // first needed by the dequantization of sub-step 4, issued during sub-step 3)
        if ((j == 1 && q == 0) || (j == 2 && q == 0)) {
          const Stage& cs = st[b_cur];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (j == 1) {
              f.pa[1][i] = cs.a[chunk_slot(wm * 128 + i * 32 + li, 2 * h + 1)];
            } else {
              f.pb[1][i] = cs.b[chunk_slot(wn * 128 + i * 32 + li, 2 * h + 1)];
            }
          }
        }
        const int n = q >> 1, m = 2 * (q & 1);
        acc[n][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xb[cb][n], xa[cb][m], acc[n][m], 0, 0, 0);
        acc[n][m + 1] =
            __builtin_amdgcn_mfma_f32_32x32x16_f16(xb[cb][n], xa[cb][m + 1], acc[n][m + 1], 0, 0, 0);
        // convert fragment q of the next sub-step now, multiply fragment q-1 (converted in the
        // previous group; fragment 7 of this sub-step's set was converted in the previous sub-step)
        const Raw rq = frag_cvt(f, q, (j + 1) & 7);
        if (q == 0) {
          xb[cb][3] = raw_mul(r7);     // needed by groups 6-7 of this sub-step
        } else {
          const f16x8 v = raw_mul(rprev);
          if (q - 1 < 4) xa[nb][q - 1] = v; else xb[nb][q - 5] = v;
        }
        if (q == 7) r7 = rq; else rprev = rq;
        // issue order inside the group: one MFMA, six VALU instructions, the other MFMA, the rest,
        // so each MFMA's 32 cycles cover about half of the group's dequantization (the compiler's
        // own order front-loads the VALU work after the first MFMA)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const int b_free = b_cur;
    b_cur = b_next; b_next = b_ahead; b_ahead = b_free;
  }
  wait_vmcnt<0>();

  // operands carried 2^-8 each (scale_pair): the accumulators hold 2^-16 of the true sums, which
  // the epilogue undoes on the accumulator (ACC16)
  float alpha[4];
  if (ROWSCALE) {
    const float wg = *w_gsf_ptr;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t gm = m0 + wm * 128 + m * 32 + li;
      alpha[m] = gm < M ? 1.0f / (alpha_ptr[gm] * wg) : 0.0f;
    }
  } else {
    const float a = *alpha_ptr;
#pragma unroll
    for (int m = 0; m < 4; ++m) alpha[m] = a;
  }
  static_assert(sizeof(st) >= 4 * (kEpiWaveBytes + 1024), "epilogue images overlay the stage buffers");
  if constexpr (BIAS == kGeluNvfp4) {
    store_tile_gelu_nvfp4(acc, alpha, m0, n0, wm, wn, M, N, static_cast<uint8_t*>(out), sf_out,
                          out_gsf, rtab, gtab, reinterpret_cast<uint8_t*>(st), t, wave, lane, li, h);
  } else {
    (void)rtab; (void)gtab; (void)sf_out; (void)out_gsf;
    store_tile<OUT_F32, BIAS, true>(acc, alpha, m0, n0, wm, wn, M, N, out, ldc, vec_store,
                              reinterpret_cast<uint8_t*>(st), wave, lane, li, h, bias);
  }
}


// ---------------------------------------------------------------------------------------------
// Fragment-layout operands (bsp_mm_fp4_frag). The packed bytes of a 32-row tile and a 64-element K
// step are one contiguous 1 KB fragment in which the 16 bytes of lane i + 32 h are row i's
// elements 32 h .. 32 h + 31 of the step; the scales stay in the 128x4 layout. A wave reads its
// operands straight into registers, with no LDS staging and no barrier: per step and row tile one
// fully coalesced 1 KB load, and per row a 2-byte load of the two scales of the lane's 32 elements
// (blocks 4 s + 2 h and + 1; a row's dword of a 128x4 column group holds the four blocks of one
// step). Sub-step j (0..3) of a step uses the lane's elements 8 j .. 8 j + 7, so one MFMA pairs
// K 64 s + 8 j + (0..7) from lanes h = 0 with 64 s + 32 + 8 j + (0..7) from lanes h = 1 -- the same
// placement for both operands -- and each lane's eight elements lie in one 16-block, whose scale
// is byte j / 2 of its pair. Three steps of operands live in a register ring, loaded two steps
// ahead (a step is 64 MFMAs per wave); the dequantization is interleaved with the MFMAs as in the
// LDS-staged loop above. Against row-major operands read the same way (32 bytes of each of 32 rows
// per load) this avoids the partial use of every 128-byte line per step.

// One 64-K step of a wave's operands.
struct StepFrags {
  u32x4 pa[4], pb[4];     // the lane's 16 bytes in each of the wave's A and B row tiles
  uint32_t sa[4], sb[4];  // the two scale bytes of those 32 elements (zero-extended)
};

// Where a wave's operands come from for the whole K loop.
struct FragPlan {
  rsrc_t fa[4], fb[4];  // per 32-row tile: its fragments over all K
  rsrc_t qa, qb;        // the wave's 128-row scale tile over all K
  uint32_t vo;          // lane offset inside a fragment: (i + 32 h) * 16
  uint32_t vs;          // lane offset inside a scale tile: i * 16 + 2 h (row tile r adds 4 r)
};

// m0w, n0w: the wave's first A and B rows (multiples of 128). Tiles past an operand re-read its
// last tile: computed, never stored.
__device__ __forceinline__ FragPlan make_frag_plan(const uint8_t* A, const uint8_t* SA,
                                                   const uint8_t* B, const uint8_t* SB, int64_t M,
                                                   int64_t N, int64_t K, int64_t m0w, int64_t n0w,
                                                   int li, int h) {
  FragPlan p;
  const int64_t ks = K / 64;  // fragments per row tile = 128x4 column groups
  const int64_t mt32 = (M + 31) / 32, nt32 = (N + 31) / 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t ta = m0w / 32 + i < mt32 ? m0w / 32 + i : mt32 - 1;
    const int64_t tb = n0w / 32 + i < nt32 ? n0w / 32 + i : nt32 - 1;
    p.fa[i] = make_rsrc(A + ta * ks * 1024, ks * 1024);
    p.fb[i] = make_rsrc(B + tb * ks * 1024, ks * 1024);
  }
  // scale dword of row r, column group g: (tile * groups + g) * 512 + (r % 32) * 16 + (r / 32 % 4) * 4
  const int64_t mt = (M + 127) / 128, nt = (N + 127) / 128;
  const int64_t ta = m0w / 128 < mt ? m0w / 128 : mt - 1;
  const int64_t tb = n0w / 128 < nt ? n0w / 128 : nt - 1;
  p.qa = make_rsrc(SA + ta * ks * 512, ks * 512);
  p.qb = make_rsrc(SB + tb * ks * 512, ks * 512);
  p.vo = (uint32_t)((li + 32 * h) * 16);
  p.vs = (uint32_t)(li * 16 + 2 * h);
  return p;
}

// Load u (0..15) of step s: 0-3 A fragments, 4-7 B, 8-11 A scale pairs, 12-15 B.
__device__ __forceinline__ void load_one(StepFrags& f, const FragPlan& p, uint32_t s, int u) {
  const int i = u & 3;
  if (u < 4) f.pa[i] = ld16(p.fa[i], p.vo, s * 1024);
  else if (u < 8) f.pb[i] = ld16(p.fb[i], p.vo, s * 1024);
  else if (u < 12) f.sa[i] = ld2(p.qa, p.vs + 4 * i, s * 512);
  else f.sb[i] = ld2(p.qb, p.vs + 4 * i, s * 512);
}

__device__ __forceinline__ void load_step(StepFrags& f, const FragPlan& p, uint32_t s) {
#pragma unroll
  for (int u = 0; u < 16; ++u) load_one(f, p, s, u);
}

// Converts of fragment q (0-3: A row tiles, 4-7: B) of sub-step j. The first use of a step's
// scales (j == 0) turns the lane's two e4m3 bytes into the f16 pair of their values in place, with
// the hardware fp8 -> f16 conversion (exact for every e4m3 code, subnormals included; scale 1);
// sub-steps 0-1 take the low half, 2-3 the high half. Unlike the LDS-staged loop's bit-built
// scales these carry no 2^-8: every product e2m1 * e4m3 is at most 2688 and at least 2^-10 in
// magnitude when nonzero, with at most 6 significant bits: exact in f16.
__device__ __forceinline__ Raw step_cvt(StepFrags& f, int q, int j) {
  const uint32_t w = q < 4 ? comp(f.pa[q], j) : comp(f.pb[q - 4], j);
  uint32_t& sw = q < 4 ? f.sa[q] : f.sb[q - 4];
  if (j == 0)
    sw = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false));
  const f16x2 t = __builtin_bit_cast(f16x2, sw);
  Raw r;
  r.s = (j >> 1) ? __builtin_shufflevector(t, t, 1, 1) : __builtin_shufflevector(t, t, 0, 0);
  r.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  r.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  r.p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  r.p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return r;
}

// The dequantization pipeline between MFMA groups: xa/xb [sub-step parity][row tile] hold the f16
// operands; fragment 7 of the next sub-step and the last converted fragment wait as Raw.
struct DeqState {
  f16x8 xa[2][4], xb[2][4];
  Raw r7, rprev;
};

// Keeps each step's MFMAs in place (the builtins carry no ordering, and a step's MFMAs drifting
// into the next would keep ring buffers live across it).
__device__ __forceinline__ void pin_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) asm volatile("" : "+a"(acc[n][m]));
  __builtin_amdgcn_sched_barrier(0);
}

// One 64-K step on ring buffer BUF: its 4 sub-steps of 16 MFMAs, each interleaved with the
// dequantization of the next sub-step (the next step's first from buffer (BUF + 1) % 3), and the
// 16 loads of step `sl` into buffer (BUF + 2) % 3, one every other MFMA group (a burst of them
// would stall issue).
template <int BUF>
__device__ __forceinline__ void frag_step(f32x16 (&acc)[4][4], StepFrags (&F)[3], DeqState& d,
                                          const FragPlan& p, uint32_t sl) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cb = j & 1, nb = cb ^ 1;
    StepFrags& nf = F[j < 3 ? BUF : (BUF + 1) % 3];
    const int nj = (j + 1) & 3;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_barrier(0);
      if ((q & 1) == 0) {
        load_one(F[(BUF + 2) % 3], p, sl, 4 * j + (q >> 1));
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      const int n = q >> 1, m = 2 * (q & 1);
      acc[n][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(d.xb[cb][n], d.xa[cb][m], acc[n][m], 0, 0, 0);
      acc[n][m + 1] =
          __builtin_amdgcn_mfma_f32_32x32x16_f16(d.xb[cb][n], d.xa[cb][m + 1], acc[n][m + 1], 0, 0, 0);
      const Raw rq = step_cvt(nf, q, nj);
      if (q == 0) {
        d.xb[cb][3] = raw_mul(d.r7);  // needed by groups 6-7 of this sub-step
      } else {
        const f16x8 v = raw_mul(d.rprev);
        if (q - 1 < 4) d.xa[nb][q - 1] = v; else d.xb[nb][q - 5] = v;
      }
      if (q == 7) d.r7 = rq; else d.rprev = rq;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
  }
  pin_acc(acc);
}

// BIAS: kBiasNone or kBiasBf16After (as bsp_mm_fp4_bias).
template <bool OUT_F32, int BIAS>
__global__ __launch_bounds__(256, 1) void mm_fp4_frag_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ alpha_ptr, int64_t M, int64_t N,
    int64_t K, void* __restrict__ out, int64_t ldc, int ntm, int ntn, bool vec_store,
    const void* __restrict__ bias) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kEpiWaveBytes];  // epilogue images only
  const int t = threadIdx.x;
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  int tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t KS = K / 64;
  const FragPlan p = make_frag_plan(A, SA, B, SB, M, N, K, m0 + wm * 128, n0 + wn * 128, li, h);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  StepFrags F[3];
  load_step(F[0], p, 0);
  load_step(F[1], p, KS > 1 ? 1 : 0);
  DeqState d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d.xa[0][i] = raw_mul(step_cvt(F[0], i, 0));
    if (i < 3) d.xb[0][i] = raw_mul(step_cvt(F[0], 4 + i, 0));
  }
  d.r7 = step_cvt(F[0], 7, 0);
  d.rprev = d.r7;

  // steps run in groups of three (the ring period); loads past the end repeat the last step
  int64_t s = 0;
  for (; s + 3 <= KS; s += 3) {
    frag_step<0>(acc, F, d, p, (uint32_t)(s + 2 < KS ? s + 2 : KS - 1));
    frag_step<1>(acc, F, d, p, (uint32_t)(s + 3 < KS ? s + 3 : KS - 1));
    frag_step<2>(acc, F, d, p, (uint32_t)(s + 4 < KS ? s + 4 : KS - 1));
  }
  if (s < KS) frag_step<0>(acc, F, d, p, (uint32_t)(KS - 1));
  if (s + 1 < KS) frag_step<1>(acc, F, d, p, (uint32_t)(KS - 1));
  wait_vmcnt<0>();

  // the operands carry their true values (step_cvt), so the accumulators hold the sums themselves
  const float a = *alpha_ptr;
  const float alpha[4] = {a, a, a, a};
  store_tile<OUT_F32, BIAS, false>(acc, alpha, m0, n0, wm, wn, M, N, out, ldc, vec_store, lds, wave,
                                   lane, li, h, bias);
}

}  // namespace fp4

template <bool ROWSCALE, bool SFA8, int BIAS = kBiasNone>
static void launch_mm_fp4_t(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                            const float* alpha, const float* w_gsf, int64_t M, int64_t N, int64_t K,
                            void* out, int64_t ldc, int out_dtype, hipStream_t s,
                            const void* bias = nullptr, uint8_t* sf_out = nullptr,
                            const float* out_gsf = nullptr) {
  const int64_t ntm = ceil_div(M, fp4::BM), ntn = ceil_div(N, fp4::BN);
  const int64_t tiles = ntm * ntn;
  const size_t esz = out_dtype == BSP_OUT_F32 ? 4 : 2;
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & (4 * esz - 1)) == 0);
  const int64_t rows8 = ceil_div(M, 8) * 8;
  if constexpr (BIAS == kGeluNvfp4)
    hipLaunchKernelGGL((fp4::mm_fp4_kernel<false, ROWSCALE, SFA8, BIAS>), dim3((unsigned)tiles), dim3(256),
                       0, s, a, sa, b, sb, alpha, w_gsf, M, N, K, out, ldc, (int)ntm, (int)ntn, vec,
                       rows8, bias, sf_out, out_gsf);
  else if (out_dtype == BSP_OUT_F32)
    hipLaunchKernelGGL((fp4::mm_fp4_kernel<true, ROWSCALE, SFA8, BIAS>), dim3((unsigned)tiles), dim3(256),
                       0, s, a, sa, b, sb, alpha, w_gsf, M, N, K, out, ldc, (int)ntm, (int)ntn, vec,
                       rows8, bias, sf_out, out_gsf);
  else
    hipLaunchKernelGGL((fp4::mm_fp4_kernel<false, ROWSCALE, SFA8, BIAS>), dim3((unsigned)tiles), dim3(256),
                       0, s, a, sa, b, sb, alpha, w_gsf, M, N, K, out, ldc, (int)ntm, (int)ntn, vec,
                       rows8, bias, sf_out, out_gsf);
}

template <int BIAS>
static void launch_mm_fp4_frag_t(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                 const uint8_t* sb, const float* alpha, int64_t M, int64_t N,
                                 int64_t K, void* out, int64_t ldc, int out_dtype, hipStream_t s,
                                 const void* bias) {
  const int64_t ntm = ceil_div(M, fp4::BM), ntn = ceil_div(N, fp4::BN);
  const int64_t tiles = ntm * ntn;
  const size_t esz = out_dtype == BSP_OUT_F32 ? 4 : 2;
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & (4 * esz - 1)) == 0);
  if (out_dtype == BSP_OUT_F32)
    hipLaunchKernelGGL((fp4::mm_fp4_frag_kernel<true, BIAS>), dim3((unsigned)tiles), dim3(256), 0, s, a,
                       sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  else
    hipLaunchKernelGGL((fp4::mm_fp4_frag_kernel<false, BIAS>), dim3((unsigned)tiles), dim3(256), 0, s, a,
                       sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
}

}  // namespace bsp

using namespace bsp;

// bias_align: 0 for the entry points without a bias, else the bias element size (its alignment);
// a_sf_align: 16 for 128x4 activation scales (16-byte loads), 4 for layout_8x4 (dword loads)
static int mm_fp4_checks(const char* fn, const uint8_t* a_packed, const uint8_t* a_sf,
                         const uint8_t* b_packed, const uint8_t* b_sf, const float* alpha_dev,
                         int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
                         const void* bias = nullptr, unsigned bias_align = 0,
                         unsigned a_sf_align = 16) {
  BSP_REQUIRE(M >= 0 && N >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld N=%lld K=%lld", fn,
              (long long)M, (long long)N, (long long)K);
  BSP_REQUIRE(out_dtype == BSP_OUT_BF16 || out_dtype == BSP_OUT_F32, BSP_EDTYPE,
              "%s: out_dtype must be BSP_OUT_BF16 (0) or BSP_OUT_F32 (1), got %d", fn, out_dtype);
  BSP_REQUIRE(K % 64 == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of 64", fn, (long long)K);
  // the loads address a tile's 256 rows with 32-bit offsets
  BSP_REQUIRE(K <= (1ll << 24), BSP_ESHAPE, "%s: K (%lld) must be at most 16777216", fn, (long long)K);
  BSP_REQUIRE(M <= 1 || ldc >= N, BSP_ESHAPE, "%s: ldc (%lld) < N (%lld)", fn, (long long)ldc,
              (long long)N);
  if (M == 0 || N == 0) return 1;
  BSP_REQUIRE(a_packed && a_sf && b_packed && b_sf && alpha_dev && out, BSP_EINVAL, "%s: null pointer", fn);
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(a_packed) | reinterpret_cast<uintptr_t>(b_packed) |
                reinterpret_cast<uintptr_t>(b_sf)) & 15u) == 0 &&
                  (reinterpret_cast<uintptr_t>(a_sf) & (a_sf_align - 1)) == 0,
              BSP_EINVAL, "%s: operands and weight scales must be 16-byte, activation scales %u-byte aligned",
              fn, a_sf_align);
  BSP_REQUIRE(ceil_div(M, 256) * ceil_div(N, 256) < (1ll << 31), BSP_ESHAPE, "%s: too many tiles", fn);
  BSP_REQUIRE(bias_align == 0 || (bias && (reinterpret_cast<uintptr_t>(bias) & (bias_align - 1)) == 0),
              BSP_EINVAL, "%s: bias must be a non-null device pointer aligned to its element size", fn);
  if (int e = check_device()) return e;
  return 0;
}

extern "C" int bsp_mm_fp4(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                          const uint8_t* b_sf, const float* alpha_dev, int64_t M, int64_t N,
                          int64_t K, void* out, int64_t ldc, int out_dtype, void* stream) {
  int e = mm_fp4_checks("bsp_mm_fp4", a_packed, a_sf, b_packed, b_sf, alpha_dev, M, N, K, out, ldc,
                        out_dtype);
  if (e) return e > 0 ? BSP_OK : e;
  launch_mm_fp4_t<false, false>(a_packed, a_sf, b_packed, b_sf, alpha_dev, nullptr, M, N, K, out, ldc,
                                out_dtype, (hipStream_t)stream);
  return check_launch("bsp_mm_fp4");
}

extern "C" int bsp_mm_fp4_bias(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                               const uint8_t* b_sf, const float* alpha_dev, const void* bias_bf16,
                               int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
                               void* stream) {
  int e = mm_fp4_checks("bsp_mm_fp4_bias", a_packed, a_sf, b_packed, b_sf, alpha_dev, M, N, K, out, ldc,
                        out_dtype, bias_bf16, 2);
  if (e) return e > 0 ? BSP_OK : e;
  launch_mm_fp4_t<false, false, kBiasBf16After>(a_packed, a_sf, b_packed, b_sf, alpha_dev, nullptr, M, N,
                                                K, out, ldc, out_dtype, (hipStream_t)stream, bias_bf16);
  return check_launch("bsp_mm_fp4_bias");
}

extern "C" int bsp_mm_fp4_gelu_nvfp4(const uint8_t* a_packed, const uint8_t* a_sf,
                                     const uint8_t* b_packed, const uint8_t* b_sf,
                                     const float* alpha_dev, const float* out_gsf_dev, int64_t M,
                                     int64_t N, int64_t K, uint8_t* out_packed, uint8_t* out_sf,
                                     void* stream) {
  BSP_REQUIRE(N % 128 == 0, BSP_ESHAPE, "bsp_mm_fp4_gelu_nvfp4: N (%lld) must be a multiple of 128",
              (long long)N);
  BSP_REQUIRE(M == 0 || N == 0 || (out_sf && out_gsf_dev), BSP_EINVAL,
              "bsp_mm_fp4_gelu_nvfp4: null pointer");
  BSP_REQUIRE((reinterpret_cast<uintptr_t>(out_packed) & 3u) == 0 &&
                  (reinterpret_cast<uintptr_t>(out_sf) & 15u) == 0,
              BSP_EINVAL, "bsp_mm_fp4_gelu_nvfp4: out_packed must be 4-byte and out_sf 16-byte aligned");
  // the output is [M, N/2] packed bytes; the ldc and out_dtype given to the checks are nominal
  int e = mm_fp4_checks("bsp_mm_fp4_gelu_nvfp4", a_packed, a_sf, b_packed, b_sf, alpha_dev, M, N, K,
                        out_packed, N, BSP_OUT_BF16);
  if (e) return e > 0 ? BSP_OK : e;
  launch_mm_fp4_t<false, false, kGeluNvfp4>(a_packed, a_sf, b_packed, b_sf, alpha_dev, nullptr, M, N,
                                            K, out_packed, N / 2, BSP_OUT_BF16, (hipStream_t)stream,
                                            nullptr, out_sf, out_gsf_dev);
  return check_launch("bsp_mm_fp4_gelu_nvfp4");
}

extern "C" int bsp_mm_fp4_8x4(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                              const uint8_t* b_sf, const float* alpha_dev, int64_t M, int64_t N,
                              int64_t K, void* out, int64_t ldc, int out_dtype, void* stream) {
  int e = mm_fp4_checks("bsp_mm_fp4_8x4", a_packed, a_sf, b_packed, b_sf, alpha_dev, M, N, K, out, ldc,
                        out_dtype, nullptr, 0, 4);
  if (e) return e > 0 ? BSP_OK : e;
  launch_mm_fp4_t<false, true>(a_packed, a_sf, b_packed, b_sf, alpha_dev, nullptr, M, N, K, out, ldc,
                               out_dtype, (hipStream_t)stream);
  return check_launch("bsp_mm_fp4_8x4");
}

extern "C" int bsp_mm_fp4_per_token(const uint8_t* a_packed, const uint8_t* a_sf,
                                    const uint8_t* b_packed, const uint8_t* b_sf,
                                    const float* x_gsf_rows, const float* w_gsf_dev, int64_t M,
                                    int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
                                    void* stream) {
  int e = mm_fp4_checks("bsp_mm_fp4_per_token", a_packed, a_sf, b_packed, b_sf, x_gsf_rows, M, N, K,
                        out, ldc, out_dtype);
  if (e) return e > 0 ? BSP_OK : e;
  BSP_REQUIRE(w_gsf_dev, BSP_EINVAL, "bsp_mm_fp4_per_token: null pointer");
  launch_mm_fp4_t<true, false>(a_packed, a_sf, b_packed, b_sf, x_gsf_rows, w_gsf_dev, M, N, K, out,
                               ldc, out_dtype, (hipStream_t)stream);
  return check_launch("bsp_mm_fp4_per_token");
}

extern "C" int bsp_mm_fp4_frag(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                               const uint8_t* b_sf, const float* alpha_dev, const void* bias_bf16,
                               int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
                               void* stream) {
  int e = mm_fp4_checks("bsp_mm_fp4_frag", a_packed, a_sf, b_packed, b_sf, alpha_dev, M, N, K, out, ldc,
                        out_dtype, bias_bf16, bias_bf16 ? 2 : 0);
  if (e) return e > 0 ? BSP_OK : e;
  if (bias_bf16)
    launch_mm_fp4_frag_t<kBiasBf16After>(a_packed, a_sf, b_packed, b_sf, alpha_dev, M, N, K, out, ldc,
                                         out_dtype, (hipStream_t)stream, bias_bf16);
  else
    launch_mm_fp4_frag_t<kBiasNone>(a_packed, a_sf, b_packed, b_sf, alpha_dev, M, N, K, out, ldc,
                                    out_dtype, (hipStream_t)stream, nullptr);
  return check_launch("bsp_mm_fp4_frag");
}
