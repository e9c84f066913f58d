// mm_mxfp8, and the MXFP4 GEMM (mm_fp4 with MX scales), on gfx950's block-scaled MFMA.
// C = alpha * A . B^T with OCP MX operands: one e8m0 scale per 32 K elements per row of each
// operand, fp32 accumulation, bf16 or fp32 output.
//   vLLM-Omni mxfp8_config.py (DiffusionMXFP8Config; NPUMxfp8LinearMethod._quant_matmul): e4m3
//   elements, per-row e8m0 scales of both operands, group [1, 1, 32]; scales row-major [rows, K/32].
//   FastVideo nvfp4_config.py (_mm_fp4, use_nvfp4=False; "MX-FP4" in the module docstring): e2m1
//   elements with MX scales; scales in the 128x4 layout mm_fp4 takes for its operands.
//
// The MX block scale is what v_mfma_scale_f32_32x32x64_f8f6f4 consumes: one e8m0 scale per row and
// 32-element K block, supplied by the lane half that owns the block (lane i + 32 b for block b of
// row i). Operand placement inside a lane (measured on the hardware with one-hot operands and
// distinct per-lane scales): with 4-bit elements lane half h holds the 32 elements of block h
// (16 contiguous bytes); with 8-bit elements bytes 0-15 of every lane are elements of block 0 and
// bytes 16-31 elements of block 1, lane half h supplying the 16-element half h of each block.
//
// Tiling: 256x256 C tile per 256-thread workgroup, 128x128 per wave (4x4 MFMA 32x32 tiles). A stage
// holds 64 bytes per row of each operand (64 K of e4m3 or 128 K of e2m1) in LDS as four 16-byte
// chunks XOR-swizzled by row, plus the stage's scale bytes per row, filled by global_load_lds
// (no register staging), in a 4-stage ring loaded three stages ahead (a stage computes in ~1000
// cycles, shorter than the memory latency under load). The loads of stage kt+3 are issued one per
// MFMA pair during stage kt rather than in a burst. Fragments of the next stage are read into a
// second register set behind a barrier placed 768 MFMA cycles before the stage ends; their scale
// dwords are shifted for the lane half only when that stage starts, so nothing waits on the LDS
// reads while the current stage's MFMAs are still to be issued. The epilogue is shared with mm_fp4
// (store_tile in gemm_common.hpp: whole tiles leave through LDS as whole rows).
//
// MXFP8 scales are row-major, so a stage's scales are one dword per row, 256 rows 160+ bytes
// apart: a load instruction of them touches 64 cache lines for 256 bytes, and two per stage cost
// a fifth of the kernel's time. When K % 512 == 0 and the scale matrices are 16-byte aligned the
// kernel instead fetches each row's 16 bytes for 512 K (eight stages) with one 16-byte load per
// row and operand every eight stages, rewrites them pair-major in LDS, and reads each lane's
// scales as before with one 16-byte LDS read (scale blocks; otherwise the per-stage dwords).
#include "gemm_common.hpp"

namespace bsp {
namespace mx {

constexpr int BM = 256, BN = 256, NSTAGE = 4;  // loads run three stages ahead

template <int FMT> struct Cfg;
template <> struct Cfg<0> {  // MXFP8: e4m3, scales row-major [rows, K/32]
  static constexpr int BK = 64, KSTEPS = 1, CODE = 0, BAR_PAIRS = 6;
};
template <> struct Cfg<1> {  // MXFP4: e2m1, scales in the 128x4 layout
  static constexpr int BK = 128, KSTEPS = 2, CODE = 4, BAR_PAIRS = 12;
};

// global_load_lds instructions per wave per stage. MXFP8 with scale blocks (SCB) fetches its scales
// separately, 16 bytes per row for eight stages at a time (issue_scale_block below).
template <int FMT, bool SCB> constexpr int kLoads = FMT == 0 ? (SCB ? 8 : 10) : 9;

// MXFP8 scale blocks: a block is each row's 16 scale bytes for 512 K (four 128-K stage pairs).
// Per operand and block, four 1 KB pair areas in the order of a stage's scale area (below), in two
// buffers (the current block and the next).
constexpr int kScbDwords = 4 * 256;

struct Stage {
  u32x4 a[BM * 4];     // row r, chunk c at chunk_slot(r, c)
  u32x4 b[BN * 4];
  u32x4 sa[64];        // scales, see issue_stage
  u32x4 sb[64];
};

typedef __attribute__((address_space(3))) void lds_t;

// 16-byte chunk c of row r. The XOR pattern makes the 16-byte reads of 8 or 16 consecutive rows
// (one LDS phase of 32 or 64 banks) hit distinct banks.
__device__ __forceinline__ int chunk_slot(int row, int c) {
  return row * 4 + (c ^ (((row >> 1) ^ (row >> 2)) & 3));
}

// s_waitcnt vmcnt(n), n < 64 (bits [3:0] and [15:14] of the immediate), leaving lgkmcnt and
// expcnt unconstrained
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Scale staging: the four rows a lane's four MFMA tiles use (r, r+32, r+64, r+96 of one 128-row
// half) sit next to each other, so a lane fetches all its scales with one LDS read.
//  MXFP8: dword p of the 1 KB area holds row (p / 128) * 128 + (p % 4) * 32 + (p % 128) / 4's four
//         scale bytes of the 128-K pair of stages the stage belongs to (16-byte reads);
//  MXFP4: the two 512-byte 128x4 tiles of the stage's column group, copied verbatim (in that
//         layout the 16 bytes at (r % 32) * 16 are rows r, r+32, r+64, r+96; 16-byte reads).
// PART < 0: all loads of the stage; else only load PART (0-3 A chunks, 4-7 B chunks, 8 the
// scales (MXFP8: A's dword), 9 B's scale dword (MXFP8))
template <int FMT, int PART = -1, bool SCB = false>
__device__ __forceinline__ void issue_stage(Stage& st, const uint8_t* __restrict__ A,
                                            const uint8_t* __restrict__ B,
                                            const uint8_t* __restrict__ SA,
                                            const uint8_t* __restrict__ SB, int64_t M, int64_t N,
                                            int64_t K, int64_t m0, int64_t n0, int64_t kt, int wave,
                                            int lane) {
  const int64_t rowbytes = FMT == 0 ? K : K / 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot0 = (wave * 4 + i) * 64;
    const int s = slot0 + lane;
    const int row = s >> 2;
    const int c = (s & 3) ^ (((row >> 1) ^ (row >> 2)) & 3);
    const int64_t off = kt * 64 + c * 16;
    if (PART < 0 || PART == i) {
      int64_t ra = m0 + row; ra = ra < M ? ra : M - 1;
      __builtin_amdgcn_global_load_lds(A + ra * rowbytes + off, (lds_t*)&st.a[slot0], 16, 0, 0);
    }
    if (PART < 0 || PART == 4 + i) {
      int64_t rb = n0 + row; rb = rb < N ? rb : N - 1;
      __builtin_amdgcn_global_load_lds(B + rb * rowbytes + off, (lds_t*)&st.b[slot0], 16, 0, 0);
    }
  }
  if (PART >= 0 && PART < 8) return;
  if constexpr (FMT == 0 && SCB) return;  // scales come in blocks (issue_scale_block)
  if constexpr (FMT == 0) {
    // each wave: 64 dwords of A's and 64 of B's area; the dword of a row holds the scale bytes of
    // this 128-K pair of stages (4-byte aligned: K % 128 == 0), the stage uses 2 of them
    const int64_t ng = K / 32;
    const int p = wave * 64 + lane;
    const int row = (p >> 7) * 128 + (p & 3) * 32 + ((p & 127) >> 2);
    int64_t ra = m0 + row; ra = ra < M ? ra : M - 1;
    int64_t rb = n0 + row; rb = rb < N ? rb : N - 1;
    uint32_t* la = reinterpret_cast<uint32_t*>(st.sa) + wave * 64;
    uint32_t* lb = reinterpret_cast<uint32_t*>(st.sb) + wave * 64;
    const int64_t kb = (kt & ~(int64_t)1) * 2;
    if (PART < 0 || PART == 8) __builtin_amdgcn_global_load_lds(SA + ra * ng + kb, (lds_t*)la, 4, 0, 0);
    if (PART < 0 || PART == 9) __builtin_amdgcn_global_load_lds(SB + rb * ng + kb, (lds_t*)lb, 4, 0, 0);
  } else {
    // 64 lanes x 16 B = the stage's two 512-byte tiles of one operand: waves 0-1 load A's, waves
    // 2-3 B's (each pair loads the same bytes to the same place, which keeps every wave's load
    // count per stage equal for the vmcnt bookkeeping)
    const int64_t groups = (K / 32 + 3) / 4;
    const int which = wave >> 1;
    const int tt = lane >> 5, q = lane & 31;
    const int64_t r0 = which ? n0 / 128 : m0 / 128;
    const int64_t nt = which ? (N + 127) / 128 : (M + 127) / 128;
    int64_t tr = r0 + tt; tr = tr < nt ? tr : nt - 1;
    const uint8_t* src = (which ? SB : SA) + (tr * groups + kt) * 512 + q * 16;
    __builtin_amdgcn_global_load_lds(src, (lds_t*)(which ? st.sb : st.sa), 16, 0, 0);
  }
}

// MXFP8 scale block bb (K [512 bb, 512 bb + 512)) of the tile's 256 A rows and 256 B rows: wave w
// loads rows 64w .. 64w+63 of each operand, one row's 16 bytes per lane, into its own 1 KB raw
// areas raw_a / raw_b (lane l's row at byte 16 l). K % 512 == 0 and 16-byte aligned scale matrices
// make every load an aligned 16-byte read inside the row.
__device__ __forceinline__ void issue_scale_block(uint32_t* raw_a, uint32_t* raw_b,
                                                  const uint8_t* __restrict__ SA,
                                                  const uint8_t* __restrict__ SB, int64_t M,
                                                  int64_t N, int64_t K, int64_t m0, int64_t n0,
                                                  int64_t bb, int wave, int lane) {
  const int64_t ng = K / 32;
  const int row = wave * 64 + lane;
  int64_t ra = m0 + row; ra = ra < M ? ra : M - 1;
  int64_t rb = n0 + row; rb = rb < N ? rb : N - 1;
  __builtin_amdgcn_global_load_lds(SA + ra * ng + bb * 16, (lds_t*)raw_a, 16, 0, 0);
  __builtin_amdgcn_global_load_lds(SB + rb * ng + bb * 16, (lds_t*)raw_b, 16, 0, 0);
}

// Rewrites the wave's 64 landed rows of a scale block pair-major: dword j of row r goes to dword
// (r / 128) * 128 + (r % 32) * 4 + (r / 32) % 4 of pair area j, the order of a stage's scale area,
// so that each lane later fetches its four rows' scales with one 16-byte read. Each wave reads
// only the rows it loaded; the writes reach the other waves through the next barrier (the caller
// waits for them first).
__device__ __forceinline__ void transpose_scale_block(const uint32_t* raw_a, const uint32_t* raw_b,
                                                      uint32_t* dst_a, uint32_t* dst_b, int wave,
                                                      int lane) {
  const int r = wave * 64 + lane;
  const int d = (r >> 7) * 128 + (r & 31) * 4 + ((r >> 5) & 3);
  const u32x4 va = reinterpret_cast<const u32x4*>(raw_a)[lane];
  const u32x4 vb = reinterpret_cast<const u32x4*>(raw_b)[lane];
  dst_a[d] = va.x; dst_a[256 + d] = va.y; dst_a[512 + d] = va.z; dst_a[768 + d] = va.w;
  dst_b[d] = vb.x; dst_b[256 + d] = vb.y; dst_b[512 + d] = vb.z; dst_b[768 + d] = vb.w;
}

// s_waitcnt lgkmcnt(0), leaving vmcnt and expcnt unconstrained
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// A wave's operands of one stage, per 32x32 tile i (0-3), and the stage's scale bytes of the
// lane's row for each tile. MXFP8: one 32-byte operand per tile (the lane's halves of the two
// blocks of the single 64-K step); MXFP4: one 16-byte operand per tile and K step.
template <int FMT> struct Frags;
template <> struct Frags<0> {
  i32x8 a[4], b[4];
  uint32_t sa[4], sb[4];
};
template <> struct Frags<1> {
  u32x4 a[2][4], b[2][4];
  uint32_t sa[4], sb[4];
};

__device__ __forceinline__ i32x8 join(u32x4 x, u32x4 y) {
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

// scb_a / scb_b (MXFP8 with scale blocks): the block buffer holding the stage's scales, and j the
// stage pair's index in its block (the dword of each row); null otherwise.
template <int FMT>
__device__ __forceinline__ void read_frags(Frags<FMT>& f, const Stage& s, int wm, int wn, int li, int h,
                                           const uint32_t* scb_a = nullptr,
                                           const uint32_t* scb_b = nullptr, int j = 0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + li;
    const int rb = wn * 128 + i * 32 + li;
    if constexpr (FMT == 0) {
      f.a[i] = join(s.a[chunk_slot(ra, h)], s.a[chunk_slot(ra, 2 + h)]);
      f.b[i] = join(s.b[chunk_slot(rb, h)], s.b[chunk_slot(rb, 2 + h)]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f.a[ks][i] = s.a[chunk_slot(ra, 2 * ks + h)];
        f.b[ks][i] = s.b[chunk_slot(rb, 2 * ks + h)];
      }
    }
  }
  if (FMT == 0 && scb_a) {  // pair area j of the scale block, ordered like a stage's scale area
    const u32x4 va = reinterpret_cast<const u32x4*>(scb_a + 256 * j)[wm * 32 + li];
    const u32x4 vb = reinterpret_cast<const u32x4*>(scb_b + 256 * j)[wn * 32 + li];
    f.sa[0] = va.x; f.sa[1] = va.y; f.sa[2] = va.z; f.sa[3] = va.w;
    f.sb[0] = vb.x; f.sb[1] = vb.y; f.sb[2] = vb.z; f.sb[3] = vb.w;
  } else {  // MXFP8: row dwords in the interleaved order; MXFP4: the 128x4 tiles verbatim. stage_mfma
     // shifts them right by 8h, so that the byte a lane half needs is byte 2*odd (MXFP8) or 2*ks
     // (MXFP4) for both halves and the MFMA's op_sel immediate can pick it.
    const u32x4 va = s.sa[wm * 32 + li];
    const u32x4 vb = s.sb[wn * 32 + li];
    (void)h;
    f.sa[0] = va.x; f.sa[1] = va.y; f.sa[2] = va.z; f.sa[3] = va.w;
    f.sb[0] = vb.x; f.sb[1] = vb.y; f.sb[2] = vb.z; f.sb[3] = vb.w;
  }
}

// MFMA operands of tile i for K-step ks
__device__ __forceinline__ i32x8 op_a(const Frags<0>& f, int i, int) { return f.a[i]; }
__device__ __forceinline__ i32x8 op_b(const Frags<0>& f, int i, int) { return f.b[i]; }
__device__ __forceinline__ i32x8 op_a(const Frags<1>& f, int i, int ks) {
  const u32x4 x = f.a[ks][i];
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};  // e2m1: 4 registers are read
}
__device__ __forceinline__ i32x8 op_b(const Frags<1>& f, int i, int ks) {
  const u32x4 x = f.b[ks][i];
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
}

// One stage of MFMAs from `cur`; the barrier and the read of the next stage into `nxt` are placed
// Cfg::BAR_PAIRS MFMA pairs before the end.
struct LoadArgs {
  const uint8_t* A; const uint8_t* B; const uint8_t* SA; const uint8_t* SB;
  int64_t M, N, K, m0, n0;
  int wave, lane;
};

template <int FMT, int P>
__device__ __forceinline__ void issue_part(Stage& st, int64_t kt, const LoadArgs& l) {
  issue_stage<FMT, P>(st, l.A, l.B, l.SA, l.SB, l.M, l.N, l.K, l.m0, l.n0, kt, l.wave, l.lane);
}

// Scale blocks of MXFP8 (SCB): the next stage's scales come from block buffer (nscb_a, nscb_b),
// pair area nj. Stage 8b issues block b+1 into the waves' raw areas (raw_a, raw_b) (issue_blk,
// block ld_blk); it is older than stage 8b+3's loads, so the wait of stage 8b+1 saw it land.
// Stage 8b+2 rewrites it into buffer (xp_a, xp_b) (xpose) and waits for those writes before its
// barrier; the buffer is block b-1's, whose last read (for stage 8b-1) came before stage 8b-1's
// barrier, and block b+1 is first read for stage 8b+8, after six more barriers. A wave's raw area
// is reloaded only after its own reads of it have returned.
struct ScaleBlocks {
  const uint32_t* nscb_a; const uint32_t* nscb_b; int nj;
  uint32_t* raw_a; uint32_t* raw_b; int64_t ld_blk; bool issue_blk;
  uint32_t* xp_a; uint32_t* xp_b; bool xpose;
};

template <int FMT, int ODD, bool SCB>
__device__ __forceinline__ void stage_mfma(f32x16 (&acc)[4][4], const Frags<FMT>& cur, Frags<FMT>& nxt,
                                           const Stage& next_st, int wm, int wn, int li, int h,
                                           Stage& ld_st, int64_t ld_kt, const LoadArgs& la,
                                           const ScaleBlocks& sb) {
  using C = Cfg<FMT>;
  constexpr int LOADS = kLoads<FMT, SCB>;
  constexpr int PAIRS = 8 * C::KSTEPS;
  constexpr int WP = PAIRS - C::BAR_PAIRS;
  constexpr int EXTRA = LOADS > PAIRS ? LOADS - PAIRS : 0;             // loads doubled up on pairs 0..
  constexpr int ISSUED = WP + (EXTRA < WP ? EXTRA : WP);               // this stage's loads before WP
  uint32_t ssa[4], ssb[4];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) {
    if (p == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { ssa[i] = cur.sa[i] >> (8 * h); ssb[i] = cur.sb[i] >> (8 * h); }
      if (SCB && sb.issue_blk)
        issue_scale_block(sb.raw_a, sb.raw_b, la.SA, la.SB, la.M, la.N, la.K, la.m0, la.n0,
                          sb.ld_blk, la.wave, la.lane);
      if (SCB && sb.xpose) transpose_scale_block(sb.raw_a, sb.raw_b, sb.xp_a, sb.xp_b, la.wave, la.lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (p == WP) {
      // stage kt+1 landed; kt+2 and part of kt+3 may be in flight (a scale block issued this stage
      // only makes the wait stricter)
      wait_vmcnt<LOADS + ISSUED>();
      if (SCB && sb.xpose) wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
      if (SCB) read_frags<FMT>(nxt, next_st, wm, wn, li, h, sb.nscb_a, sb.nscb_b, sb.nj);
      else read_frags<FMT>(nxt, next_st, wm, wn, li, h);
    }
    const int ks = p >> 3, q = p & 7;
    const int n = q >> 1, m0 = 2 * (q & 1);
    constexpr int SEL0 = FMT == 0 ? 2 * ODD : 0;  // scale byte (of the 8h-shifted dword)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int m = m0 + mm;
      if (ks == 0)
        acc[n][m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            op_b(cur, n, 0), op_a(cur, m, 0), acc[n][m], C::CODE, C::CODE, SEL0, (int)ssb[n], SEL0,
            (int)ssa[m]);
      else
        acc[n][m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            op_b(cur, n, 1), op_a(cur, m, 1), acc[n][m], C::CODE, C::CODE, 2, (int)ssb[n], 2,
            (int)ssa[m]);
    }
    // one load of stage kt+3 after each MFMA pair (two on the first pairs when there are more
    // loads than pairs)
    if (p < LOADS) {
      if (p == 0) issue_part<FMT, 0>(ld_st, ld_kt, la);
      if (p == 1) issue_part<FMT, 1>(ld_st, ld_kt, la);
      if (p == 2) issue_part<FMT, 2>(ld_st, ld_kt, la);
      if (p == 3) issue_part<FMT, 3>(ld_st, ld_kt, la);
      if (p == 4) issue_part<FMT, 4>(ld_st, ld_kt, la);
      if (p == 5) issue_part<FMT, 5>(ld_st, ld_kt, la);
      if (p == 6) issue_part<FMT, 6>(ld_st, ld_kt, la);
      if (p == 7) issue_part<FMT, 7>(ld_st, ld_kt, la);
      if (p == 8) issue_part<FMT, 8>(ld_st, ld_kt, la);
    }
    if (p < EXTRA) {
      if (p == 0) issue_part<FMT, 8>(ld_st, ld_kt, la);
      if (p == 1) issue_part<FMT, 9>(ld_st, ld_kt, la);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int FMT, bool OUT_F32, int BIAS, bool SCB>
__global__ __launch_bounds__(256, 1) void mm_mx_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ alpha_ptr, int64_t M, int64_t N,
    int64_t K, void* __restrict__ out, int64_t ldc, int ntm, int ntn, bool vec_store,
    const void* __restrict__ bias) {
  using C = Cfg<FMT>;
  constexpr int LOADS = kLoads<FMT, SCB>;
  __shared__ Stage st[NSTAGE];
  __shared__ uint32_t scb[SCB ? 2 : 1][2][SCB ? kScbDwords : 1];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;
  int tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t nk = K / C::BK;
  const int64_t last = nk - 1;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Stage kt goes to buffer kt % 4, three stages ahead; past the end the last stage is re-loaded
  // into buffers nobody reads again, so every stage issues and waits for the same loads.
  // SCB: a wave's raw scale-block rows sit in the scale area of stage slot `wave` (unused then)
  uint32_t* const raw_a = reinterpret_cast<uint32_t*>(st[wave].sa);
  uint32_t* const raw_b = reinterpret_cast<uint32_t*>(st[wave].sb);
  if constexpr (SCB) issue_scale_block(raw_a, raw_b, SA, SB, M, N, K, m0, n0, 0, wave, lane);
  issue_stage<FMT, -1, SCB>(st[0], A, B, SA, SB, M, N, K, m0, n0, 0, wave, lane);
  issue_stage<FMT, -1, SCB>(st[1], A, B, SA, SB, M, N, K, m0, n0, last < 1 ? last : 1, wave, lane);
  issue_stage<FMT, -1, SCB>(st[2], A, B, SA, SB, M, N, K, m0, n0, last < 2 ? last : 2, wave, lane);
  wait_vmcnt<2 * LOADS>();   // stage 0 (and scale block 0, issued before it) landed
  if constexpr (SCB) {
    transpose_scale_block(raw_a, raw_b, scb[0][0], scb[0][1], wave, lane);
    wait_lgkmcnt0();
  }
  __builtin_amdgcn_s_barrier();
  Frags<FMT> f0, f1;
  if constexpr (SCB) read_frags<FMT>(f0, st[0], wm, wn, li, h, scb[0][0], scb[0][1], 0);
  else read_frags<FMT>(f0, st[0], wm, wn, li, h);
  const int64_t nblk = K / 512;  // scale blocks (SCB: K % 512 == 0)
  // the scale-block arguments of stage kt (next stage kt + 1; BK = 64, so pair = stage / 2)
  auto blocks = [&](int64_t kt) -> ScaleBlocks {
    ScaleBlocks b{nullptr, nullptr, 0, nullptr, nullptr, 0, false, nullptr, nullptr, false};
    if constexpr (SCB) {
      const int64_t np = (kt + 1) >> 1, nb = np >> 2;
      b.nscb_a = scb[nb & 1][0]; b.nscb_b = scb[nb & 1][1]; b.nj = (int)(np & 3);
      b.raw_a = raw_a; b.raw_b = raw_b;
      b.ld_blk = kt / 8 + 1 < nblk ? kt / 8 + 1 : nblk - 1;  // the last block reloads itself
      b.issue_blk = (kt & 7) == 0;
      b.xp_a = scb[(kt / 8 + 1) & 1][0]; b.xp_b = scb[(kt / 8 + 1) & 1][1];
      b.xpose = (kt & 7) == 2;
    }
    return b;
  };

  // Stages in pairs so that the two fragment sets swap roles without a register copy; an odd
  // last stage is peeled after the loop (a branch inside the loop makes the compiler spill).
  // Buffer reuse: stage kt+3's loads (issued at stage kt) overwrite the buffer of stage kt-1, whose
  // fragments were read before stage kt-1's barrier, which every wave has passed.
  const LoadArgs la{A, B, SA, SB, M, N, K, m0, n0, wave, lane};
  const int64_t pairs = nk / 2;
  for (int64_t pi = 0; pi < pairs; ++pi) {
    const int64_t kt = 2 * pi;
    stage_mfma<FMT, 0, SCB>(acc, f0, f1, st[(kt + 1) % NSTAGE], wm, wn, li, h, st[(kt + 3) % NSTAGE],
                            kt + 3 < last ? kt + 3 : last, la, blocks(kt));
    stage_mfma<FMT, 1, SCB>(acc, f1, f0, st[(kt + 2) % NSTAGE], wm, wn, li, h, st[(kt + 4) % NSTAGE],
                            kt + 4 < last ? kt + 4 : last, la, blocks(kt + 1));
  }
  if (nk & 1) {
    const int64_t kt = nk - 1;  // even (never with SCB: nk = K / 64 is a multiple of 8)
    stage_mfma<FMT, 0, SCB>(acc, f0, f1, st[(kt + 1) % NSTAGE], wm, wn, li, h, st[(kt + 3) % NSTAGE],
                            last, la, blocks(kt));
  }
  wait_vmcnt<0>();
  const float a = alpha_ptr ? *alpha_ptr : 1.0f;
  const float alpha[4] = {a, a, a, a};
  static_assert(sizeof(st) >= 4 * kEpiWaveBytes, "epilogue images overlay the stage buffers");
  store_tile<OUT_F32, BIAS, false>(acc, alpha, m0, n0, wm, wn, M, N, out, ldc, vec_store,
                            reinterpret_cast<uint8_t*>(st), wave, lane, li, h, bias);
}

template <int FMT, int BIAS = kBiasNone>
int launch(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
           const float* alpha, int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
           hipStream_t s, const char* name, const void* bias = nullptr) {
  const int64_t ntm = ceil_div(M, BM), ntn = ceil_div(N, BN);
  const int64_t tiles = ntm * ntn;
  const size_t esz = out_dtype == BSP_OUT_F32 ? 4 : 2;
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & (4 * esz - 1)) == 0);
  // MXFP8 scale blocks need 16-byte reads inside each scale row
  const bool scb = FMT == 0 && K % 512 == 0 &&
                   ((reinterpret_cast<uintptr_t>(sa) | reinterpret_cast<uintptr_t>(sb)) & 15) == 0;
  if (out_dtype == BSP_OUT_F32 && scb)
    hipLaunchKernelGGL((mm_mx_kernel<FMT, true, BIAS, FMT == 0>), dim3((unsigned)tiles), dim3(256), 0, s,
                       a, sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  else if (out_dtype == BSP_OUT_F32)
    hipLaunchKernelGGL((mm_mx_kernel<FMT, true, BIAS, false>), dim3((unsigned)tiles), dim3(256), 0, s,
                       a, sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  else if (scb)
    hipLaunchKernelGGL((mm_mx_kernel<FMT, false, BIAS, FMT == 0>), dim3((unsigned)tiles), dim3(256), 0, s,
                       a, sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  else
    hipLaunchKernelGGL((mm_mx_kernel<FMT, false, BIAS, false>), dim3((unsigned)tiles), dim3(256), 0, s,
                       a, sa, b, sb, alpha, M, N, K, out, ldc, (int)ntm, (int)ntn, vec, bias);
  return check_launch(name);
}

}  // namespace mx
}  // namespace bsp

using namespace bsp;

// bias_align: 0 for the entry points without a bias, else the bias element size (its alignment)
static int mx_checks(const char* fn, const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                     const uint8_t* b_sf, int64_t M, int64_t N, int64_t K, void* out, int64_t ldc,
                     int out_dtype, int64_t kmult, int sf_align, const void* bias = nullptr,
                     unsigned bias_align = 0) {
  BSP_REQUIRE(M >= 0 && N >= 0 && K > 0, BSP_EINVAL, "%s: bad size M=%lld N=%lld K=%lld", fn,
              (long long)M, (long long)N, (long long)K);
  BSP_REQUIRE(out_dtype == BSP_OUT_BF16 || out_dtype == BSP_OUT_F32, BSP_EDTYPE,
              "%s: out_dtype must be BSP_OUT_BF16 (0) or BSP_OUT_F32 (1), got %d", fn, out_dtype);
  BSP_REQUIRE(K % kmult == 0, BSP_ESHAPE, "%s: K (%lld) must be a multiple of %lld", fn, (long long)K,
              (long long)kmult);
  BSP_REQUIRE(M <= 1 || ldc >= N, BSP_ESHAPE, "%s: ldc (%lld) < N (%lld)", fn, (long long)ldc, (long long)N);
  if (M == 0 || N == 0) return 1;
  BSP_REQUIRE(a && a_sf && b && b_sf && out, BSP_EINVAL, "%s: null pointer", fn);
  BSP_REQUIRE(((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) == 0 &&
                  ((reinterpret_cast<uintptr_t>(a_sf) | reinterpret_cast<uintptr_t>(b_sf)) & (sf_align - 1)) == 0,
              BSP_EINVAL, "%s: operands must be 16-byte and scales %d-byte aligned", fn, sf_align);
  BSP_REQUIRE(ceil_div(M, 256) * ceil_div(N, 256) < (1ll << 31), BSP_ESHAPE, "%s: too many tiles", fn);
  BSP_REQUIRE(bias_align == 0 || (bias && (reinterpret_cast<uintptr_t>(bias) & (bias_align - 1)) == 0),
              BSP_EINVAL, "%s: bias must be a non-null device pointer aligned to its element size", fn);
  if (int e = check_device()) return e;
  return 0;
}

extern "C" int bsp_mm_mxfp8(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                            const uint8_t* b_sf, int64_t M, int64_t N, int64_t K, void* out,
                            int64_t ldc, int out_dtype, void* stream) {
  int e = mx_checks("bsp_mm_mxfp8", a, a_sf, b, b_sf, M, N, K, out, ldc, out_dtype, 128, 4);
  if (e) return e > 0 ? BSP_OK : e;
  return mx::launch<0>(a, a_sf, b, b_sf, nullptr, M, N, K, out, ldc, out_dtype, (hipStream_t)stream,
                       "bsp_mm_mxfp8");
}

extern "C" int bsp_mm_mxfp4(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                            const uint8_t* b_sf, const float* alpha_dev, int64_t M, int64_t N,
                            int64_t K, void* out, int64_t ldc, int out_dtype, void* stream) {
  int e = mx_checks("bsp_mm_mxfp4", a, a_sf, b, b_sf, M, N, K, out, ldc, out_dtype, 128, 16);
  if (e) return e > 0 ? BSP_OK : e;
  return mx::launch<1>(a, a_sf, b, b_sf, alpha_dev, M, N, K, out, ldc, out_dtype, (hipStream_t)stream,
                       "bsp_mm_mxfp4");
}

extern "C" int bsp_mm_mxfp8_bias(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                                 const uint8_t* b_sf, const float* bias_f32, int64_t M, int64_t N,
                                 int64_t K, void* out, int64_t ldc, int out_dtype, void* stream) {
  int e = mx_checks("bsp_mm_mxfp8_bias", a, a_sf, b, b_sf, M, N, K, out, ldc, out_dtype, 128, 4,
                    bias_f32, 4);
  if (e) return e > 0 ? BSP_OK : e;
  return mx::launch<0, kBiasF32Before>(a, a_sf, b, b_sf, nullptr, M, N, K, out, ldc, out_dtype,
                                       (hipStream_t)stream, "bsp_mm_mxfp8_bias", bias_f32);
}

extern "C" int bsp_mm_mxfp4_bias(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b,
                                 const uint8_t* b_sf, const float* alpha_dev, const void* bias_bf16,
                                 int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
                                 void* stream) {
  int e = mx_checks("bsp_mm_mxfp4_bias", a, a_sf, b, b_sf, M, N, K, out, ldc, out_dtype, 128, 16,
                    bias_bf16, 2);
  if (e) return e > 0 ? BSP_OK : e;
  return mx::launch<1, kBiasBf16After>(a, a_sf, b, b_sf, alpha_dev, M, N, K, out, ldc, out_dtype,
                                       (hipStream_t)stream, "bsp_mm_mxfp4_bias", bias_bf16);
}
