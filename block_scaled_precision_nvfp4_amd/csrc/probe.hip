// Measured-achievable ceilings of this chip, for reading the kernels' roofline fractions: an
// MFMA-only loop per matrix-core format (the instruction each GEMM issues, with operands like the
// GEMM's) and streaming kernels with the quantizers' read:write mix. Built into libbsp_probe.so,
// which only the benchmark loads; nothing in the linear-layer path calls it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/bsp_probe.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {  // a 32-bit integer hash (xorshift-multiply)
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}

// f16 operand holding e2m1 value * e4m3 scale * 2^-8, as mm_fp4 feeds its MFMA: the value's
// magnitude index and sign and the scale's code come from the hash.
__device__ __forceinline__ _Float16 nvfp4_like_f16(uint32_t h) {
  const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const uint32_t sc = 0x20u + ((h >> 4) & 0x3Fu);                 // e4m3 codes 0x20 .. 0x5F
  const float s = __uint_as_float(((sc >> 3) + 120u) << 23 | (sc & 7u) << 20);
  const float v = grid[h & 7u] * s * 0.00390625f;
  return (_Float16)((h & 8u) ? -v : v);
}

// FMT 0: v_mfma_f32_32x32x16_f16 on NVFP4-like fp16 operands (mm_fp4's instruction);
// FMT 1: v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 operands (mm_mxfp8's);
// FMT 2: the same with e2m1 operands (mm_mxfp4's);
// FMT 3: v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 operands (the fp8 shape this chip runs fastest).
// kChains independent accumulator chains per wave: with four, the 32-cycle instructions (FMT 0
// and 2) kept the matrix core only about 77 % busy; with eight it stays busy at one wave per SIMD,
// as in the GEMMs.
constexpr int kChains = 8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int FMT>
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int iters, uint32_t seed) {
  const uint32_t base = mix(seed ^ (blockIdx.x * 256u + threadIdx.x));
  typedef typename std::conditional<FMT == 3, f32x4, f32x16>::type acc_t;
  constexpr int kAccN = FMT == 3 ? 4 : 16;
  acc_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = acc_t{};
  if constexpr (FMT == 0) {
    f16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[i][e] = nvfp4_like_f16(mix(base + 16u * i + e));
        b[i][e] = nvfp4_like_f16(mix(base + 977u + 16u * i + e));
      }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c & 1], b[(c >> 1) & 1], acc[c], 0, 0, 0);
    }
  } else {
    i32x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t x = mix(base + 16u * i + e), y = mix(base + 977u + 16u * i + e);
        if (FMT != 2) {  // no e4m3 NaN bytes (0x7F / 0xFF): flip their lowest bit
#pragma unroll
          for (int j = 0; j < 32; j += 8) {
            if (((x >> j) & 0x7Fu) == 0x7Fu) x ^= 1u << j;
            if (((y >> j) & 0x7Fu) == 0x7Fu) y ^= 1u << j;
          }
        }
        a[i][e] = (int)x;
        b[i][e] = (int)y;
      }
    constexpr int code = FMT == 2 ? 4 : 0;
    const int sa = 0x7F7F7F7F, sb = 0x7E7E7E7E;  // e8m0 scales 1 and 1/2
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        if constexpr (FMT == 3)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[c & 1], b[(c >> 1) & 1], acc[c],
                                                                    code, code, 0, sa, 0, sb);
        else
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c & 1], b[(c >> 1) & 1], acc[c],
                                                                   code, code, 0, sa, 0, sb);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < kAccN; ++e) s += acc[c][e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));

// Streaming over n16 16-byte chunks with sixteen loads in flight per thread (as many as the
// quantizers keep), nontemporal as their loads and stores are. WRITE_DIV 0: read only (one word per
// thread written at the end); 1: copy; 4: a quarter of the bytes read are written (about the NVFP4
// quantize's 2 : 0.56).
constexpr int kInFlight = 16;
template <int WRITE_DIV>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ src,
                                                     uint32_t* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    nt_u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(src) + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      if (WRITE_DIV == 1) {
        __builtin_nontemporal_store(v[u], reinterpret_cast<nt_u32x4*>(dst) + i + u * stride);
      } else if (WRITE_DIV == 4) {
        __builtin_nontemporal_store(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w, dst + i + u * stride);
      } else {
        x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      }
    }
  }
  for (; i < n16; i += stride) {
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(src) + i);
    if (WRITE_DIV == 1) __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4*>(dst) + i);
    else if (WRITE_DIV == 4) __builtin_nontemporal_store(v.x ^ v.y ^ v.z ^ v.w, dst + i);
    else x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (WRITE_DIV == 0) dst[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace

extern "C" int bsp_probe_mfma_loop(int fmt, int workgroups, int iters, float* out, void* stream) {
  if (fmt < 0 || fmt > 3 || workgroups <= 0 || iters <= 0 || !out) return -1;
  const dim3 g(workgroups), b(256);
  hipStream_t s = (hipStream_t)stream;
  if (fmt == 0) hipLaunchKernelGGL(mfma_loop_kernel<0>, g, b, 0, s, out, iters, 12345u);
  else if (fmt == 1) hipLaunchKernelGGL(mfma_loop_kernel<1>, g, b, 0, s, out, iters, 12345u);
  else if (fmt == 2) hipLaunchKernelGGL(mfma_loop_kernel<2>, g, b, 0, s, out, iters, 12345u);
  else hipLaunchKernelGGL(mfma_loop_kernel<3>, g, b, 0, s, out, iters, 12345u);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bsp_probe_stream(int write_div, const void* src, void* dst, int64_t n16, int workgroups,
                                void* stream) {
  if (!(write_div == 0 || write_div == 1 || write_div == 4) || !src || !dst || n16 <= 0 ||
      workgroups <= 0 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
    return -1;
  const dim3 g(workgroups), b(256);
  hipStream_t s = (hipStream_t)stream;
  const u32x4* p = static_cast<const u32x4*>(src);
  uint32_t* q = static_cast<uint32_t*>(dst);
  if (write_div == 0) hipLaunchKernelGGL(stream_kernel<0>, g, b, 0, s, p, q, n16);
  else if (write_div == 1) hipLaunchKernelGGL(stream_kernel<1>, g, b, 0, s, p, q, n16);
  else hipLaunchKernelGGL(stream_kernel<4>, g, b, 0, s, p, q, n16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
