/* libbsp_probe: measured-achievable ceilings of the GPU, used by the benchmark to report each
 * kernel's fraction of what this chip sustains beside its fraction of the published peaks.
 * Not part of the linear-layer path. All calls enqueue on `stream` (a hipStream_t, or NULL) and
 * return 0, -1 for bad arguments, or -5 when the launch fails. */
#ifndef BSP_PROBE_H
#define BSP_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA-only loop: `workgroups` workgroups of 256 threads, each wave issuing `iters` x 8 independent
 * matrix instructions (eight accumulator chains) on register operands, with no memory traffic but
 * the final store:
 *   fmt 0: v_mfma_f32_32x32x16_f16 (32768 flops each) on fp16 values of the form e2m1 x e4m3 x 2^-8,
 *          the operands mm_fp4 multiplies;
 *   fmt 1: v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 operands (131072 flops), mm_mxfp8's;
 *   fmt 2: the same with e2m1 operands, mm_mxfp4's;
 *   fmt 3: v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 operands (65536 flops).
 * out: device fp32 [workgroups * 256], one value per thread (keeps the loop from being removed). */
int bsp_probe_mfma_loop(int fmt, int workgroups, int iters, float* out, void* stream);

/* Streaming over n16 16-byte chunks of src (16-byte aligned device memory) with nontemporal loads
 * and stores, sixteen loads in flight per thread, grid-stride over `workgroups` x 256 threads:
 *   write_div 0: read only; dst receives one uint32 per thread (workgroups * 256 * 4 bytes);
 *   write_div 1: copy, dst holds n16 * 16 bytes;
 *   write_div 4: one uint32 written per chunk read (read:write 4:1, near the NVFP4 quantize's
 *                2 : 0.56 per element), dst holds n16 * 4 bytes. */
int bsp_probe_stream(int write_div, const void* src, void* dst, int64_t n16, int workgroups,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSP_PROBE_H */
