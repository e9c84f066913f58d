/* A plain C99 consumer of the library: compiles against include/bsp.h alone and links libbsp.so.
 * It exercises only host-side paths (queries and argument validation), so it runs without a GPU.
 * Exit status 0 and the line "c consumer ok" mean every check held. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bsp.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  int64_t bytes = -1;
  CHECK(bsp_version() == 100);
  CHECK(bsp_nvfp4_sf_bytes(32760, 5120, &bytes) == BSP_OK && bytes == 32768LL * 320);
  CHECK(bsp_nvfp4_sf_bytes_8x4(13, 80, &bytes) == BSP_OK && bytes == 16LL * 8);
  CHECK(bsp_mxfp4_sf_bytes(1, 32, &bytes) == BSP_OK && bytes == 128LL * 4);
  CHECK(bsp_nvfp4_sf_bytes(-1, 16, &bytes) == BSP_EINVAL);
  CHECK(strlen(bsp_last_error()) > 0);

  /* validation happens on the host before anything is launched */
  void* p = (void*)(uintptr_t)16;
  CHECK(bsp_nvfp4_quantize(p, 4, 24, 24, (const float*)p, (uint8_t*)p, (uint8_t*)p, NULL) == BSP_ESHAPE);
  CHECK(strstr(bsp_last_error(), "multiple of 16") != NULL);
  CHECK(bsp_nvfp4_quantize(NULL, 0, 32, 32, NULL, NULL, NULL, NULL) == BSP_OK);  /* M == 0: no-op */
  CHECK(bsp_mm_fp4((const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p,
                   (const float*)p, 8, 8, 96, p, 8, BSP_OUT_BF16, NULL) == BSP_ESHAPE);
  CHECK(bsp_mm_fp4((const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p,
                   (const float*)p, 8, 8, 128, p, 8, 7, NULL) == BSP_EDTYPE);
  CHECK(bsp_mm_mxfp8((const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, 8, 8, 64,
                     p, 8, BSP_OUT_BF16, NULL) == BSP_ESHAPE);
  CHECK(bsp_nvfp4_alpha(NULL, (const float*)p, (float*)p, NULL) == BSP_EINVAL);
  /* the norm + quantize prologue: eps must be positive and finite, K a multiple of 16 */
  CHECK(bsp_rmsnorm_bf16(p, 4, 32, 32, NULL, 0.0f, p, 32, NULL) == BSP_EINVAL);
  CHECK(bsp_rmsnorm_bf16(p, 4, 24, 24, NULL, 1e-6f, p, 24, NULL) == BSP_ESHAPE);
  CHECK(bsp_nvfp4_quantize_rmsnorm(p, 4, 32, 32, NULL, 1e-6f, (const float*)p, NULL, (uint8_t*)p, NULL) ==
        BSP_EINVAL);
  CHECK(bsp_nvfp4_quantize_rmsnorm(NULL, 0, 32, 32, NULL, 1e-6f, NULL, NULL, NULL, NULL) == BSP_OK);
  /* one row-tile past the quantizer's grid limit */
  CHECK(bsp_nvfp4_quantize(p, 65535LL * 128 + 1, 32, 32, (const float*)p, (uint8_t*)p, (uint8_t*)p, NULL) ==
        BSP_ESHAPE);
  /* the fragment layouts: sizes, and K rules checked before a launch */
  int64_t sfb = -1;
  CHECK(bsp_nvfp4_frag_bytes(33, 192, &bytes) == BSP_OK && bytes == 64LL * 96);
  CHECK(bsp_nvfp4_frag_bytes(4, 96, &bytes) == BSP_ESHAPE);
  CHECK(bsp_mxfp4_frag_bytes(33, 512, &bytes, &sfb) == BSP_OK && bytes == 64LL * 256 && sfb == 64LL * 16);
  CHECK(bsp_mxfp8_frag_bytes(33, 512, &bytes, &sfb) == BSP_OK && bytes == 64LL * 512 && sfb == 64LL * 16);
  CHECK(bsp_nvfp4_quantize_frag(p, 4, 96, 96, (const float*)p, (uint8_t*)p, (uint8_t*)p, NULL) == BSP_ESHAPE);
  CHECK(bsp_mm_fp4_frag((const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p,
                        (const float*)p, NULL, 8, 8, 96, p, 8, BSP_OUT_BF16, NULL) == BSP_ESHAPE);
  CHECK(bsp_mm_fp4_frag((const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p,
                        (const float*)p, NULL, 8, 8, (1LL << 24) + 64, p, 8, BSP_OUT_BF16, NULL) == BSP_ESHAPE);
  CHECK(bsp_mm_mxfp4_frag((const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, NULL,
                          NULL, 8, 8, 384, p, 8, BSP_OUT_BF16, NULL) == BSP_ESHAPE);
  CHECK(bsp_mm_mxfp8_frag((const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p, NULL,
                          8, 8, 384, p, 8, BSP_OUT_BF16, NULL) == BSP_ESHAPE);
  CHECK(bsp_mm_fp4_frag(NULL, NULL, NULL, NULL, NULL, NULL, 0, 8, 64, NULL, 8, BSP_OUT_BF16, NULL) ==
        BSP_OK);  /* M == 0: no-op */
  printf("c consumer ok\n");
  return 0;
}
