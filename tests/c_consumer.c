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
  printf("c consumer ok\n");
  return 0;
}
