// Library-wide C ABI: error text, version, size queries and the gfx950 device check.
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace bsp {

std::string& last_error_slot() {
  static thread_local std::string msg;
  return msg;
}

// The kernels use gfx950-only instructions (v_cvt_scalef32_*, v_mfma_*_f8f6f4, 32x32x16 f16 MFMA).
int check_device() {
  static std::mutex mu;
  static std::vector<int> state;  // per device: 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BSP_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if ((int)state.size() <= dev) state.resize(dev + 1, 0);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(BSP_EHIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (state[dev] < 0) last_error_slot() = std::string("device is ") + prop.gcnArchName + ", not gfx950";
  }
  if (state[dev] < 0) return fail(BSP_EUNSUPPORTED, "libbsp needs a gfx950 (MI355X) device");
  return BSP_OK;
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cus;  // per device: 0 unknown
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cus.size() <= dev) cus.resize(dev + 1, 0);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace bsp

extern "C" const char* bsp_last_error(void) { return bsp::last_error_slot().c_str(); }

extern "C" int bsp_version(void) { return 100; }

extern "C" int bsp_nvfp4_sf_bytes(int64_t rows, int64_t K, int64_t* bytes) {
  BSP_REQUIRE(bytes, BSP_EINVAL, "bsp_nvfp4_sf_bytes: null output pointer");
  BSP_REQUIRE(rows >= 0 && K >= 0, BSP_EINVAL, "bsp_nvfp4_sf_bytes: negative size");
  *bytes = bsp::ceil_div(rows, 128) * 128 * bsp::ceil_div(K, 64) * 4;
  return BSP_OK;
}

extern "C" int bsp_nvfp4_sf_bytes_8x4(int64_t rows, int64_t K, int64_t* bytes) {
  BSP_REQUIRE(bytes, BSP_EINVAL, "bsp_nvfp4_sf_bytes_8x4: null output pointer");
  BSP_REQUIRE(rows >= 0 && K >= 0, BSP_EINVAL, "bsp_nvfp4_sf_bytes_8x4: negative size");
  *bytes = bsp::ceil_div(rows, 8) * 8 * bsp::ceil_div(K, 64) * 4;
  return BSP_OK;
}
