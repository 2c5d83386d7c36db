// Device queries used by the C ABI (HIP runtime, host side only).
#include <hip/hip_runtime_api.h>

#include <mutex>
#include <string>

#include "seer_internal.h"

namespace seer {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
int g_cus[kMaxDevices] = {0};
}  // namespace

int device_cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(std::string("hipGetDevice: ") + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device ordinal out of range");
    return SEER_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_cus[dev] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus <= 0) {
      set_error(std::string("hipDeviceGetAttribute(CU count): ") + hipGetErrorString(e));
      return SEER_ERR_HIP;
    }
    g_cus[dev] = cus;
  }
  *out = g_cus[dev];
  return SEER_OK;
}

}  // namespace seer
