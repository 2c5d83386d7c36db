// seer_decode_step_noalloc: the fused decode step with its workspace in a
// static device array of the library instead of a caller's buffer, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds one copy of the array until the process
// ends.  Host code never passes the array's name to a kernel or a copy: in
// host code that name is a stand-in, not a device address.  The device
// address is taken once per device with hipGetSymbolAddress, with that device
// current, and kept in a per-device table.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "seer_internal.h"

static __device__ __align__(256) unsigned char scratch[seer::kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {nullptr};  // device address of `scratch` per device

int hip_fail(const char* what, hipError_t e) {
  seer::set_error(std::string(what) + ": " + hipGetErrorString(e));
  return SEER_ERR_HIP;
}

// The current device's scratch address, taken on the first call on that
// device (with it current) and kept.  Nothing in the array needs particular
// contents: the step's gate launch zeroes the decode's split counters.
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) {
    seer::set_error("device ordinal out of range");
    return SEER_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return hip_fail("hipGetSymbolAddress(scratch)", e);
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SEER_OK;
}

}  // namespace

extern "C" int seer_decode_step_noalloc(
    const seer_dims* dims, const uint16_t* q_nope, const uint16_t* q, const uint16_t* k_nope,
    const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* w_q, const uint16_t* w_k,
    const int32_t* seq_lens, int32_t* kcomp_lens, uint16_t* kcomp, int32_t max_new_blocks,
    double rope_theta, int32_t mode, int32_t topk_blocks, float threshold, int32_t max_selected,
    int32_t* block_idx, int32_t* num_selected, float* logits, float scale, int32_t num_split,
    uint16_t* out, float* lse, void* stream) {
  // the workspace seer_decode_step would be given by a caller sizing it with
  // seer_decode_step_workspace_bytes (0: invalid arguments, which the step
  // itself then reports before any launch)
  const size_t need = seer_decode_step_workspace_bytes(dims, max_selected, num_split);
  if (need == 0)
    return seer_decode_step(dims, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                            kcomp_lens, kcomp, max_new_blocks, rope_theta, mode, topk_blocks,
                            threshold, max_selected, block_idx, num_selected, logits, scale,
                            num_split, nullptr, 0, out, lse, stream);
  if (need > seer::kNoAllocScratchBytes) {
    seer::set_error("seer_decode_step_noalloc: this step needs a " + std::to_string(need) +
                    "-byte workspace; the static scratch holds " +
                    std::to_string(seer::kNoAllocScratchBytes) +
                    " bytes (use seer_decode_step with a workspace, or fewer splits)");
    return SEER_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const int rc = scratch_for_current_device(&ws);
  if (rc != SEER_OK) return rc;
  return seer_decode_step(dims, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                          kcomp_lens, kcomp, max_new_blocks, rope_theta, mode, topk_blocks,
                          threshold, max_selected, block_idx, num_selected, logits, scale,
                          num_split, ws, need, out, lse, stream);
}
