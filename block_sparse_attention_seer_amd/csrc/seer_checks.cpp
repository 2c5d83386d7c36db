// Argument checks, workspace sizes and error strings of the C ABI.
// Deliberately free of HIP so that it builds and runs on a CPU-only host.

#include <cstdint>
#include <cstring>
#include <string>

#include "seer_internal.h"

namespace seer {

namespace {
thread_local std::string g_last_error;

bool one_of(int v, int a, int b) { return v == a || v == b; }
}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }
const char* last_error() { return g_last_error.c_str(); }

int check_ptr(const void* p, size_t align, const char* name, std::string* why) {
  if (p == nullptr) {
    *why = std::string(name) + " is NULL";
    return SEER_ERR_INVALID_ARG;
  }
  if (reinterpret_cast<uintptr_t>(p) % align != 0) {
    *why = std::string(name) + " is not " + std::to_string(align) + "-byte aligned";
    return SEER_ERR_INVALID_ARG;
  }
  return SEER_OK;
}

int check_dims(const seer_dims* d, std::string* why) {
  if (d == nullptr) {
    *why = "dims is NULL";
    return SEER_ERR_INVALID_ARG;
  }
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->max_seq_len < 1) {
    *why = "batch, num_q_heads, num_kv_heads and max_seq_len must be >= 1";
    return SEER_ERR_INVALID_ARG;
  }
  if (d->reserved != 0) {
    *why = "dims.reserved must be 0";
    return SEER_ERR_INVALID_ARG;
  }
  if (d->num_q_heads % d->num_kv_heads != 0) {
    *why = "num_q_heads must be a multiple of num_kv_heads";
    return SEER_ERR_INVALID_ARG;
  }
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g > kMaxGroup) {
    *why = "group size num_q_heads/num_kv_heads above 16 is not supported";
    return SEER_ERR_UNSUPPORTED;
  }
  if (!one_of(d->head_dim, 64, 128)) {
    *why = "head_dim must be 64 or 128";
    return SEER_ERR_UNSUPPORTED;
  }
  if (!one_of(d->d_gate, 64, 128)) {
    *why = "d_gate must be 64 or 128";
    return SEER_ERR_UNSUPPORTED;
  }
  if (!one_of(d->block_size, 64, 128)) {
    *why = "block_size must be 64 or 128";
    return SEER_ERR_UNSUPPORTED;
  }
  if (d->kv_stride_t < d->head_dim || d->kv_stride_h < 0 || d->kv_stride_b < 0) {
    *why = "kv strides must be non-negative and kv_stride_t >= head_dim";
    return SEER_ERR_INVALID_ARG;
  }
  if ((d->kv_stride_t % 8) || (d->kv_stride_h % 8) || (d->kv_stride_b % 8)) {
    *why = "kv strides must be multiples of 8 elements (16-byte rows)";
    return SEER_ERR_INVALID_ARG;
  }
  // Every (sequence, head) slab must fit the 32-bit token offsets the
  // kernels use inside one slab.
  if (static_cast<int64_t>(d->max_seq_len) * d->kv_stride_t > (int64_t(1) << 31) - 1024) {
    *why = "max_seq_len * kv_stride_t exceeds 2^31 elements";
    return SEER_ERR_UNSUPPORTED;
  }
  return SEER_OK;
}

int check_kv(const seer_dims* d, const void* k, const char* name, std::string* why) {
  (void)d;
  return check_ptr(k, 16, name, why);
}

int64_t nb_max(const seer_dims* d) {
  return (static_cast<int64_t>(d->max_seq_len) + d->block_size - 1) / d->block_size;
}

size_t gate_workspace_bytes(const seer_dims* d) {
  return static_cast<size_t>(d->batch) * d->num_kv_heads * d->d_gate * sizeof(float);
}

size_t step_gate_bytes(const seer_dims* d) {
  return (gate_workspace_bytes(d) + kCounterBytes - 1) / kCounterBytes * kCounterBytes;
}

size_t decode_workspace_bytes(int64_t pairs, int num_split, int g, int head_dim) {
  if (num_split <= 1) return 0;  // a single split writes the output directly
  size_t counters = static_cast<size_t>(pairs) * sizeof(int32_t);
  counters = (counters + kCounterBytes - 1) / kCounterBytes * kCounterBytes;
  const size_t parts = static_cast<size_t>(pairs) * num_split * g;
  size_t lse = parts * sizeof(float);
  lse = (lse + kCounterBytes - 1) / kCounterBytes * kCounterBytes;
  return counters + lse + parts * head_dim * sizeof(float);
}

size_t decode_sk_workspace_bytes(int64_t pairs, int num_split, int g, int head_dim) {
  size_t counters = static_cast<size_t>(pairs) * sizeof(int32_t);
  counters = (counters + kCounterBytes - 1) / kCounterBytes * kCounterBytes;
  const size_t parts = static_cast<size_t>(pairs) * (num_split > 1 ? num_split : 1) * 2 * g;
  size_t lse = parts * sizeof(float);
  lse = (lse + kCounterBytes - 1) / kCounterBytes * kCounterBytes;
  return counters + lse + parts * head_dim * sizeof(float);
}

int64_t prefill_padded_len(const seer_dims* d) {
  return (static_cast<int64_t>(d->max_seq_len) + kPrefillTokenTile - 1) / kPrefillTokenTile *
         kPrefillTokenTile;
}

size_t prefill_vt_bytes(const seer_dims* d) {
  const size_t vt = static_cast<size_t>(d->batch) * d->num_kv_heads * d->head_dim *
                    static_cast<size_t>(prefill_padded_len(d)) * 2;
  return (vt + 255) / 256 * 256;
}

size_t prefill_workspace_bytes(const seer_dims* d) {
  return prefill_vt_bytes(d) + static_cast<size_t>(d->batch) * d->num_q_heads *
                                   static_cast<size_t>(nb_max(d)) *
                                   static_cast<size_t>(prefill_padded_len(d)) * 4;
}

int auto_num_split(const seer_dims* d, int max_blocks, int num_cus) {
  // Measured on MI355X: the decode kernel keeps HBM busy once about eight
  // waves per compute unit are in flight chip-wide (each wave streams its
  // chunks with all loads of a chunk outstanding), so every CU needs work:
  // aim at 8 waves per CU in total with the workgroup size the launcher
  // picks, but no more splits than leave one 64-token chunk per wave (more
  // would only add partials to merge, not bytes in flight).
  const int g = d->num_q_heads / d->num_kv_heads;
  const int64_t pairs = static_cast<int64_t>(d->batch) * d->num_kv_heads;
  const int64_t chunks = static_cast<int64_t>(max_blocks) * (d->block_size / 64);
  const int cus = num_cus > 0 ? num_cus : 256;
  const int nw = decode_waves_per_group(g, d->head_dim);
  const int64_t target_wgs = static_cast<int64_t>(cus) * 8 / nw;
  int64_t s = (target_wgs + pairs - 1) / pairs;
  if (s > chunks / nw) s = chunks / nw;
  if (s < 1) s = 1;
  if (s > kMaxSplit) s = kMaxSplit;
  return static_cast<int>(s);
}

bool decode_waves_fit(int nw, int g, int head_dim) {
  return static_cast<int64_t>(nw) * g * head_dim * static_cast<int64_t>(sizeof(float)) <=
         kDecodeMergeLds;
}

int decode_waves_per_group(int g, int head_dim) {
  // Eight waves (one workgroup per CU at the kernel's register use) when
  // their merge (8 x g x head_dim floats of LDS) fits the budget, else four.
  return decode_waves_fit(8, g, head_dim) ? 8 : 4;
}

}  // namespace seer

extern "C" const char* seer_status_string(int status) {
  switch (status) {
    case SEER_OK: return "SEER_OK";
    case SEER_ERR_INVALID_ARG: return "SEER_ERR_INVALID_ARG: invalid argument";
    case SEER_ERR_UNSUPPORTED: return "SEER_ERR_UNSUPPORTED: configuration not supported";
    case SEER_ERR_WORKSPACE: return "SEER_ERR_WORKSPACE: workspace missing or too small";
    case SEER_ERR_HIP: return "SEER_ERR_HIP: HIP runtime error";
    default: return "SEER_ERR_UNKNOWN";
  }
}

extern "C" const char* seer_last_error_message(void) { return seer::last_error(); }

extern "C" const char* seer_version(void) { return "seer-mi355x 0.1.0 (gfx950)"; }
