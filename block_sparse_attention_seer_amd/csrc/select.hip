// Block selection kernel (staged call seer_select_blocks), for gfx950.
//
// [CP Knowl 5] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): token-budget top-k on un-softmaxed logits
// or threshold on the softmax; [CP Knowl 14]: top-p (nucleus) mass; the
// incomplete last block is always selected.
// One 512-thread workgroup per (sequence, KV head) loads the row of logits
// into LDS and runs the selection shared with the fused gate kernel (same
// workgroup size), so the staged and the fused paths select identically.
#include <cmath>

#include "select_dev.hpp"
#include "seer_internal.h"

namespace seer {

namespace {

constexpr int kSelThreads = 512;

struct SelectParams {
  const float* logits;
  const int32_t* kcomp_lens;
  const int32_t* seq_lens;
  int32_t* block_idx;
  int32_t* num_selected;
  int Hkv, BS, Lmax, NBmax, mode, topk, max_sel;
  float log_tau;         // ln(tau), -inf for tau = 0
  uint32_t mass_target;  // top-p: ceil(p * 2^30)
};

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  extern __shared__ uint32_t s_keys[];  // NBmax floats (bits)
  __shared__ SelectSmem s_sel;
  const int pair = blockIdx.x;
  const int b = pair / p.Hkv;
  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  const int total_blocks = (L + p.BS - 1) / p.BS;
  int nc = p.kcomp_lens[b];
  nc = min(min(max(nc, 0), p.NBmax), L / p.BS);
  const float* z = p.logits + static_cast<int64_t>(pair) * p.NBmax;
  for (int j = threadIdx.x; j < nc; j += kSelThreads) s_keys[j] = __float_as_uint(z[j]);
  select_smem_init(s_sel);
  __syncthreads();
  select_blocks_wg<kSelThreads>(s_keys, s_sel, nc, total_blocks, p.mode, p.topk, p.log_tau,
                                p.mass_target, p.max_sel,
                                p.block_idx + static_cast<int64_t>(pair) * p.max_sel,
                                p.num_selected + pair);
}

}  // namespace

float log_threshold(float tau) {
  return tau > 0.f ? static_cast<float>(std::log(static_cast<double>(tau))) : -INFINITY;
}

uint32_t topp_mass_target(float p) {
  const double t = std::ceil(static_cast<double>(p) * 1073741824.0);
  return t <= 0.0 ? 0u : (t >= 2147483647.0 ? 2147483647u : static_cast<uint32_t>(t));
}

int launch_select(const seer_dims& d, const SelectArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nbm = static_cast<int>(nb_max(&d));
  SelectParams p{a.logits, a.kcomp_lens, a.seq_lens, a.block_idx, a.num_selected,
                 d.num_kv_heads, d.block_size, d.max_seq_len, nbm, a.mode, a.topk,
                 a.max_selected, log_threshold(a.tau), topp_mass_target(a.tau)};
  const size_t lds = static_cast<size_t>(nbm) * sizeof(uint32_t);
  hipLaunchKernelGGL(select_kernel, dim3(d.batch * d.num_kv_heads), dim3(kSelThreads), lds, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("select launch: ") + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  return SEER_OK;
}

}  // namespace seer
