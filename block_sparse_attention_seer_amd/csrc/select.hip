// Binarisation of block scores into active-block indices, for gfx950.
//
// [CP Knowl 5] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): (1) token budget -> top-k block indices
// on the un-softmaxed logits; (2) threshold: blocks whose score exceeds tau,
// no sorting, so each head gets its own sparsity.  When the length is not a
// multiple of b the incomplete last block is always selected.
// [CP Knowl 6]: the index tensor is [batch, heads_kv, max_selected_blocks].
//
// One workgroup (4 waves) per (sequence, KV head).  Top-k is an exact radix
// select: four 8-bit passes over order-preserving 32-bit keys find the k-th
// largest key T; then every key > T is taken plus the lowest-index keys equal
// to T.  Output order is ascending block index via a block-wide prefix sum
// over contiguous per-thread index ranges -- no sort of the list is needed.
#include <cmath>

#include "seer_device.hpp"
#include "seer_internal.h"

namespace seer {

namespace {

struct SelectParams {
  const float* logits;
  const int32_t* kcomp_lens;
  const int32_t* seq_lens;
  int32_t* block_idx;
  int32_t* num_selected;
  int Hkv, BS, Lmax, NBmax, mode, topk, max_sel;
  float log_tau;  // ln(tau), -inf for tau = 0
};

constexpr int kThreads = 256;

// Exclusive prefix sum over the workgroup (thread order); *total gets the sum.
__device__ int block_exclusive_scan(int v, int* total, int* s_wave) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    const int x = s_wave[i];
    off += (i < w) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

__device__ float block_reduce_max(float v, float* s_f) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) s_f[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = s_f[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, s_f[i]);
  __syncthreads();
  return r;
}

__device__ float block_reduce_sum(float v, float* s_f) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) s_f[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) r += s_f[i];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void select_kernel(SelectParams p) {
  extern __shared__ uint32_t s_keys[];  // nc order-preserving keys (or raw float bits)
  __shared__ int s_hist[256];
  __shared__ int s_wave[kThreads / 64];
  __shared__ float s_f[kThreads / 64];
  __shared__ uint32_t s_digit;
  __shared__ int s_above;

  const int pair = blockIdx.x;
  const int b = pair / p.Hkv;
  const int tid = threadIdx.x;
  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  const int total_blocks = (L + p.BS - 1) / p.BS;
  int nc = p.kcomp_lens[b];
  nc = min(max(nc, 0), p.NBmax);
  nc = min(nc, L / p.BS);
  const float* z = p.logits + static_cast<int64_t>(pair) * p.NBmax;
  int32_t* out = p.block_idx + static_cast<int64_t>(pair) * p.max_sel;

  // Contiguous per-thread index ranges keep the output ascending.
  const int vpt = (nc + kThreads - 1) / kThreads;
  const int j0 = min(nc, tid * vpt);
  const int j1 = min(nc, j0 + vpt);

  // Selection rule for scored block j: take(key) below.
  bool take_all = false, take_none = false;
  uint32_t T = 0;       // top-k: k-th largest key
  int need = 0;         // top-k: keys equal to T still wanted
  float thr = 0.f;      // threshold: logit bound

  if (p.mode == SEER_SELECT_TOPK) {
    const int k = min(p.topk, nc);
    if (k >= nc) {
      take_all = true;
    } else if (k <= 0) {
      take_none = true;
    } else {
      for (int j = tid; j < nc; j += kThreads) s_keys[j] = float_key(z[j]);
      uint32_t prefix = 0, pmask = 0;
      need = k;
      for (int shift = 24; shift >= 0; shift -= 8) {
        s_hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < nc; j += kThreads) {
          const uint32_t key = s_keys[j];
          if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid < 64) {
          // lane covers digits 4*lane .. 4*lane+3; suffix sums from the top.
          int hb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) hb[i] = s_hist[4 * tid + i];
          const int mine = hb[0] + hb[1] + hb[2] + hb[3];
          int suf = mine;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_down(suf, o);
            if (tid + o < 64) suf += t;
          }
          const int above_group = suf - mine;  // keys with a digit above this lane's
          if (above_group < need && need <= suf) {
            int cnt = above_group;
            int dsel = 4 * tid;
            for (int i = 3; i >= 0; --i) {
              if (cnt + hb[i] >= need) {
                dsel = 4 * tid + i;
                break;
              }
              cnt += hb[i];
            }
            s_digit = static_cast<uint32_t>(dsel);
            s_above = cnt;
          }
        }
        __syncthreads();
        prefix |= s_digit << shift;
        pmask |= 0xffu << shift;
        need -= s_above;
        __syncthreads();
      }
      T = prefix;
    }
  } else {
    // softmax_j > tau  <=>  z_j > ln(tau) + logsumexp(z)
    float mx = -INFINITY;
    for (int j = tid; j < nc; j += kThreads) mx = fmaxf(mx, z[j]);
    mx = block_reduce_max(mx, s_f);
    float se = 0.f;
    if (nc > 0)
      for (int j = tid; j < nc; j += kThreads) se += expf(z[j] - mx);
    se = block_reduce_sum(se, s_f);
    thr = (nc > 0) ? p.log_tau + (mx + logf(se)) : INFINITY;
    for (int j = tid; j < nc; j += kThreads) s_keys[j] = __float_as_uint(z[j]);
    __syncthreads();
  }

  // ---- count this thread's selections (ascending within its range)
  int eq_before = 0;
  if (p.mode == SEER_SELECT_TOPK && !take_all && !take_none) {
    int eq = 0;
    for (int j = j0; j < j1; ++j) eq += (s_keys[j] == T);
    int tot_eq;
    eq_before = block_exclusive_scan(eq, &tot_eq, s_wave);
  }
  int nsel = 0;
  {
    int rank = eq_before;
    for (int j = j0; j < j1; ++j) {
      bool sel;
      if (p.mode == SEER_SELECT_TOPK) {
        if (take_all) sel = true;
        else if (take_none) sel = false;
        else {
          const uint32_t key = s_keys[j];
          sel = key > T || (key == T && rank < need);
          rank += (key == T);
        }
      } else {
        sel = __uint_as_float(s_keys[j]) > thr;
      }
      nsel += sel;
    }
  }
  int scored_total;
  const int pos0 = block_exclusive_scan(nsel, &scored_total, s_wave);

  // ---- write the scored selections
  {
    int rank = eq_before;
    int pos = pos0;
    for (int j = j0; j < j1; ++j) {
      bool sel;
      if (p.mode == SEER_SELECT_TOPK) {
        if (take_all) sel = true;
        else if (take_none) sel = false;
        else {
          const uint32_t key = s_keys[j];
          sel = key > T || (key == T && rank < need);
          rank += (key == T);
        }
      } else {
        sel = __uint_as_float(s_keys[j]) > thr;
      }
      if (sel) {
        if (pos < p.max_sel) out[pos] = j;
        ++pos;
      }
    }
  }
  // ---- blocks without a cache entry (normally the partial block) are forced
  const int forced = max(0, total_blocks - nc);
  for (int f = tid; f < forced; f += kThreads) {
    const int pos = scored_total + f;
    if (pos < p.max_sel) out[pos] = nc + f;
  }
  const int written = min(scored_total + forced, p.max_sel);
  for (int i = written + tid; i < p.max_sel; i += kThreads) out[i] = -1;
  if (tid == 0) p.num_selected[pair] = written;
}

}  // namespace

int launch_select(const seer_dims& d, const SelectArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nbm = static_cast<int>(nb_max(&d));
  SelectParams p{a.logits, a.kcomp_lens, a.seq_lens, a.block_idx, a.num_selected,
                 d.num_kv_heads, d.block_size, d.max_seq_len, nbm, a.mode, a.topk,
                 a.max_selected,
                 a.tau > 0.f ? static_cast<float>(std::log(static_cast<double>(a.tau))) : -INFINITY};
  const size_t lds = static_cast<size_t>(nbm) * sizeof(uint32_t);
  hipLaunchKernelGGL(select_kernel, dim3(d.batch * d.num_kv_heads), dim3(kThreads), lds, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("select launch: ") + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  return SEER_OK;
}

}  // namespace seer
