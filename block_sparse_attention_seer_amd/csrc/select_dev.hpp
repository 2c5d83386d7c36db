// Binarisation of block scores into active-block indices: the device part
// shared by the select kernel and the fused gate kernel, for gfx950.
//
// [CP Knowl 5] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): (1) token budget -> top-k block indices
// on the un-softmaxed logits; (2) threshold: blocks whose score exceeds tau,
// no sorting, so each head gets its own sparsity.  When the length is not a
// multiple of b the incomplete last block is always selected.
// [CP Knowl 6]: the index tensor is [batch, heads_kv, max_selected_blocks].
//
// One wave does the whole selection of a (sequence, KV head), so it needs
// no workgroup barrier: LDS operations of one wave complete in issue order,
// and cross-lane steps are shuffles.  Top-k is an exact radix select over
// order-preserving 32-bit keys, most significant 8 bits first: each pass
// histograms the keys still in play and keeps the bucket holding the k-th
// largest key; it stops as soon as that bucket is taken whole, and only
// exact duplicates of the k-th key need all four passes and a rank so that
// the lower indices win.  Output order is ascending block index via a wave
// prefix sum over contiguous per-lane index ranges -- no sort is needed.
#pragma once

#include "../../include/seer.h"
#include "seer_device.hpp"

namespace seer {

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Orders LDS traffic of this wave: every earlier LDS access has completed.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Called by the 64 lanes of one wave.  keys[0..nc) (LDS) hold the logits of
// the scored blocks as float bits and are overwritten; hist is 256 ints of
// LDS.  Appends the unscored blocks nc .. total_blocks-1 and writes the
// ascending, -1 padded row out[0..max_sel) plus its count.
__device__ void select_blocks_wave(uint32_t* keys, int* hist, int nc, int total_blocks, int mode,
                                   int topk, float log_tau, int max_sel, int32_t* out,
                                   int32_t* count_out) {
  const int lane = threadIdx.x & 63;
  const int vpl = (nc + 63) / 64;
  const int j0 = min(nc, lane * vpl);
  const int j1 = min(nc, j0 + vpl);

  // Top-k: a key is taken iff (key & pmask) > prefix, or it equals prefix
  // and it is within the first `need` such keys by index (or all of them
  // when the bucket holds exactly `need`).
  bool take_all = false, take_none = false, exact = true;
  uint32_t prefix = 0, pmask = 0;
  int need = 0;
  float thr = 0.f;  // threshold mode: logit bound

  if (mode == SEER_SELECT_TOPK) {
    const int k = min(topk, nc);
    if (k >= nc) {
      take_all = true;
    } else if (k <= 0) {
      take_none = true;
    } else {
      for (int j = j0; j < j1; ++j) keys[j] = float_key(__uint_as_float(keys[j]));
      need = k;
      exact = false;
      for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
        wave_lds_sync();
        for (int j = j0; j < j1; ++j) {
          const uint32_t key = keys[j];
          if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        wave_lds_sync();
        // lane covers digits 4*lane .. 4*lane+3; suffix sums from the top
        int hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hb[i] = hist[4 * lane + i];
        const int mine = hb[0] + hb[1] + hb[2] + hb[3];
        int suf = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_down(suf, o);
          if (lane + o < 64) suf += t;
        }
        const int above_group = suf - mine;  // keys with a digit above this lane's
        const bool owner = above_group < need && need <= suf;
        int cnt = above_group, dsel = 4 * lane, bucket = hb[0];
        if (owner) {
          for (int i = 3; i >= 0; --i) {
            if (cnt + hb[i] >= need) {
              dsel = 4 * lane + i;
              bucket = hb[i];
              break;
            }
            cnt += hb[i];
          }
        }
        const unsigned long long m = __ballot(owner);
        const int src = __ffsll(static_cast<long long>(m)) - 1;  // exactly one owner lane
        dsel = __shfl(dsel, src);
        cnt = __shfl(cnt, src);
        bucket = __shfl(bucket, src);
        prefix |= static_cast<uint32_t>(dsel) << shift;
        pmask |= 0xffu << shift;
        need -= cnt;
        wave_lds_sync();  // every lane has read the histogram
        if (bucket == need) {  // the k-th key's bucket is taken whole
          exact = true;
          break;
        }
      }
    }
  } else {
    // softmax_j > tau  <=>  z_j > ln(tau) + logsumexp(z)
    float mx = -INFINITY;
    for (int j = j0; j < j1; ++j) mx = fmaxf(mx, __uint_as_float(keys[j]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float se = 0.f;
    if (nc > 0)
      for (int j = j0; j < j1; ++j) se += expf(__uint_as_float(keys[j]) - mx);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) se += __shfl_xor(se, o);
    thr = (nc > 0) ? log_tau + (mx + logf(se)) : INFINITY;
  }

  // ranks among keys equal to the final prefix (only for exact ties)
  int eq_before = 0;
  if (mode == SEER_SELECT_TOPK && !take_all && !take_none && !exact) {
    int eq = 0;
    for (int j = j0; j < j1; ++j) eq += ((keys[j] & pmask) == prefix);
    eq_before = wave_inclusive_scan(eq) - eq;
  }
  auto selected = [&](int j, int& rank) -> bool {
    if (mode != SEER_SELECT_TOPK) return __uint_as_float(keys[j]) > thr;
    if (take_all) return true;
    if (take_none) return false;
    const uint32_t mk = keys[j] & pmask;
    if (mk > prefix) return true;
    if (mk < prefix) return false;
    const bool take = exact || rank < need;
    ++rank;
    return take;
  };
  int nsel = 0;
  {
    int rank = eq_before;
    for (int j = j0; j < j1; ++j) nsel += selected(j, rank);
  }
  const int incl = wave_inclusive_scan(nsel);
  const int scored_total = __shfl(incl, 63);
  {
    int rank = eq_before;
    int pos = incl - nsel;
    for (int j = j0; j < j1; ++j) {
      if (selected(j, rank)) {
        if (pos < max_sel) out[pos] = j;
        ++pos;
      }
    }
  }
  // blocks without a cache entry (normally the partial block) are forced
  const int forced = max(0, total_blocks - nc);
  for (int f = lane; f < forced; f += 64) {
    const int pos = scored_total + f;
    if (pos < max_sel) out[pos] = nc + f;
  }
  const int written = min(scored_total + forced, max_sel);
  for (int i = written + lane; i < max_sel; i += 64) out[i] = -1;
  if (lane == 0) *count_out = written;
}

}  // namespace seer
