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
// NT threads select (a whole 512-thread workgroup in the kernels here, so
// that each thread holds one key at the usual sizes; with NT = 64 one wave
// selects without workgroup barriers); thread t owns a contiguous range of
// block indices, so a prefix sum over per-thread counts writes the selected
// indices in ascending order without a sort.
//
// Top-k is an exact selection by narrowing: the keys still "in play" always
// form one interval [lo, hi] of the order-preserving 32-bit key (every key
// above hi is taken, every key below lo is not), and `need` of them are
// still to take.  Each pass histograms the in-play keys into 256 buckets,
// keeps the bucket that holds the need-th largest and stops once that bucket
// is to be taken whole.  The first pass buckets linearly on the float value
// between the smallest and largest logit, which for logits of similar size
// leaves a handful of keys in play; later passes bucket on the key bits
// below the interval's leading bit (8 bits per pass, so at most four).  If
// the interval closes on one value, its duplicates are taken in index order
// (lower index first).
//
// Top-p ([CP Knowl 14] names it as the adaptive direction) runs the same
// narrowing with probability mass in place of counts: each key's softmax
// mass is rounded to an integer number of 2^-30 units, the buckets sum those
// integers, and the cut is the first key (descending, equal logits in index
// order) where the running mass reaches ceil(p * 2^30) -- exact and
// independent of the summation order.
#pragma once

#include "../../include/seer.h"
#include "seer_device.hpp"

namespace seer {

constexpr int kSelMaxWaves = 16;
constexpr int kSelCand = 32;  // top-k fast path: boundary-bucket keys ranked directly

struct alignas(16) SelectSmem {
  int hist[256];  // 16-byte aligned: the top-k fast path reads it four at a time
  int hmass[256];  // top-p: per-bucket mass in units of 2^-30 of the total
  float fred[2][kSelMaxWaves];
  uint32_t ured[2][kSelMaxWaves];
  int scan[2][kSelMaxWaves];
  int pick[4];
  uint32_t cand_key[kSelCand];  // top-k fast path: the boundary bucket's keys
  int cand_idx[kSelCand];
  int ncand;
};

// Clears the histograms; call with every thread, then a barrier, before the
// first selection.
__device__ __forceinline__ void select_smem_init(SelectSmem& sm) {
  if (threadIdx.x < 256) {
    sm.hist[threadIdx.x] = 0;
    sm.hmass[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) sm.ncand = 0;
}

// Top-p mass unit: 2^30 units make the whole softmax.
constexpr float kMassUnits = 1073741824.f;

// Makes the LDS writes of the NT selecting threads visible to all of them:
// a workgroup barrier, or for a single wave only an ordering point (the LDS
// operations of one wave complete in issue order).
template <int NT>
__device__ __forceinline__ void sel_sync() {
  if constexpr (NT == 64) {
    wave_lds_order();
  } else {
    __syncthreads();
  }
}

// Exclusive prefix sum of v over the NT threads in thread order, and the
// total.  `part` (NT/64 ints of LDS) must not be in use by another scan
// that some thread may still be reading.
template <int NT>
__device__ __forceinline__ int wg_exclusive_scan(int v, int* part, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if constexpr (NW == 1) {
    *total = __builtin_amdgcn_readlane(incl, 63);
    return incl - v;
  }
  if (lane == 63) part[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int s = part[i];
    before += (i < w) ? s : 0;
    tot += s;
  }
  *total = tot;
  return before + incl - v;
}

template <int NT>
__device__ __forceinline__ void wg_minmax_f(float& mn, float& mx, SelectSmem& sm) {
  constexpr int NW = NT / 64;
  const int w = threadIdx.x >> 6;
  mn = wave_min(mn);
  mx = wave_max(mx);
  if constexpr (NW == 1) return;
  if ((threadIdx.x & 63) == 0) {
    sm.fred[0][w] = mn;
    sm.fred[1][w] = mx;
  }
  __syncthreads();
  mn = sm.fred[0][0];
  mx = sm.fred[1][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    mn = fminf(mn, sm.fred[0][i]);
    mx = fmaxf(mx, sm.fred[1][i]);
  }
}

template <int NT>
__device__ __forceinline__ void wg_minmax_u(uint32_t& mn, uint32_t& mx, SelectSmem& sm) {
  constexpr int NW = NT / 64;
  const int w = threadIdx.x >> 6;
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  if constexpr (NW == 1) return;
  if ((threadIdx.x & 63) == 0) {
    sm.ured[0][w] = mn;
    sm.ured[1][w] = mx;
  }
  __syncthreads();
  mn = sm.ured[0][0];
  mx = sm.ured[1][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    mn = min(mn, sm.ured[0][i]);
    mx = max(mx, sm.ured[1][i]);
  }
}

// After the histogram of this pass is complete (sm.hist, callers add to it
// before calling): the bucket holding the need-th largest counted key, the
// number of counted keys in higher buckets, and that bucket's count.  Wave 0
// scans and clears the histogram for the next pass.  1 <= need <= counted.
template <int NT>
__device__ __forceinline__ void hist_pick(SelectSmem& sm, int need, int& bucket, int& above,
                                          int& count) {
  sel_sync<NT>();
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    int hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hb[i] = sm.hist[4 * lane + i];
      sm.hist[4 * lane + i] = 0;
    }
    const int mine = (hb[0] + hb[1]) + (hb[2] + hb[3]);
    const int incl = wave_inclusive_scan(mine);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const int suf = total - incl + mine;  // keys in buckets >= 4*lane
    int cnt = suf - mine;                 // keys in buckets >= 4*lane + 4
    if (cnt < need && need <= suf) {      // exactly one lane
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (cnt + hb[i] >= need) {
          sm.pick[0] = 4 * lane + i;
          sm.pick[1] = cnt;
          sm.pick[2] = hb[i];
          break;
        }
        cnt += hb[i];
      }
    }
  }
  sel_sync<NT>();
  bucket = sm.pick[0];
  above = sm.pick[1];
  count = sm.pick[2];
}

// Top-p: after the mass histogram of this pass is complete (sm.hmass, with
// the counts in sm.hist): the bucket where the mass accumulated from the top
// first reaches `need`, the mass of the higher buckets, and the bucket's mass
// and count.  Wave 0 scans and clears both histograms.  1 <= need <= counted
// mass.
template <int NT>
__device__ __forceinline__ void hist_pick_mass(SelectSmem& sm, int need, int& bucket, int& above,
                                               int& mass, int& count) {
  sel_sync<NT>();
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    int hm[4], hc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hm[i] = sm.hmass[4 * lane + i];
      hc[i] = sm.hist[4 * lane + i];
      sm.hmass[4 * lane + i] = 0;
      sm.hist[4 * lane + i] = 0;
    }
    const int mine = (hm[0] + hm[1]) + (hm[2] + hm[3]);
    const int incl = wave_inclusive_scan(mine);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const int suf = total - incl + mine;  // mass in buckets >= 4*lane
    int cm = suf - mine;                  // mass in buckets >= 4*lane + 4
    if (cm < need && need <= suf) {       // exactly one lane
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (cm + hm[i] >= need) {
          sm.pick[0] = 4 * lane + i;
          sm.pick[1] = cm;
          sm.pick[2] = hm[i];
          sm.pick[3] = hc[i];
          break;
        }
        cm += hm[i];
      }
    }
  }
  sel_sync<NT>();
  bucket = sm.pick[0];
  above = sm.pick[1];
  mass = sm.pick[2];
  count = sm.pick[3];
}

// The keys j0 .. j0+n-1 of one thread: held in registers when KPL > 0 (n <=
// KPL), else read from LDS on every visit.  each(f) calls f(j, z) in index
// order.
template <int KPL>
struct KeyRange {
  const uint32_t* keys;
  int j0, n;
  float zr[KPL > 0 ? KPL : 1];
  __device__ __forceinline__ KeyRange(const uint32_t* k, int first, int count)
      : keys(k), j0(first), n(count) {
    if constexpr (KPL > 0) {
#pragma unroll
      for (int i = 0; i < KPL; ++i) zr[i] = (i < n) ? __uint_as_float(keys[j0 + i]) : 0.f;
    }
  }
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    if constexpr (KPL > 0) {
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (i < n) f(j0 + i, zr[i]);
    } else {
      for (int i = 0; i < n; ++i) f(j0 + i, __uint_as_float(keys[j0 + i]));
    }
  }
};

// The selection proper; KPL as in KeyRange (all NT threads take the same
// instantiation).
template <int NT, int KPL>
__device__ __forceinline__ void select_blocks_impl(const uint32_t* keys, SelectSmem& sm, int nc,
                                                   int total_blocks, int mode, int topk,
                                                   float log_tau, uint32_t mass_target,
                                                   int max_sel, int32_t* out,
                                                   int32_t* count_out) {
  static_assert(NT % 64 == 0 && NT / 64 <= kSelMaxWaves, "workgroup size");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int vpt = (nc + NT - 1) / NT;
  const int j0 = min(nc, tid * vpt);
  const int j1 = min(nc, j0 + vpt);
  const KeyRange<KPL> kr(keys, j0, j1 - j0);

  // Blocks without a cache entry (normally just the partial block) are
  // always active ([CP Knowl 5]).  They come first when the row is short:
  // the last min(forced, max_sel) of them are kept, and the scored blocks
  // get the room left (top-k's k shrinks to it).
  const int forced = max(0, total_blocks - nc);
  const int kept_forced = min(forced, max_sel);
  const int room = max_sel - kept_forced;

  // A key is taken iff  key > lo, or key == lo and (whole || rank < need)
  // (top-k), or z > thr (threshold); `all` / `none` short-cut both.
  bool all = false, none = false, whole = true;
  uint32_t lo = 0;
  int need = 0;
  float thr = 0.f;

  if (mode == SEER_SELECT_TOPK) {
    const int k = min(min(topk, nc), room);
    if (k >= nc) {
      all = true;
    } else if (k <= 0) {
      none = true;
    } else {
      need = k;
      int m = nc;  // keys in play
      float zmn = INFINITY, zmx = -INFINITY;
      kr.each([&](int, float z) {
        zmn = fminf(zmn, z);
        zmx = fmaxf(zmx, z);
      });
      wg_minmax_f<NT>(zmn, zmx, sm);
      const float scale = 256.f / (zmx - zmn);
      uint32_t hi;
      uint32_t kmn = 0xffffffffu, kmx = 0u;
      if (zmx > zmn && scale > 0.f && scale < INFINITY) {
        // linear buckets on the value; monotone in z (NaN counts lowest)
        auto fbucket = [&](float z) -> int {
          return (z == z) ? min(255, static_cast<int>((z - zmn) * scale)) : 0;
        };
        kr.each([&](int, float z) { atomicAdd(&sm.hist[fbucket(z)], 1); });
        int b, above;
        hist_pick<NT>(sm, need, b, above, m);
        need -= above;
        // the kept bucket as an interval of keys
        kr.each([&](int, float z) {
          if (fbucket(z) == b) {
            const uint32_t key = float_key(z);
            kmn = min(kmn, key);
            kmx = max(kmx, key);
          }
        });
      } else {
        kr.each([&](int, float z) {
          const uint32_t key = float_key(z);
          kmn = min(kmn, key);
          kmx = max(kmx, key);
        });
      }
      wg_minmax_u<NT>(kmn, kmx, sm);
      lo = kmn;
      hi = kmx;
      // narrow on key bits until the kept bucket is taken whole or is a
      // single value
      while (m != need && lo != hi) {
        const int shift = max(0, 32 - __clz(static_cast<int>(hi - lo)) - 8);
        kr.each([&](int, float z) {
          const uint32_t key = float_key(z);
          if (key >= lo && key <= hi) atomicAdd(&sm.hist[(key - lo) >> shift], 1);
        });
        int b, above;
        hist_pick<NT>(sm, need, b, above, m);
        need -= above;
        const uint64_t nlo = static_cast<uint64_t>(lo) + (static_cast<uint64_t>(b) << shift);
        const uint64_t nhi = nlo + (uint64_t{1} << shift) - 1;
        lo = static_cast<uint32_t>(nlo);
        hi = static_cast<uint32_t>(min(nhi, static_cast<uint64_t>(hi)));
      }
      whole = (m == need);
    }
  } else if (mode == SEER_SELECT_TOPP) {
    // Top-p: the smallest prefix of the descending order whose softmax mass
    // reaches p.  Each key's mass is w = rint(exp(z - max) / sum * 2^30)
    // (sum in a fixed order; equal logits get equal w); the prefix ends at
    // the first key where the running mass reaches T = ceil(p * 2^30).
    // The narrowing is the top-k one with mass in place of counts; on a run
    // of equal logits the first ceil(remaining / w) in index order are taken.
    float mx = -INFINITY;
    kr.each([&](int, float z) { mx = fmaxf(mx, z); });
    mx = wave_max(mx);
    if constexpr (NW > 1) {
      if ((tid & 63) == 0) sm.fred[0][tid >> 6] = mx;
      __syncthreads();
      mx = sm.fred[0][0];
#pragma unroll
      for (int i = 1; i < NW; ++i) mx = fmaxf(mx, sm.fred[0][i]);
    }
    float se = 0.f;
    kr.each([&](int, float z) { se += expf(z - mx); });
    se = wave_sum(se);
    if constexpr (NW > 1) {
      if ((tid & 63) == 0) sm.fred[1][tid >> 6] = se;
      __syncthreads();
      se = sm.fred[1][0];
#pragma unroll
      for (int i = 1; i < NW; ++i) se += sm.fred[1][i];
    }
    const float unit = kMassUnits / se;
    auto wmass = [&](float z) -> int { return static_cast<int>(rintf(expf(z - mx) * unit)); };
    int wsum = 0;
    kr.each([&](int, float z) { wsum += wmass(z); });
    int total_mass;
    (void)wg_exclusive_scan<NT>(wsum, sm.scan[0], &total_mass);
    const int target = static_cast<int>(mass_target);
    if (nc <= 0 || target <= 0) {
      none = true;
    } else if (target > total_mass) {
      all = true;
    } else {
      int need_m = target;
      int bmass = total_mass, bcount = nc;  // the kept bucket
      float zmn = INFINITY, zmx = -INFINITY;
      kr.each([&](int, float z) {
        zmn = fminf(zmn, z);
        zmx = fmaxf(zmx, z);
      });
      wg_minmax_f<NT>(zmn, zmx, sm);
      const float scale = 256.f / (zmx - zmn);
      uint32_t hi;
      uint32_t kmn = 0xffffffffu, kmx = 0u;
      if (zmx > zmn && scale > 0.f && scale < INFINITY) {
        auto fbucket = [&](float z) -> int {
          return (z == z) ? min(255, static_cast<int>((z - zmn) * scale)) : 0;
        };
        kr.each([&](int, float z) {
          const int bkt = fbucket(z);
          atomicAdd(&sm.hist[bkt], 1);
          atomicAdd(&sm.hmass[bkt], wmass(z));
        });
        int b, above;
        hist_pick_mass<NT>(sm, need_m, b, above, bmass, bcount);
        need_m -= above;
        kr.each([&](int, float z) {
          if (fbucket(z) == b) {
            const uint32_t key = float_key(z);
            kmn = min(kmn, key);
            kmx = max(kmx, key);
          }
        });
      } else {
        kr.each([&](int, float z) {
          const uint32_t key = float_key(z);
          kmn = min(kmn, key);
          kmx = max(kmx, key);
        });
      }
      wg_minmax_u<NT>(kmn, kmx, sm);
      lo = kmn;
      hi = kmx;
      // narrow until the kept bucket is taken whole (its mass is exactly what
      // is still needed, or it holds one key) or holds a single value
      while (need_m < bmass && bcount > 1 && lo != hi) {
        const int shift = max(0, 32 - __clz(static_cast<int>(hi - lo)) - 8);
        kr.each([&](int, float z) {
          const uint32_t key = float_key(z);
          if (key >= lo && key <= hi) {
            atomicAdd(&sm.hist[(key - lo) >> shift], 1);
            atomicAdd(&sm.hmass[(key - lo) >> shift], wmass(z));
          }
        });
        int b, above;
        hist_pick_mass<NT>(sm, need_m, b, above, bmass, bcount);
        need_m -= above;
        const uint64_t nlo = static_cast<uint64_t>(lo) + (static_cast<uint64_t>(b) << shift);
        const uint64_t nhi = nlo + (uint64_t{1} << shift) - 1;
        lo = static_cast<uint32_t>(nlo);
        hi = static_cast<uint32_t>(min(nhi, static_cast<uint64_t>(hi)));
      }
      whole = (need_m >= bmass || bcount == 1);
      if (!whole) {  // bcount equal logits of mass bmass / bcount each
        const int w0 = bmass / bcount;
        need = (need_m + w0 - 1) / w0;
      }
    }
  } else {
    // softmax_j > tau  <=>  z_j > ln(tau) + logsumexp(z); fixed summation order
    float mx = -INFINITY;
    kr.each([&](int, float z) { mx = fmaxf(mx, z); });
    mx = wave_max(mx);
    if constexpr (NW > 1) {
      if ((tid & 63) == 0) sm.fred[0][tid >> 6] = mx;
      __syncthreads();
      mx = sm.fred[0][0];
#pragma unroll
      for (int i = 1; i < NW; ++i) mx = fmaxf(mx, sm.fred[0][i]);
    }
    float se = 0.f;
    kr.each([&](int, float z) { se += expf(z - mx); });
    se = wave_sum(se);
    if constexpr (NW > 1) {
      if ((tid & 63) == 0) sm.fred[1][tid >> 6] = se;
      __syncthreads();
      se = sm.fred[1][0];
#pragma unroll
      for (int i = 1; i < NW; ++i) se += sm.fred[1][i];
    }
    thr = (nc > 0) ? log_tau + (mx + logf(se)) : INFINITY;
  }

  const bool ranked = (mode == SEER_SELECT_TOPK || mode == SEER_SELECT_TOPP);
  const bool topk_range = ranked && !all && !none;
  // ranks among the duplicates of lo, in index order (only if not whole)
  int eq_before = 0;
  if (topk_range && !whole) {
    int eq = 0;
    kr.each([&](int, float z) { eq += (float_key(z) == lo); });
    int unused;
    eq_before = wg_exclusive_scan<NT>(eq, sm.scan[0], &unused);
  }
  auto taken = [&](float z, int& rank) -> bool {
    if (!ranked) return z > thr;
    if (all) return true;
    if (none) return false;
    const uint32_t key = float_key(z);
    if (key > lo) return true;
    if (key < lo) return false;
    const bool t = whole || rank < need;
    ++rank;
    return t;
  };
  int nsel = 0;
  {
    int rank = eq_before;
    kr.each([&](int, float z) { nsel += taken(z, rank); });
  }
  int scored_total;
  int pos = wg_exclusive_scan<NT>(nsel, sm.scan[1], &scored_total);
  {
    int rank = eq_before;
    kr.each([&](int j, float z) {
      if (taken(z, rank)) {
        if (pos < room) out[pos] = j;
        ++pos;
      }
    });
  }
  // then the forced blocks (top-k fits them by construction; threshold and
  // top-p rows hold every block, so nothing scored is cut there)
  const int scored_written = min(scored_total, room);
  const int f0 = total_blocks - kept_forced;
  for (int f = tid; f < kept_forced; f += NT) out[scored_written + f] = f0 + f;
  const int written = scored_written + kept_forced;
  for (int i = written + tid; i < max_sel; i += NT) out[i] = -1;
  if (tid == 0) *count_out = written;
}

// Top-k when every thread holds at most one key (nc <= NT) and 0 < k < nc,
// in three or four workgroup barriers (the general narrowing above takes
// seven): the value histogram is scanned by every wave itself, and the
// bucket holding the k-th largest key is resolved by ranking its few keys
// against each other instead of by further histogram passes.  It selects
// the same set as the narrowing (the k largest; equal logits: lower index
// first).  Returns false, having written nothing and with the histograms
// zero, when it does not apply (the caller then runs the narrowing).
//   1. wave min / max of the logits to LDS; barrier;
//   2. every thread: the workgroup min / max, then its key's bucket among
//      256 linear buckets on [min, max] into the histogram; barrier;
//   3. every wave: the histogram scan -> bucket b, the count above it, its
//      count m (identical in every wave);
//   4. if m keys exceed what is still needed: b's keys append (key, index)
//      to a list; barrier; each counts the list entries ahead of it
//      (m > kSelCand: not applicable);
//   5. the ascending output: per-wave ballot counts; barrier; prefix; write.
template <int NT>
__device__ __forceinline__ bool select_topk_one_key(const uint32_t* keys, SelectSmem& sm, int nc,
                                                    int total_blocks, int k, int max_sel,
                                                    int32_t* out, int32_t* count_out) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const bool have = tid < nc;
  const float z = have ? __uint_as_float(keys[tid]) : 0.f;
  // 1.
  {
    const float mn = wave_min(have ? z : INFINITY);
    const float mx = wave_max(have ? z : -INFINITY);
    if (lane == 0) {
      sm.fred[0][w] = mn;
      sm.fred[1][w] = mx;
    }
  }
  __syncthreads();
  // 2.
  float zmn = sm.fred[0][0], zmx = sm.fred[1][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    zmn = fminf(zmn, sm.fred[0][i]);
    zmx = fmaxf(zmx, sm.fred[1][i]);
  }
  const float scale = 256.f / (zmx - zmn);
  if (!(zmx > zmn && scale > 0.f && scale < INFINITY)) {  // uniform
    __syncthreads();  // every wave has read fred before the narrowing rewrites it
    return false;
  }
  const int bkt = (z == z) ? min(255, static_cast<int>((z - zmn) * scale)) : 0;
  if (have) atomicAdd(&sm.hist[bkt], 1);
  __syncthreads();
  // 3. every wave: lane l holds buckets 4l .. 4l+3
  int b_star, above, m;
  {
    const int4 h4 = *reinterpret_cast<const int4*>(&sm.hist[4 * lane]);
    const int hb[4] = {h4.x, h4.y, h4.z, h4.w};
    const int mine = (hb[0] + hb[1]) + (hb[2] + hb[3]);
    const int incl = wave_inclusive_scan(mine);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const int suf = total - incl + mine;  // keys in buckets >= 4 lane
    int cnt = suf - mine;                 // keys in buckets >= 4 lane + 4
    int pick = -1, pa = 0, pm = 0;
    if (cnt < k && k <= suf) {
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (pick < 0 && cnt + hb[i] >= k) {
          pick = 4 * lane + i;
          pa = cnt;
          pm = hb[i];
        }
        cnt += hb[i];
      }
    }
    const unsigned long long who = __ballot(pick >= 0);
    const int src = __builtin_ffsll(static_cast<long long>(who)) - 1;  // exactly one lane
    b_star = __builtin_amdgcn_readlane(pick, src);
    above = __builtin_amdgcn_readlane(pa, src);
    m = __builtin_amdgcn_readlane(pm, src);
  }
  const int need = k - above;  // 1 <= need <= m
  if (m > need && m > kSelCand) {  // uniform: leave it to the narrowing
    __syncthreads();               // every wave has read the histogram
    if (tid < 256) sm.hist[tid] = 0;
    __syncthreads();
    return false;
  }
  bool taken = have && bkt > b_star;
  if (m == need) {
    taken = taken || (have && bkt == b_star);
  } else {
    // 4. rank the boundary bucket's keys: (key descending, index ascending)
    const uint32_t key = float_key(z);
    if (have && bkt == b_star) {
      const int slot = atomicAdd(&sm.ncand, 1);
      sm.cand_key[slot] = key;
      sm.cand_idx[slot] = tid;
    }
    __syncthreads();
    if (have && bkt == b_star) {
      int ahead = 0;
      for (int c = 0; c < m; ++c) {
        const uint32_t kc = sm.cand_key[c];
        ahead += (kc > key) || (kc == key && sm.cand_idx[c] < tid);
      }
      taken = ahead < need;
    }
  }
  // 5. positions in index order (thread order)
  const unsigned long long bal = __ballot(taken);
  const int before_in_wave = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) sm.scan[1][w] = __builtin_popcountll(bal);
  __syncthreads();
  if (tid < 256) sm.hist[tid] = 0;  // left zero, as the narrowing leaves them
  if (tid == 0) sm.ncand = 0;
  int before = 0, scored_total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = sm.scan[1][i];
    before += (i < w) ? c : 0;
    scored_total += c;
  }
  // forced blocks first when the row is short (the caller's k fits them)
  const int forced = max(0, total_blocks - nc);
  const int kept_forced = min(forced, max_sel);
  const int room = max_sel - kept_forced;
  const int pos = before + before_in_wave;
  if (taken && pos < room) out[pos] = tid;
  const int scored_written = min(scored_total, room);
  const int f0 = total_blocks - kept_forced;
  for (int f = tid; f < kept_forced; f += NT) out[scored_written + f] = f0 + f;
  const int written = scored_written + kept_forced;
  for (int i = written + tid; i < max_sel; i += NT) out[i] = -1;
  if (tid == 0) *count_out = written;
  return true;
}

// Called by all NT threads once keys[0..nc) (LDS, the logits as float bits)
// are visible to every one of them.  The histograms (select_smem_init) must
// be zero on entry and are left zero.  mass_target = ceil(p * 2^30) for
// top-p.  Appends the unscored blocks nc .. total_blocks-1 and writes the
// ascending, -1 padded row out[0..max_sel) plus its count.  Up to 32 keys
// per thread are held in registers.
template <int NT>
__device__ __forceinline__ void select_blocks_wg(const uint32_t* keys, SelectSmem& sm, int nc,
                                                 int total_blocks, int mode, int topk,
                                                 float log_tau, uint32_t mass_target,
                                                 int max_sel, int32_t* out, int32_t* count_out) {
  const int vpt = (nc + NT - 1) / NT;
  if (mode == SEER_SELECT_TOPK && vpt <= 1) {
    const int forced = max(0, total_blocks - nc);
    const int k = min(min(topk, nc), max_sel - min(forced, max_sel));
    if (k > 0 && k < nc &&
        select_topk_one_key<NT>(keys, sm, nc, total_blocks, k, max_sel, out, count_out))
      return;
  }
  if (vpt <= 1)
    select_blocks_impl<NT, 1>(keys, sm, nc, total_blocks, mode, topk, log_tau, mass_target,
                              max_sel, out, count_out);
  else if (vpt <= 8)
    select_blocks_impl<NT, 8>(keys, sm, nc, total_blocks, mode, topk, log_tau, mass_target,
                              max_sel, out, count_out);
  else if (vpt <= 32)
    select_blocks_impl<NT, 32>(keys, sm, nc, total_blocks, mode, topk, log_tau, mass_target,
                               max_sel, out, count_out);
  else
    select_blocks_impl<NT, 0>(keys, sm, nc, total_blocks, mode, topk, log_tau, mass_target,
                              max_sel, out, count_out);
}

}  // namespace seer
