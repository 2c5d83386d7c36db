// Block-sparse flash decoding with split-KV and a log-sum-exp merge, for
// gfx950 (MI355X).
//
// [CP Knowl 6] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): the kernel runs over a (batch, heads_kv,
// num_split) grid, divides each (batch, KV head)'s work along num_split
// using its list of active blocks rather than the sequence's block count,
// and visits only the active block indices, skipping invalid entries.
// [PN key design 4] (papernotes page "Sparse Attention Adaptation for Long
// Reasoning"): the same flash-decoding schedule along the GQA group.
//
// MI355X design (not the pages' H100 design):
//   * one workgroup = NW waves = one split of one (b, h).  The (b, h)'s
//     active blocks are cut into 64-token chunks; split s owns the s-th of S
//     even chunk ranges and deals them round-robin to its waves, each
//     keeping its own online softmax.  The index row is staged in LDS,
//     requested together with the selection count;
//   * both contractions run on MFMA v_mfma_f32_16x16x32_bf16 with the g
//     query heads of the group padded to 16:
//       S^T[token][head] = K[token][:] . q[head][:]      (A = K rows straight
//                                                         from HBM, B = q)
//       O[head][dim]    += P[head][token] V[token][dim]  (A = P from the S
//                                                         accumulators, B = V)
//     The score accumulators already sit in the P operand's layout, so P
//     never leaves registers.  V is loaded as 8-byte pieces (4 dims of one
//     token) and the B operand (8 tokens of one dim) is assembled with
//     byte permutes, so V never goes through LDS.  All K and V loads of a
//     chunk (32 KiB per wave at d = 128) are in flight together;
//   * a paged cache (one block per page) changes only where a chunk's rows
//     start: the workgroup stages its sequence's block-table row in LDS with
//     the index row, and an out-of-range page is skipped like an invalid
//     index entry;
//   * the waves of a split merge in LDS; with one split the workgroup writes
//     the output directly.  Otherwise each split writes an (lse, o) partial
//     with device-coherent stores, counts itself on a per-(b, h) counter,
//     and the split that completes the count merges all partials (coherent
//     loads), writes the output and resets the counter.  Coherent accesses
//     go around the per-XCD L2, so no release/acquire fence is needed: those
//     turn into L2 write-back / invalidate on gfx950, which serialise across
//     workgroups;
//   * K rows use ordinary loads and V rows non-temporal ones: every chunk's
//     scores wait on K, while V is consumed later and need not take Infinity
//     Cache capacity;
//   * selections of very different sizes (threshold, top-p) can instead be
//     divided stream-K: each workgroup takes an equal share of all pairs'
//     chunks, decodes the pairs in it one after another, and a pair cut
//     between shares merges through the same counter protocol.
#include "seer_device.hpp"
#include "seer_internal.h"

namespace seer {

namespace {

constexpr int kIdxLds = 512;     // index-row entries staged in LDS per workgroup
constexpr int kTableLds = 2048;  // paged cache: block-table entries staged in LDS
// 16-token tiles per chunk (2 or 4).  Measured on MI355X: 4 (32 KiB of K
// and V in flight per wave at d = 128) streams faster than 2, whose finer
// share per wave does not make up for the halved bytes in flight.
constexpr int kTilesPerChunk = 4;
constexpr int kMergeInline = 8;  // splits merged from registers in one round trip
static_assert(kTilesPerChunk == 2 || kTilesPerChunk == 4, "tiles per chunk");

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_lens;
  const int32_t* block_idx;
  const int32_t* num_selected;
  int32_t* counters;  // [pairs] finished splits of each pair (zero between launches)
  float* part_lse;  // [pairs, S, G]   log2-domain lse of each split
  float* part_o;    // [pairs, S, G, D] normalised split outputs
  uint16_t* out;
  float* lse;
  int64_t sb, sh;
  int st;
  int Hq, Hkv, G, Lmax, max_sel, num_split;
  float scale_log2;  // softmax scale times log2(e): scores are kept in log2 units
  // fused step: workgroup 0 raises the cache counters of every sequence
  int32_t* commit_lens;
  int commit_max_new, B, BS, NBmax;
  // paged cache: the page of block j of sequence b is
  // block_table[b * table_stride + j]; a page holds H_kv x b rows of d
  const int32_t* block_table;
  int table_stride, num_pages;
  int64_t page_stride, page_head_stride;
};

// bf16 j (0..3) of a's four values in the low half, of b's in the high half.
__device__ __forceinline__ uint32_t pick2(uint2 a, uint2 b, int j) {
  const uint32_t x = (j < 2) ? a.x : a.y;
  const uint32_t y = (j < 2) ? b.x : b.y;
  return (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
}

// The part of one (b, h) that a workgroup computes.  Fixed splits cut the
// pair's active chunks into num_split even ranges and take range `split`;
// stream-K parts carry their chunk range [c_begin, c_end).  A pair of more
// than one part leaves each part's result in a slot of the workspace: part 0
// in slot0, part k > 0 in slot1 + (k - 1) * slot_step.
struct Part {
  int pair;
  int split, num_split;  // fixed splits
  int c_begin, c_end;    // stream-K
  int nparts;
  int64_t my_slot, slot0, slot1, slot_step;
};

template <int D, int BS, bool DENSE, int NW, bool PAGED, bool SK>
__device__ __forceinline__ void decode_part(const DecodeParams& p, const Part& pt, float* sm_o) {
  constexpr int TPC = kTilesPerChunk;  // 16-token tiles per chunk
  constexpr int KS = D / 32;   // k-steps of the score contraction
  constexpr int VH = D / 64;   // 64-dim halves of the value contraction
  constexpr int CPB = BS / (16 * TPC);  // chunks per block

  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];

  const int pair = pt.pair;
  const int b = pair / p.Hkv;
  const int h = pair - b * p.Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 15;
  const int lq = lane >> 4;
  const int G = p.G;

  const int32_t* idx = DENSE ? nullptr : p.block_idx + static_cast<int64_t>(pair) * p.max_sel;
  // The first kIdxLds entries of the index row go to LDS, requested at once
  // with the selection count instead of after it.
  __shared__ int s_idx[kIdxLds];
  if (!DENSE) {
    // a stream-K part stages only the entries of its own chunks
    const int i_end = min(p.max_sel, kIdxLds);
    const int i_lo = SK ? min(pt.c_begin / CPB, i_end) : 0;
    const int i_hi = SK ? min((pt.c_end + CPB - 1) / CPB, i_end) : i_end;
    for (int i = i_lo + tid; i < i_hi; i += NW * 64) s_idx[i] = idx[i];
  }
  // paged cache: this sequence's block-table row, requested with the rest
  __shared__ int s_table[PAGED ? kTableLds : 1];
  if (PAGED)
    for (int i = tid; i < min(p.table_stride, kTableLds); i += NW * 64)
      s_table[i] = p.block_table[static_cast<int64_t>(b) * p.table_stride + i];

  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  const int nblk = (L + BS - 1) / BS;
  int nslots;
  if (DENSE) {
    nslots = nblk;
  } else {
    nslots = p.num_selected[pair];
    nslots = min(max(nslots, 0), p.max_sel);
  }
  // Work unit: a chunk of TPC 16-token tiles of an active block.
  // The pair's chunks are cut into S even ranges, one per split; wave w of a
  // split takes chunks c_begin + w, c_begin + w + NW, ...  (A fixed
  // assignment keeps the summation order, and so the output bits, the same
  // from run to run.)
  const int nchunks = nslots * CPB;
  const int c_begin =
      SK ? pt.c_begin : static_cast<int>(static_cast<int64_t>(nchunks) * pt.split / pt.num_split);
  const int c_end = SK ? min(pt.c_end, nchunks)
                       : static_cast<int>(static_cast<int64_t>(nchunks) * (pt.split + 1) /
                                          pt.num_split);

  const uint16_t* kb = p.k + b * p.sb + h * p.sh;
  const uint16_t* vb = p.v + b * p.sb + h * p.sh;

  // q of head ln as the B operand of the score MFMA (zero for padding heads).
  uint4 qop[KS];
  {
    const uint16_t* qb = p.q + (static_cast<int64_t>(b) * p.Hq + h * G) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qop[s] = (ln < G) ? ld16(qb + ln * D + 32 * s + 8 * lq) : make_uint4(0u, 0u, 0u, 0u);
  }

  float m_run = -INFINITY;  // running max of head ln (log2 units)
  float l_run = 0.f;        // running sum over this lane's tokens of head ln
  f32x4_t oacc[VH * 4];
#pragma unroll
  for (int t = 0; t < VH * 4; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int last = L - 1;
  __syncthreads();

  for (int c = c_begin + w; c < c_end; c += NW) {
    const int slot = c / CPB;
    const int blk = DENSE ? slot : (slot < kIdxLds ? s_idx[slot] : idx[slot]);
    const int base = blk * BS + (c - slot * CPB) * (16 * TPC);
    if (blk < 0 || blk >= nblk || base >= L) continue;  // invalid entry: skipped
    // row 0 of the chunk's block in the cache
    const uint16_t* kc;
    const uint16_t* vc;
    if constexpr (PAGED) {
      if (blk >= p.table_stride) continue;
      const int page = blk < kTableLds
                           ? s_table[blk]
                           : p.block_table[static_cast<int64_t>(b) * p.table_stride + blk];
      if (page < 0 || page >= p.num_pages) continue;  // invalid page: skipped as well
      kc = p.k + page * p.page_stride + h * p.page_head_stride;
      vc = p.v + page * p.page_stride + h * p.page_head_stride;
    } else {
      kc = kb + static_cast<int64_t>(blk) * BS * p.st;
      vc = vb + static_cast<int64_t>(blk) * BS * p.st;
    }
    // first token of each of the chunk's tiles, or -1 past the sequence
    int tok0[TPC];
#pragma unroll
    for (int nt = 0; nt < TPC; ++nt) tok0[nt] = (base + 16 * nt < L) ? base + 16 * nt : -1;

    // K rows tok0 + ln, dims 32*s + 8*lq .. +7 (the A operand).
    uint4 kr[TPC][KS];
#pragma unroll
    for (int nt = 0; nt < TPC; ++nt) {
      if (tok0[nt] >= 0) {
        const int row = min(tok0[nt] + ln, last) - blk * BS;  // within the block
        const uint16_t* kp = kc + row * p.st + 8 * lq;
#pragma unroll
        for (int s = 0; s < KS; ++s) kr[nt][s] = ld16(kp + 32 * s);
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) kr[nt][s] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // V rows tok0 + 4*lq + r, dims 64*hh + 4*ln .. +3.
    uint2 vr[TPC][4][VH];
#pragma unroll
    for (int nt = 0; nt < TPC; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (tok0[nt] >= 0) {
          const int row = min(tok0[nt] + 4 * lq + r, last) - blk * BS;
          const uint16_t* vp = vc + row * p.st + 4 * ln;
#pragma unroll
          for (int hh = 0; hh < VH; ++hh) vr[nt][r][hh] = ld8_stream(vp + 64 * hh);
        } else {
#pragma unroll
          for (int hh = 0; hh < VH; ++hh) vr[nt][r][hh] = make_uint2(0u, 0u);
        }
      }
    // Keep all K and V loads of the chunk in flight together: nothing below
    // may be scheduled above this point.
    __builtin_amdgcn_sched_barrier(0);

    // Scores: sc[nt][r] = S[token tok0[nt] + 4 lq + r][head ln].
    f32x4_t sc[TPC];
#pragma unroll
    for (int nt = 0; nt < TPC; ++nt) {
      sc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sc[nt] = mfma16x16x32(kr[nt][s], qop[s], sc[nt]);
    }

    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < TPC; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tok0[nt] + 4 * lq + r;
        float x = sc[nt][r] * p.scale_log2;
        x = (tok0[nt] >= 0 && tok <= last) ? x : -INFINITY;
        sc[nt][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = max_xor<32>(max_xor<16>(mx));
    const float m_new = fmaxf(m_run, mx);  // finite: some tile holds a valid token
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    // Probabilities, rounded to bf16 once; the row sum uses the rounded
    // values so that O is an exact convex combination of the V rows.
    uint32_t pk[TPC][2];
    float psum = 0.f;
#pragma unroll
    for (int nt = 0; nt < TPC; ++nt)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const float p0 = fast_exp2(sc[nt][2 * rr] - m_new);
        const float p1 = fast_exp2(sc[nt][2 * rr + 1] - m_new);
        const uint32_t u = f2bf2(p0, p1);
        pk[nt][rr] = u;
        psum += bf_lo(u) + bf_hi(u);
      }
    l_run = l_run * alpha + psum;

    // Rescale the O rows: row 4*lq + r2 belongs to head 4*lq + r2, whose
    // alpha sits in lane 4*lq + r2.
#pragma unroll
    for (int r2 = 0; r2 < 4; ++r2) {
      const float a = __shfl(alpha, 4 * lq + r2);
#pragma unroll
      for (int t = 0; t < VH * 4; ++t) oacc[t][r2] *= a;
    }

    // O[head][64 hh + 4 ln + j] += P[head][tokens] . V[tokens][..]; the 8
    // tokens of k-group lq in step s2 are tok0[2 s2 + kk/4] + 4 lq + kk%4.
#pragma unroll
    for (int s2 = 0; s2 < TPC / 2; ++s2) {
      const uint4 pa = make_uint4(pk[2 * s2][0], pk[2 * s2][1], pk[2 * s2 + 1][0], pk[2 * s2 + 1][1]);
#pragma unroll
      for (int hh = 0; hh < VH; ++hh)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint4 vbop;
          vbop.x = pick2(vr[2 * s2][0][hh], vr[2 * s2][1][hh], j);
          vbop.y = pick2(vr[2 * s2][2][hh], vr[2 * s2][3][hh], j);
          vbop.z = pick2(vr[2 * s2 + 1][0][hh], vr[2 * s2 + 1][1][hh], j);
          vbop.w = pick2(vr[2 * s2 + 1][2][hh], vr[2 * s2 + 1][3][hh], j);
          oacc[hh * 4 + j] = mfma16x16x32(pa, vbop, oacc[hh * 4 + j]);
        }
    }
  }

  // ---- merge the waves of this split
  l_run = sum_xor<32>(sum_xor<16>(l_run));
  if (lq == 0) {
    sm_m[w][ln] = m_run;
    sm_l[w][ln] = l_run;
  }
#pragma unroll
  for (int hh = 0; hh < VH; ++hh)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r2 = 0; r2 < 4; ++r2) {
        const int head = 4 * lq + r2;
        if (head < G) sm_o[(w * G + head) * D + 64 * hh + 4 * ln + j] = oacc[hh * 4 + j][r2];
      }
  __syncthreads();

  const int nel = G * D;
  const int64_t out_base = static_cast<int64_t>(b) * p.Hq + h * G;
  const int64_t part = pt.my_slot;
  for (int e = tid; e < nel; e += NW * 64) {
    const int head = e / D;
    const int dim = e - head * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][head]);
    float osum = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = sm_m[ww][head];
        const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        osum += f * sm_o[(ww * G + head) * D + dim];
        lsum += f * sm_l[ww][head];
      }
    }
    const bool any = lsum > 0.f;
    const float o = any ? osum / lsum : 0.f;
    if (pt.nparts == 1) {
      p.out[(out_base + head) * D + dim] = f2bf(o);
      if (dim == 0 && p.lse != nullptr)
        p.lse[out_base + head] = any ? (M + fast_log2(lsum)) * kLn2 : -INFINITY;
    } else {
      // device-coherent stores (they write through the per-XCD L2)
      __hip_atomic_store(&p.part_o[(part * G + head) * D + dim], o, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (dim == 0)
        __hip_atomic_store(&p.part_lse[part * G + head], any ? M + fast_log2(lsum) : -INFINITY,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (pt.nparts == 1) return;

  // ---- the last split of this (b, h) to finish merges all splits.
  // Partials travel only through device-coherent stores and loads, so the
  // hand-off needs no cache write-back or invalidation: each thread waits
  // until its stores are performed, the workgroup then counts itself on a
  // device-scope counter, and the workgroup that completes the count reads
  // the partials back coherently.
  __shared__ int sm_last;
  __shared__ float sm_w[kMaxSplit * 16];
  __shared__ float sm_lse[16];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(p.counters + pair, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    sm_last = (prev == pt.nparts - 1);
  }
  __syncthreads();
  if (!sm_last) return;
  const int S = pt.nparts;
  auto slot_of = [&](int k) -> int64_t { return k == 0 ? pt.slot0 : pt.slot1 + (k - 1) * pt.slot_step; };
  if (S <= kMergeInline) {
    // one round trip: each element's S partial outputs and its head's S
    // partial lse values are requested together; the weights are formed per
    // element, in the same order as below
    for (int e = tid; e < nel; e += NW * 64) {
      const int head = e / D;
      const int dim = e - head * D;
      float ls[kMergeInline], os[kMergeInline];
#pragma unroll
      for (int s = 0; s < kMergeInline; ++s) {
        if (s < S) {
          const int64_t sl = slot_of(s);
          ls[s] = __hip_atomic_load(p.part_lse + sl * G + head, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
          os[s] = __hip_atomic_load(p.part_o + (sl * G + head) * D + dim, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      float M = -INFINITY;
#pragma unroll
      for (int s = 0; s < kMergeInline; ++s)
        if (s < S) M = fmaxf(M, ls[s]);
      float f[kMergeInline];
      float tot = 0.f;
#pragma unroll
      for (int s = 0; s < kMergeInline; ++s) {
        f[s] = (s < S && M != -INFINITY && ls[s] != -INFINITY) ? fast_exp2(ls[s] - M) : 0.f;
        tot += f[s];
      }
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
      float o = 0.f;
#pragma unroll
      for (int s = 0; s < kMergeInline; ++s)
        if (s < S) o += (f[s] * inv) * os[s];
      p.out[(out_base + head) * D + dim] = f2bf(o);
      if (dim == 0 && p.lse != nullptr)
        p.lse[out_base + head] = tot > 0.f ? (M + fast_log2(tot)) * kLn2 : -INFINITY;
    }
  } else if (S <= kMaxSplit) {
    for (int i = tid; i < S * G; i += NW * 64)
      sm_w[i] = __hip_atomic_load(p.part_lse + slot_of(i / G) * G + i % G, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (tid < G) {
      const int head = tid;
      float M = -INFINITY;
      for (int s = 0; s < S; ++s) M = fmaxf(M, sm_w[s * G + head]);
      float tot = 0.f;
      for (int s = 0; s < S; ++s) {
        const float ls = sm_w[s * G + head];
        const float f = (M == -INFINITY || ls == -INFINITY) ? 0.f : fast_exp2(ls - M);
        sm_w[s * G + head] = f;
        tot += f;
      }
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
      for (int s = 0; s < S; ++s) sm_w[s * G + head] *= inv;
      sm_lse[head] = tot > 0.f ? (M + fast_log2(tot)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    for (int e = tid; e < nel; e += NW * 64) {
      const int head = e / D;
      const int dim = e - head * D;
      float o = 0.f;
      for (int s = 0; s < S; ++s)
        o += sm_w[s * G + head] * __hip_atomic_load(p.part_o + (slot_of(s) * G + head) * D + dim,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      p.out[(out_base + head) * D + dim] = f2bf(o);
      if (dim == 0 && p.lse != nullptr) p.lse[out_base + head] = sm_lse[head];
    }
  } else {
    // More parts than the weights held in LDS (a stream-K pair cut over
    // many workgroups): the same weights, in the same order, formed and
    // applied kMaxSplit parts at a time.
    __shared__ float sm_mx[16];
    __shared__ float sm_inv[16];
    if (tid < G) {
      const int head = tid;
      float M = -INFINITY;
      for (int s = 0; s < S; ++s)
        M = fmaxf(M, __hip_atomic_load(p.part_lse + slot_of(s) * G + head, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT));
      float tot = 0.f;
      for (int s = 0; s < S; ++s) {
        const float ls = __hip_atomic_load(p.part_lse + slot_of(s) * G + head, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        tot += (M == -INFINITY || ls == -INFINITY) ? 0.f : fast_exp2(ls - M);
      }
      sm_mx[head] = M;
      sm_inv[head] = tot > 0.f ? 1.f / tot : 0.f;
      sm_lse[head] = tot > 0.f ? (M + fast_log2(tot)) * kLn2 : -INFINITY;
    }
    constexpr int EPT = (kMaxGroup * D + NW * 64 - 1) / (NW * 64);
    float acc[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) acc[i] = 0.f;
    for (int s0 = 0; s0 < S; s0 += kMaxSplit) {
      const int ns = min(kMaxSplit, S - s0);
      __syncthreads();  // sm_mx, sm_inv ready; the previous batch's weights consumed
      for (int i = tid; i < ns * G; i += NW * 64) {
        const int head = i % G;
        const float ls = __hip_atomic_load(p.part_lse + slot_of(s0 + i / G) * G + head,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float M = sm_mx[head];
        sm_w[i] = ((M == -INFINITY || ls == -INFINITY) ? 0.f : fast_exp2(ls - M)) * sm_inv[head];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int e = tid + i * NW * 64;
        if (e >= nel) break;
        const int head = e / D;
        const int dim = e - head * D;
        for (int s = 0; s < ns; ++s)
          acc[i] += sm_w[s * G + head] *
                    __hip_atomic_load(p.part_o + (slot_of(s0 + s) * G + head) * D + dim,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + i * NW * 64;
      if (e >= nel) break;
      const int head = e / D;
      const int dim = e - head * D;
      p.out[(out_base + head) * D + dim] = f2bf(acc[i]);
      if (dim == 0 && p.lse != nullptr) p.lse[out_base + head] = sm_lse[head];
    }
  }
  if (tid == 0) __hip_atomic_store(p.counters + pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Index of the stream-K workgroup whose chunk range holds global chunk x:
// workgroup w takes [floor(w T / N), floor((w + 1) T / N)).
__device__ __forceinline__ int sk_group_of(int x, int T, int N) {
  return min(static_cast<int>((static_cast<int64_t>(x + 1) * N - 1) / T), N - 1);
}

// Fixed splits: workgroup = (pair, split).  Stream-K (uneven selections):
// every workgroup takes an equal share of all pairs' active chunks, found
// from a prefix over num_selected, and decodes the pairs that share overlaps
// one after another.  A pair inside one share writes its output directly; a
// pair cut between shares is merged by the last of its parts to finish, as
// fixed splits are.  Nothing waits on another workgroup in either scheme.
template <int D, int BS, bool DENSE, int NW, bool PAGED, bool SK>
__global__ __launch_bounds__(NW * 64, 2) void decode_kernel(DecodeParams p) {
  extern __shared__ float sm_o[];  // [NW][G][D]
  const int tid = threadIdx.x;

  // Fused step: the cache entries appended by this step's gate launch are
  // counted now, after every reader of the old count has finished.
  if (p.commit_lens != nullptr && blockIdx.x == 0) {
    for (int bb = tid; bb < p.B; bb += NW * 64)
      p.commit_lens[bb] = committed_count(p.seq_lens[bb], p.commit_lens[bb], p.BS, p.Lmax, p.NBmax,
                                          p.commit_max_new);
  }

  if constexpr (!SK) {
    Part pt{};
    pt.num_split = p.num_split;
    pt.pair = blockIdx.x / pt.num_split;
    pt.split = blockIdx.x - pt.pair * pt.num_split;
    pt.nparts = pt.num_split;
    pt.slot0 = static_cast<int64_t>(pt.pair) * pt.num_split;
    pt.my_slot = pt.slot0 + pt.split;
    pt.slot1 = pt.slot0 + 1;
    pt.slot_step = 1;
    decode_part<D, BS, DENSE, NW, PAGED, false>(p, pt, sm_o);
  } else {
    static_assert(!DENSE, "stream-K division is for selections");
    constexpr int CPB = BS / (16 * kTilesPerChunk);
    constexpr int NT = NW * 64;
    __shared__ int s_pre[kSkMaxPairs + 1];  // prefix of the pairs' chunk counts
    __shared__ int s_run[NT];
    const int P = p.B * p.Hkv;  // at most kSkMaxPairs (checked on the host)
    const int per = (P + NT - 1) / NT;
    const int i0 = min(tid * per, P);
    const int i1 = min(i0 + per, P);
    int run = 0;
    for (int i = i0; i < i1; ++i) {
      const int n = min(max(p.num_selected[i], 0), p.max_sel) * CPB;
      s_pre[i + 1] = n;
      run += n;
    }
    s_run[tid] = run;
    __syncthreads();
    if (tid < 64) {  // wave 0: exclusive scan of the NT per-thread totals
      int v[NW];
      int t = 0;
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        v[j] = s_run[tid * NW + j];
        t += v[j];
      }
      int incl = t;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (tid >= o) incl += y;
      }
      int ex = incl - t;
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        s_run[tid * NW + j] = ex;
        ex += v[j];
      }
    }
    __syncthreads();
    {
      int acc = s_run[tid];
      if (tid == 0) s_pre[0] = 0;
      for (int i = i0; i < i1; ++i) {
        acc += s_pre[i + 1];
        s_pre[i + 1] = acc;
      }
    }
    __syncthreads();
    const int T = s_pre[P];
    const int grid = static_cast<int>(gridDim.x);
    const int wg = static_cast<int>(blockIdx.x);
    const int G = p.G;
    // pairs without an active chunk: output 0, lse -inf
    for (int q = wg; q < P; q += grid) {
      if (s_pre[q + 1] != s_pre[q]) continue;
      const int bq = q / p.Hkv;
      const int64_t ob = static_cast<int64_t>(bq) * p.Hq + (q - bq * p.Hkv) * G;
      for (int e = tid; e < G * D; e += NT) p.out[ob * D + e] = 0;
      if (tid < G && p.lse != nullptr) p.lse[ob + tid] = -INFINITY;
    }
    const int N = min(grid, T);  // every one of these shares is non-empty
    if (wg >= N) return;
    const int lo = static_cast<int>(static_cast<int64_t>(wg) * T / N);
    const int hi = static_cast<int>(static_cast<int64_t>(wg + 1) * T / N);
    int q = 0;  // first pair ending past lo
    for (int z = P - 1; q < z;) {
      const int m = (q + z) >> 1;
      if (s_pre[m + 1] > lo) z = m; else q = m + 1;
    }
    for (; q < P && s_pre[q] < hi; ++q) {
      const int base = s_pre[q];
      const int cnt = s_pre[q + 1] - base;
      if (cnt == 0) continue;
      const int w0 = sk_group_of(base, T, N);
      Part pt{};
      pt.pair = q;
      pt.c_begin = max(lo, base) - base;
      pt.c_end = min(hi, base + cnt) - base;
      pt.nparts = sk_group_of(base + cnt - 1, T, N) - w0 + 1;
      // slot 2w holds the part of the pair a share starts in, 2w + 1 the
      // part of the pair that starts inside the share and runs past it
      pt.slot0 = 2 * static_cast<int64_t>(w0) +
                 (base == static_cast<int>(static_cast<int64_t>(w0) * T / N) ? 0 : 1);
      pt.slot1 = 2 * static_cast<int64_t>(w0 + 1);
      pt.slot_step = 2;
      pt.my_slot = (wg == w0) ? pt.slot0 : 2 * static_cast<int64_t>(wg);
      decode_part<D, BS, false, NW, PAGED, true>(p, pt, sm_o);
    }
  }
}

template <int D, int BS, bool DENSE, int NW, bool PAGED, bool SK = false>
void launch_one(const DecodeParams& p, int grid, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(NW) * p.G * D * sizeof(float);
  hipLaunchKernelGGL((decode_kernel<D, BS, DENSE, NW, PAGED, SK>), dim3(grid), dim3(NW * 64), lds,
                     stream, p);
}

// stream-K: selections over a contiguous cache
template <int NW>
void launch_variant_sk(int key, const DecodeParams& p, int grid, hipStream_t s) {
  switch (key) {
    case 0: launch_one<64, 64, false, NW, false, true>(p, grid, s); break;
    case 2: launch_one<64, 128, false, NW, false, true>(p, grid, s); break;
    case 4: launch_one<128, 64, false, NW, false, true>(p, grid, s); break;
    default: launch_one<128, 128, false, NW, false, true>(p, grid, s); break;
  }
}

template <int NW, bool PAGED>
void launch_variant(int key, const DecodeParams& p, int grid, hipStream_t s) {
  switch (key) {
    case 0: launch_one<64, 64, false, NW, PAGED>(p, grid, s); break;
    case 1: launch_one<64, 64, true, NW, PAGED>(p, grid, s); break;
    case 2: launch_one<64, 128, false, NW, PAGED>(p, grid, s); break;
    case 3: launch_one<64, 128, true, NW, PAGED>(p, grid, s); break;
    case 4: launch_one<128, 64, false, NW, PAGED>(p, grid, s); break;
    case 5: launch_one<128, 64, true, NW, PAGED>(p, grid, s); break;
    case 6: launch_one<128, 128, false, NW, PAGED>(p, grid, s); break;
    default: launch_one<128, 128, true, NW, PAGED>(p, grid, s); break;
  }
}

}  // namespace

int launch_decode(const seer_dims& d, const DecodeArgs& a, void* stream) {
  const int64_t pairs = static_cast<int64_t>(d.batch) * d.num_kv_heads;
  const int G = d.num_q_heads / d.num_kv_heads;
  const int S = a.num_split;
  DecodeParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.seq_lens = a.seq_lens;
  p.block_idx = a.block_idx;
  p.num_selected = a.num_selected;
  p.out = a.out;
  p.lse = a.lse;
  p.sb = d.kv_stride_b;
  p.sh = d.kv_stride_h;
  p.st = static_cast<int>(d.kv_stride_t);
  p.Hq = d.num_q_heads;
  p.Hkv = d.num_kv_heads;
  p.G = G;
  p.Lmax = d.max_seq_len;
  p.max_sel = a.max_selected;
  p.num_split = S;
  p.scale_log2 = a.scale * kLog2e;
  p.commit_lens = a.commit_lens;
  p.commit_max_new = a.commit_max_new;
  p.B = d.batch;
  p.BS = d.block_size;
  p.NBmax = static_cast<int>(nb_max(&d));
  p.block_table = a.block_table;
  p.table_stride = a.table_stride;
  p.num_pages = a.num_pages;
  p.page_stride = a.page_stride;
  p.page_head_stride = a.page_head_stride;
  const bool dense = (a.block_idx == nullptr);
  const bool paged = a.block_table != nullptr;
  const int nw = decode_waves_per_group(G, d.head_dim);
  // stream-K where it applies: a selection over a contiguous cache, with the
  // pairs' prefix and the wave merge both in LDS
  const bool sk = a.stream_k && !dense && !paged && pairs <= kSkMaxPairs &&
                  static_cast<int64_t>(nw) * G * d.head_dim * 4 <= kSkMergeLds;
  if (S > 1 || sk) {
    char* ws = static_cast<char*>(a.workspace);
    size_t cbytes = static_cast<size_t>(pairs) * sizeof(int32_t);
    cbytes = (cbytes + kCounterBytes - 1) / kCounterBytes * kCounterBytes;
    // stream-K: two partial slots per workgroup
    size_t lbytes = static_cast<size_t>(pairs) * S * (sk ? 2 : 1) * G * sizeof(float);
    lbytes = (lbytes + kCounterBytes - 1) / kCounterBytes * kCounterBytes;
    p.counters = reinterpret_cast<int32_t*>(ws);
    p.part_lse = reinterpret_cast<float*>(ws + cbytes);
    p.part_o = reinterpret_cast<float*>(ws + cbytes + lbytes);
  }
  const int64_t grid64 = pairs * S;
  if (grid64 > 0x7fffffff) {
    set_error("decode grid too large");
    return SEER_ERR_UNSUPPORTED;
  }
  const int grid = static_cast<int>(grid64);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int key = (d.head_dim == 128 ? 4 : 0) | (d.block_size == 128 ? 2 : 0) | (dense ? 1 : 0);
  if (sk)
    nw == 8 ? launch_variant_sk<8>(key, p, grid, s) : launch_variant_sk<4>(key, p, grid, s);
  else if (nw == 8)
    paged ? launch_variant<8, true>(key, p, grid, s) : launch_variant<8, false>(key, p, grid, s);
  else
    paged ? launch_variant<4, true>(key, p, grid, s) : launch_variant<4, false>(key, p, grid, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("decode launch: ") + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  return SEER_OK;
}

}  // namespace seer
