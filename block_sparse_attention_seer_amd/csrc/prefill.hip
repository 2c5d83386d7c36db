// Causal prefill attention (a FlashAttention-2 forward) with the fused
// block-level ground truth of the AttnGate's distillation, for gfx950
// (MI355X).
//
// [CP Knowl 3] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): the training target of the gate is the
// original model's attention map, max-pooled over keys in blocks of b, then
// max-pooled over the query heads of each GQA group, then normalised to sum
// to 1 for every query.  [CP Knowl 4]: instead of building the O(L^2) map,
// the FlashAttention-2 forward stores each tile's row maximum r_ij of the
// scores and, once the row's final max m_i and normaliser l_i are known,
// turns it into exp(r_ij - m_i) / l_i -- the largest probability in the
// block, because exp is increasing.
//
// Kernels:
//   vt_kernel     V^T of every (sequence, KV head) into the workspace
//                 ([d][tokens], zero past the sequence), with the keys of
//                 each group of 16 stored as quads (0-3, 8-11, 4-7, 12-15):
//                 the order in which the score accumulators hold them, so
//                 the P.V operand of a lane is one 16-byte LDS read;
//   fa_fwd_kernel one workgroup of 8 waves per (sequence, query head, 256
//                 query rows); wave w owns 32 rows.  Per 64-key tile the
//                 workgroup stages K and V^T in LDS (double-buffered, one
//                 barrier per tile) and each wave computes
//                   S^T[key][query] = K . Q^T   (MFMA 32x32x16, B = Q rows
//                                                 held in registers)
//                   O^T[dim][query] += V^T . P^T (B = P^T straight from the
//                                                 score accumulators)
//                 so a lane holds one query's scores: its row max is a
//                 register max plus one exchange with the lane 32 away.
//                 That row max is r_ij (b = 64) or half of it (b = 128);
//                 lanes 0..31 store it for 32 consecutive queries, one
//                 128-byte run.  The online softmax rescales only when a
//                 row max grows by more than 2^8 (p stays <= 256, exact in
//                 the end because the final normalisation uses the same m);
//   gt_kernel     one workgroup per (sequence, KV head, 64 query rows):
//                 exp2(r - lse) of every head of the group, its max over the
//                 group, the row sum, then the normalised rows through an
//                 LDS transpose (coalesced stores of the [rows][blocks]
//                 target).  Blocks after the query are 0.
// The workgroup order is XCD-aware and longest-first: the 8 XCDs take
// contiguous ranges of the work list, which runs (sequence, KV head) by
// (sequence, KV head), query tiles from the last (most keys) to the first,
// so each XCD's L2 serves the K/V tiles its concurrent workgroups share.
#include "seer_device.hpp"
#include "seer_internal.h"

namespace seer {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).  Lane l supplies
// A[l%32][8(l/32) .. +7] and B[8(l/32) .. +7][l%32]; it receives
// D[8(i/4) + 4(l/32) + i%4][l%32] in element i.
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = kWaves * 32;  // query rows per workgroup
constexpr int kKeys = 64;           // keys per tile
constexpr int kRowTile = kPrefillTokenTile;  // tokens per workgroup of vt_kernel / gt_kernel
constexpr float kLazy = 8.f;        // rescale when a row max grows by more than this (log2)

struct PrefillParams {
  const uint16_t* q;  // [B, Hq, Lmax, D]
  const uint16_t* k;  // [B, Hkv, Lmax, D] with the strides below
  const uint16_t* v;
  const int32_t* seq_lens;
  uint16_t* vt;       // [B, Hkv, D, Lpad]
  float* r;           // [B, Hq, NBmax, Lpad] block row maxima (log2 units), or null
  uint16_t* out;      // [B, Hq, Lmax, D]
  float* lse;         // [B, Hq, Lmax]
  float* gt;          // [B, Hkv, Lmax, NBmax]
  int64_t sb, sh;
  int st;
  int Hq, Hkv, G, Lmax, Lpad, NBmax, n_qtiles;
  float scale_log2;
};

// Stored position -> key within a group of 16 (quads 0, 2, 1, 3).
__device__ __forceinline__ int key_of_pos(int pos) {
  const int quad = (pos >> 2) & 3;
  const int kq = quad == 1 ? 2 : (quad == 2 ? 1 : quad);
  return (pos & ~15) + 4 * kq + (pos & 3);
}

template <int D>
__global__ __launch_bounds__(256) void vt_kernel(PrefillParams p) {
  const int t0 = blockIdx.x * kRowTile;
  const int pair = blockIdx.y;
  const int b = pair / p.Hkv, h = pair % p.Hkv;
  const int L = min(max(p.seq_lens[b], 0), p.Lmax);
  __shared__ __align__(16) uint16_t s[kRowTile][D + 8];
  const uint16_t* vb = p.v + b * p.sb + h * p.sh;
  for (int i = threadIdx.x; i < kRowTile * D / 8; i += 256) {
    const int row = i / (D / 8), c8 = i % (D / 8);
    const int tok = t0 + row;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (tok < L) val = ld16(vb + static_cast<int64_t>(tok) * p.st + 8 * c8);
    *reinterpret_cast<uint4*>(&s[row][8 * c8]) = val;
  }
  __syncthreads();
  uint16_t* vtb = p.vt + static_cast<int64_t>(pair) * D * p.Lpad + t0;
  for (int i = threadIdx.x; i < D * (kRowTile / 8); i += 256) {
    const int d = i / (kRowTile / 8), pc = i % (kRowTile / 8);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 8 * pc + 2 * e;
      w[e] = static_cast<uint32_t>(s[key_of_pos(pos)][d]) |
             (static_cast<uint32_t>(s[key_of_pos(pos + 1)][d]) << 16);
    }
    *reinterpret_cast<uint4*>(vtb + static_cast<int64_t>(d) * p.Lpad + 8 * pc) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// This thread's share of one K tile and one V^T tile (16-byte pieces).
template <int D>
struct TileRegs {
  static constexpr int KP = kKeys * D / 8 / kThreads;
  static constexpr int VP = D * kKeys / 8 / kThreads;
  uint4 k[KP];
  uint4 v[VP];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& t, const uint16_t* kb, const uint16_t* vtb,
                                          int64_t st, int Lpad, int key0, int L, int tid) {
#pragma unroll
  for (int i = 0; i < TileRegs<D>::KP; ++i) {
    const int piece = tid + i * kThreads;
    const int row = piece / (D / 8), c8 = piece % (D / 8);
    const int key = key0 + row;
    t.k[i] = key < L ? ld16(kb + key * st + 8 * c8) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::VP; ++i) {
    const int piece = tid + i * kThreads;
    const int d = piece / (kKeys / 8), c = piece % (kKeys / 8);
    t.v[i] = ld16(vtb + static_cast<int64_t>(d) * Lpad + key0 + 8 * c);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, uint16_t* sk, uint16_t* sv,
                                           int tid) {
  constexpr int KROW = D + 8, VROW = kKeys + 8;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::KP; ++i) {
    const int piece = tid + i * kThreads;
    const int row = piece / (D / 8), c8 = piece % (D / 8);
    *reinterpret_cast<uint4*>(sk + row * KROW + 8 * c8) = t.k[i];
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::VP; ++i) {
    const int piece = tid + i * kThreads;
    const int d = piece / (kKeys / 8), c = piece % (kKeys / 8);
    *reinterpret_cast<uint4*>(sv + d * VROW + 8 * c) = t.v[i];
  }
}

template <int D, int BS, bool GT>
__global__ __launch_bounds__(kThreads) void fa_fwd_kernel(PrefillParams p) {
  constexpr int KS = D / 16;  // k-steps of S^T = K Q^T
  constexpr int DT = D / 32;  // 32-row tiles of O^T
  constexpr int KROW = D + 8, VROW = kKeys + 8;
  __shared__ __align__(16) uint16_t s_k[2][kKeys * KROW];
  __shared__ __align__(16) uint16_t s_v[2][D * VROW];

  // ---- work item: XCD x takes a contiguous range of the work list
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, kk = blockIdx.x / 8;
  const int wi = xcd * (nwg / 8) + min(xcd, nwg % 8) + kk;
  const int per_kv = p.n_qtiles * p.G;
  const int kvp = wi / per_kv, rem = wi % per_kv;
  const int qt = p.n_qtiles - 1 - rem / p.G;
  const int hq = (kvp % p.Hkv) * p.G + rem % p.G;
  const int b = kvp / p.Hkv;

  const int L = min(max(p.seq_lens[b], 0), p.Lmax);
  const int q0 = qt * kRows;
  if (q0 >= L) return;
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64, hf = l / 32, ln = l % 32;
  const int qrow = q0 + 32 * w + ln;
  const int wfirst = q0 + 32 * w;
  // key tiles the workgroup stages, and those this wave computes (its 32
  // rows share their last tile)
  const int ntiles = (min(q0 + kRows, L) - 1) / kKeys + 1;
  const int wtiles = wfirst < L ? wfirst / kKeys + 1 : 0;

  const uint16_t* kb = p.k + b * p.sb + (hq / p.G) * p.sh;
  const uint16_t* vtb = p.vt + static_cast<int64_t>(b * p.Hkv + hq / p.G) * D * p.Lpad;
  TileRegs<D> regs;
  load_tile<D>(regs, kb, vtb, p.st, p.Lpad, 0, L, tid);

  // this lane's query row as the B operand (dims 16 ks + 8 hf .. +7)
  uint4 qop[KS];
  {
    const uint16_t* qr = p.q + ((static_cast<int64_t>(b) * p.Hq + hq) * p.Lmax + qrow) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = qrow < L ? ld16(qr + 16 * ks + 8 * hf) : make_uint4(0u, 0u, 0u, 0u);
  }
  store_tile<D>(regs, s_k[0], s_v[0], tid);
  __syncthreads();

  f32x16_t oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
  float m_run = -INFINITY;  // this row's reference max (log2 units)
  float l_part = 0.f;       // this lane's share of the row's normaliser
  float r_blk = -INFINITY;  // b = 128: max over the block's first tile
  float* rrow = GT ? p.r + (static_cast<int64_t>(b) * p.Hq + hq) * p.NBmax * p.Lpad + qrow
                   : nullptr;

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile<D>(regs, kb, vtb, p.st, p.Lpad, (j + 1) * kKeys, L, tid);
    if (j < wtiles) {
      const uint16_t* sk = s_k[buf];
      const uint16_t* sv = s_v[buf];
      // ---- S^T for keys 64 j + 32 mt + (8(i/4) + 4 hf + i%4), query ln
      // (both contractions alternate their independent accumulators, so no
      // MFMA waits on the one just issued; each accumulator still takes its
      // k-steps in order)
      f32x16_t sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[mt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint4 a = *reinterpret_cast<const uint4*>(sk + (32 * mt + ln) * KROW + 16 * ks +
                                                          8 * hf);
          sacc[mt] = mfma32(a, qop[ks], sacc[mt]);
        }
      // ---- causal mask, tile row max (raw scores; the scale is positive,
      // so scaling commutes with the max and goes into the exponent below)
      if (j * kKeys + kKeys - 1 > wfirst) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j * kKeys + 32 * mt + 8 * (i / 4) + 4 * hf + (i % 4);
            sacc[mt][i] = key > qrow ? -INFINITY : sacc[mt][i];
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[mt][i]);
      tmax = max_xor<32>(tmax) * p.scale_log2;
      if constexpr (GT) {
        if (BS == kKeys) {
          if (hf == 0 && qrow < L) rrow[static_cast<int64_t>(j) * p.Lpad] = tmax;
        } else {
          const bool odd = j & 1;
          const float rb = odd ? fmaxf(r_blk, tmax) : tmax;
          r_blk = rb;
          if ((odd || j == wtiles - 1) && hf == 0 && qrow < L)
            rrow[static_cast<int64_t>(j / 2) * p.Lpad] = rb;
        }
      }
      // ---- online softmax with lazy rescaling
      if (__builtin_amdgcn_ballot_w64(tmax > m_run + kLazy)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
        l_part *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[t][i] *= alpha;
        m_run = m_new;
      }
      const float mref = m_run == -INFINITY ? 0.f : m_run;
      uint4 pb[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pv[i] = fast_exp2(fmaf(sacc[mt][i], p.scale_log2, -mref));
          l_part += pv[i];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
          pb[2 * mt + c] = make_uint4(f2bf2(pv[8 * c + 0], pv[8 * c + 1]),
                                      f2bf2(pv[8 * c + 2], pv[8 * c + 3]),
                                      f2bf2(pv[8 * c + 4], pv[8 * c + 5]),
                                      f2bf2(pv[8 * c + 6], pv[8 * c + 7]));
      }
      // ---- O^T += V^T P^T (keys in the stored quad order of vt_kernel)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const uint4 a = *reinterpret_cast<const uint4*>(sv + (32 * t + ln) * VROW + 16 * ks +
                                                          8 * hf);
          oacc[t] = mfma32(a, pb[ks], oacc[t]);
        }
    }
    if (j + 1 < ntiles) store_tile<D>(regs, s_k[buf ^ 1], s_v[buf ^ 1], tid);
    __syncthreads();
  }

  if (qrow >= L) return;
  const float lsum = sum_xor<32>(l_part);
  const float inv = 1.f / lsum;
  uint16_t* orow = p.out + ((static_cast<int64_t>(b) * p.Hq + hq) * p.Lmax + qrow) * D;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * t + 8 * g4 + 4 * hf;
      uint2 pk;
      pk.x = f2bf2(oacc[t][4 * g4 + 0] * inv, oacc[t][4 * g4 + 1] * inv);
      pk.y = f2bf2(oacc[t][4 * g4 + 2] * inv, oacc[t][4 * g4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d) = pk;
    }
  if (hf == 0)
    p.lse[(static_cast<int64_t>(b) * p.Hq + hq) * p.Lmax + qrow] =
        (m_run + fast_log2(lsum)) * kLn2;
}

template <int BS>
__global__ __launch_bounds__(256) void gt_kernel(PrefillParams p) {
  const int i0 = blockIdx.x * kRowTile;
  const int pair = blockIdx.y;
  const int b = pair / p.Hkv, hkv = pair % p.Hkv;
  const int L = min(max(p.seq_lens[b], 0), p.Lmax);
  if (i0 >= L) return;
  __shared__ float s_lse[kMaxGroup][kRowTile];
  __shared__ float s_part[4][kRowTile];
  __shared__ float s_g[kRowTile][kRowTile + 1];
  const int t = threadIdx.x % kRowTile, jj = threadIdx.x / kRowTile;
  const int tok = i0 + t;
  const bool valid = tok < L;
  const int nvis = valid ? tok / BS + 1 : 0;
  const int nvis_max = (min(i0 + kRowTile, L) - 1) / BS + 1;
  const int G = p.G;
  for (int i = threadIdx.x; i < G * kRowTile; i += 256) {
    const int hg = i / kRowTile, tt = i % kRowTile;
    const int hq = hkv * G + hg;
    s_lse[hg][tt] = i0 + tt < L
                        ? p.lse[(static_cast<int64_t>(b) * p.Hq + hq) * p.Lmax + i0 + tt] * kLog2e
                        : 0.f;
  }
  __syncthreads();
  const float* rb = p.r + (static_cast<int64_t>(b) * p.Hq + hkv * G) * p.NBmax * p.Lpad + tok;
  const int64_t head_stride = static_cast<int64_t>(p.NBmax) * p.Lpad;

  // ---- pass 1: the group maxima, unnormalised, straight into the target
  // rows (64 blocks at a time through LDS, coalesced stores), and their row
  // sums (fixed order: j by j within a thread, then the four threads of a
  // row in order).  r is read once.
  float* gtb = p.gt + (static_cast<int64_t>(pair) * p.Lmax + i0) * p.NBmax;
  const int rows = min(kRowTile, L - i0);
  float sum = 0.f;
  constexpr int MPT = kRowTile / 4;  // blocks of a 64-block chunk per thread
  for (int c0 = 0; c0 < p.NBmax; c0 += kRowTile) {
    if (c0 < nvis_max) {
      // head by head, the MPT loads of a head are independent and issued
      // together (indices clamped into the buffer; blocks after the query
      // are masked to 0 below)
      float gm[MPT];
#pragma unroll
      for (int mi = 0; mi < MPT; ++mi) gm[mi] = 0.f;
      for (int hg = 0; hg < G; ++hg) {
        const float* rh = rb + hg * head_stride;
        const float lh = s_lse[hg][t];
        float x[MPT];
#pragma unroll
        for (int mi = 0; mi < MPT; ++mi) {
          const int j = min(c0 + jj + 4 * mi, p.NBmax - 1);
          x[mi] = rh[static_cast<int64_t>(j) * p.Lpad];
        }
#pragma unroll
        for (int mi = 0; mi < MPT; ++mi) gm[mi] = fmaxf(gm[mi], fast_exp2(x[mi] - lh));
      }
#pragma unroll
      for (int mi = 0; mi < MPT; ++mi) {
        const int m = jj + 4 * mi;
        const float v = (c0 + m < nvis) ? gm[mi] : 0.f;
        sum += v;
        s_g[t][m] = v;
      }
    } else {
      for (int m = jj; m < kRowTile; m += 4) s_g[t][m] = 0.f;
    }
    __syncthreads();
    const int cols = min(kRowTile, p.NBmax - c0);
    for (int i = threadIdx.x; i < rows * kRowTile; i += 256) {
      const int row = i / kRowTile, col = i % kRowTile;
      if (col < cols) gtb[static_cast<int64_t>(row) * p.NBmax + c0 + col] = s_g[row][col];
    }
    __syncthreads();
  }
  s_part[jj][t] = sum;
  __syncthreads();
  if (threadIdx.x < kRowTile) {
    const float total = ((s_part[0][t] + s_part[1][t]) + s_part[2][t]) + s_part[3][t];
    s_lse[0][t] = total > 0.f ? 1.f / total : 0.f;  // reused: the row's 1/sum
  }
  __syncthreads();
  // ---- pass 2: normalise the visible part of this workgroup's rows (just
  // written by it, so read back from L2)
  const int vis_cols = min(p.NBmax, nvis_max);
  for (int i = threadIdx.x; i < rows * vis_cols; i += 256) {
    const int row = i / vis_cols, col = i % vis_cols;
    float* e = gtb + static_cast<int64_t>(row) * p.NBmax + col;
    *e = *e * s_lse[0][row];
  }
}

template <int D>
int launch_d(const seer_dims& d, const PrefillArgs& a, PrefillParams& p, hipStream_t s) {
  const int B = d.batch;
  hipLaunchKernelGGL((vt_kernel<D>), dim3(p.Lpad / kRowTile, B * p.Hkv), dim3(256), 0, s, p);
  const int nwg = B * p.Hq * p.n_qtiles;
  const bool gt = a.gt != nullptr;
  if (d.block_size == 64) {
    if (gt)
      hipLaunchKernelGGL((fa_fwd_kernel<D, 64, true>), dim3(nwg), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((fa_fwd_kernel<D, 64, false>), dim3(nwg), dim3(kThreads), 0, s, p);
  } else {
    if (gt)
      hipLaunchKernelGGL((fa_fwd_kernel<D, 128, true>), dim3(nwg), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((fa_fwd_kernel<D, 128, false>), dim3(nwg), dim3(kThreads), 0, s, p);
  }
  if (gt) {
    const dim3 grid((d.max_seq_len + kRowTile - 1) / kRowTile, B * p.Hkv);
    if (d.block_size == 64)
      hipLaunchKernelGGL((gt_kernel<64>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((gt_kernel<128>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

}  // namespace

int launch_prefill(const seer_dims& d, const PrefillArgs& a, void* stream) {
  PrefillParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.seq_lens = a.seq_lens;
  p.Lpad = static_cast<int>(prefill_padded_len(&d));
  p.vt = static_cast<uint16_t*>(a.workspace);
  p.r = a.gt ? reinterpret_cast<float*>(static_cast<char*>(a.workspace) + prefill_vt_bytes(&d))
             : nullptr;
  p.out = a.out;
  p.lse = a.lse;
  p.gt = a.gt;
  p.sb = d.kv_stride_b;
  p.sh = d.kv_stride_h;
  p.st = static_cast<int>(d.kv_stride_t);
  p.Hq = d.num_q_heads;
  p.Hkv = d.num_kv_heads;
  p.G = d.num_q_heads / d.num_kv_heads;
  p.Lmax = d.max_seq_len;
  p.NBmax = static_cast<int>(nb_max(&d));
  p.n_qtiles = (d.max_seq_len + kRows - 1) / kRows;
  p.scale_log2 = a.scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return d.head_dim == 64 ? launch_d<64>(d, a, p, s) : launch_d<128>(d, a, p, s);
}

}  // namespace seer
