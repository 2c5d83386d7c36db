// AttnGate kernels of the decode step, for gfx950 (MI355X).
//
// [CP Knowl 1, Knowl 2] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): gate query Q_gate = RoPE(W_q reshape(Q_nope,
// [.., g*d])), compressed keys K_gate = RoPE(W_k [P_max, P_min, P_avg](K_nope)),
// block scores Q_gate K_gate^T / sqrt(d_gate).  [PN key design 1] (papernotes
// page "Sparse Attention Adaptation for Long Reasoning"): one W_q per KV head.
// [CP Knowl 5]: the K Compression Cache gets one entry per newly completed
// block, once every b tokens; top-k or threshold (or top-p, the adaptive
// direction of [CP Knowl 14]) then picks the blocks.
//
// Kernels:
//   prep_kernel    cache-entry tasks of the staged update: one newly
//                  completed block of one (sequence, KV head) each (pool,
//                  W_k GEMV, RoPE, bf16); prep_bulk_kernel does sixteen
//                  consecutive blocks per workgroup for large updates.
//   commit_kernel  raises kcomp_lens once every new entry is written.
//   gate_kernel    one 512-thread workgroup per (sequence, KV head): the
//                  pair's new cache entries (fused step), its gate query
//                  (MFMA GEMV + RoPE), its block logits (MFMA) and -- in the
//                  fused step -- the selection, all without leaving the
//                  workgroup.  Every global load of the scoring is issued
//                  up front, so the W_q, query and cache-row latencies
//                  overlap.
#include <cmath>

#include "gate_dev.hpp"
#include "select_dev.hpp"
#include "seer_internal.h"

namespace seer {

namespace {


int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  return SEER_OK;
}

// ------------------------------------------------------- staged cache update

struct PrepParams {
  // entry kcomp_lens[b] + z of pair (b, h) for workgroup pair * max_new + z
  const uint16_t* k_nope;
  const uint16_t* w_k;
  const int32_t* kcomp_lens;
  uint16_t* kcomp;
  int max_new;
  const int32_t* seq_lens;
  int64_t sb, sh, st;
  int Hkv, BS, Lmax, NBmax;
  double log2_theta;  // RoPE base, as log2
};

template <int D, int DG>
__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
  __shared__ CompressSmem<D, DG> cm;
  const int c = blockIdx.x;
  const int pair = c / p.max_new;
  const int z = c - pair * p.max_new;
  const int b = pair / p.Hkv;
  const int h = pair - b * p.Hkv;
  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  int cl = p.kcomp_lens[b];
  cl = min(max(cl, 0), p.NBmax);
  const int j = cl + z;
  if (j >= L / p.BS) return;  // uniform over the workgroup
  const double wf = rope_freq(threadIdx.x % (DG / 2), DG, p.log2_theta);
  const uint16_t* keys = p.k_nope + b * p.sb + h * p.sh + static_cast<int64_t>(j) * p.BS * p.st;
  uint16_t* dst = p.kcomp + (static_cast<int64_t>(pair) * p.NBmax + j) * DG;
  compress_block<D, DG>(cm, keys, p.st, p.BS, p.w_k + static_cast<int64_t>(h) * DG * 3 * D, wf, j,
                        dst);
}

// Bulk variant (a prompt's cache, or any update of many blocks): one
// workgroup per kBulkBlocks consecutive new entries of one pair, one MFMA
// column each, so W_k is read once for all of them.  The entries are
// bit-identical to the one-block kernel's.
constexpr int kBulkBlocks = 16;

template <int D, int DG>
__global__ __launch_bounds__(256, 4) void prep_bulk_kernel(PrepParams p) {
  __shared__ CompressSmem<D, DG, kBulkBlocks> cm;
  const int per_pair = (p.max_new + kBulkBlocks - 1) / kBulkBlocks;
  const int pair = blockIdx.x / per_pair;
  const int z0 = (blockIdx.x - pair * per_pair) * kBulkBlocks;
  const int b = pair / p.Hkv;
  const int h = pair - b * p.Hkv;
  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  int cl = p.kcomp_lens[b];
  cl = min(max(cl, 0), p.NBmax);
  const int j0 = cl + z0;
  const int nblk = min(kBulkBlocks, min(L / p.BS, cl + p.max_new) - j0);
  if (nblk <= 0) return;  // uniform over the workgroup
  const double wf = rope_freq(threadIdx.x % (DG / 2), DG, p.log2_theta);
  const uint16_t* keys = p.k_nope + b * p.sb + h * p.sh + static_cast<int64_t>(j0) * p.BS * p.st;
  uint16_t* dst = p.kcomp + (static_cast<int64_t>(pair) * p.NBmax + j0) * DG;
  compress_blocks<D, DG, kBulkBlocks>(cm, keys, p.st, p.BS,
                                      p.w_k + static_cast<int64_t>(h) * DG * 3 * D, wf, j0, nblk,
                                      dst);
}

__global__ void commit_kernel(const int32_t* seq_lens, int32_t* kcomp_lens, int B, int BS, int Lmax,
                              int NBmax, int max_new) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  kcomp_lens[b] = committed_count(seq_lens[b], kcomp_lens[b], BS, Lmax, NBmax, max_new);
}

template <int D, int DG>
void launch_prep_t(const PrepParams& p, int grid, bool bulk, hipStream_t s) {
  if (bulk)
    hipLaunchKernelGGL((prep_bulk_kernel<D, DG>), dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((prep_kernel<D, DG>), dim3(grid), dim3(256), 0, s, p);
}

// ------------------------------------------------------------------ gate

constexpr int kGateThreads = 512;
constexpr int kGateRows = 512;   // cache rows per prefetch pass
constexpr int kQueryChunks = 5;  // 128-dim chunks of g*d per W_q load group

struct GateParams {
  const uint16_t* q_nope;  // [B, H_q, d]
  const uint16_t* w_q;     // [H_kv, d_gate, g*d]
  float* q_gate_out;       // [B, H_kv, d_gate] or null
  // new cache entries of this launch (fused step): entries c .. c+nnew-1
  // with nnew = min(floor(L/b), c + max_new) - c, c = kcomp_lens[b]
  const uint16_t* k_nope;
  const uint16_t* w_k;
  int64_t sb, sh, st;
  int max_new;
  uint16_t* kcomp;
  const int32_t* kcomp_lens;
  const int32_t* seq_lens;
  float* logits_out;   // [B, H_kv, NBmax] or null
  int32_t* block_idx;  // select when non-null (one row part only)
  int32_t* num_selected;
  int32_t* clear_ctr;  // [B * H_kv] split counters of the decode launch after this one, set
                       // to zero here (fused step), or null
  int pairs;           // B * H_kv; workgroup = part * pairs + pair
  int rows_per_part;   // logit rows of one workgroup (a multiple of 64)
  int Hq, Hkv, G, BS, Lmax, NBmax;
  int mode, topk, max_sel;
  float log_tau;
  uint32_t mass_target;  // top-p: ceil(p * 2^30)
  float inv_sqrt_dg;
  double log2_theta;  // RoPE base, as log2
};

// Chunk group c0 .. c0+kQueryChunks-1 (128 dims each) of this lane's W_q
// pieces (B operand, tiles of 4 rows) and query pieces (A operand).
template <int TQ>
__device__ __forceinline__ void load_query_group(uint4 (&wb)[TQ][kQueryChunks],
                                                 uint4 (&xa)[kQueryChunks], const uint16_t* wq,
                                                 const uint16_t* xq, int c0, int nch, int K,
                                                 int n, int g, int w) {
  const bool xlane = (n & 3) == 0;  // A row 4p holds part p = n/4 of the query heads
#pragma unroll
  for (int c = 0; c < kQueryChunks; ++c) {
    const int k0 = (c0 + c) * 128;
    const bool in = (c0 + c < nch) && (k0 + 32 * (n & 3) + 8 * g < K);
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
      const int row = (w * TQ + t) * 4 + (n >> 2);
      wb[t][c] = in ? ld16(wq + static_cast<int64_t>(row) * K + k0) : make_uint4(0u, 0u, 0u, 0u);
    }
    xa[c] = (xlane && c0 + c < nch && k0 + 32 * (n >> 2) + 8 * g < K)
                ? ld16(xq + k0)
                : make_uint4(0u, 0u, 0u, 0u);
  }
}

// This lane's pieces of the cache rows of one pass that are already cached
// and in this workgroup's rows (j < lim); the rest are zero.
template <int TPW, int RPT, int P, int DG>
__device__ __forceinline__ void load_rows(uint4 (&kv)[TPW], const uint16_t* kc, int row0, int lim,
                                          int n) {
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int j = row0 + t * RPT + n / P;
    kv[t] = (j < lim) ? ld16(kc + static_cast<int64_t>(row0 + t * RPT) * DG)
                      : make_uint4(0u, 0u, 0u, 0u);
  }
}

// One 512-thread workgroup per (sequence, KV head) and part of its cache
// rows: with more than one part, each workgroup of a pair computes the gate
// query (so no workgroup waits for another) and the logits of its own rows
// [part * rows_per_part, +rows_per_part); the selection then runs in the
// decode launch.  A logit's arithmetic does not depend on the part count.
//
// Both contractions use the same MFMA layout.  A 16-column tile covers
// 16/P rows of a matrix, each split into P parts of 32 dims: column n is
// (row n/P, part n%P), so lane l's B operand is the 16 bytes at
// 64(l%16) + 16(l/16) of the tile's rows -- every load instruction reads
// whole 256-byte runs.  A row m = 4p + c holds part p of the vector
// (component c).  The diagonal lanes (lane group l/16 == n%P) receive each
// part's dot products; a row's P part sums meet in LDS and are added in part
// order.
//   gate query: rows = W_q[h] rows, taken 128 dims (P = 4) at a time with
//     the chunks' products accumulated in the MFMA; the vector is the bf16
//     concatenation of the group's q_nope heads (component 0 only, exact);
//   logits: rows = the pair's cache rows (P = d_gate/32); the vector is the
//     float32 gate query split exactly into three bf16 components, so the
//     logits keep float32 accuracy (bf16 x bf16 products are exact).
template <int D, int DG>
__global__ __launch_bounds__(kGateThreads) void gate_kernel(GateParams p) {
  constexpr int P = DG / 32;                            // 32-dim parts of a cache row
  constexpr int RPT = 16 / P;                           // cache rows per MFMA tile
  constexpr int RPW = kGateRows / (kGateThreads / 64);  // cache rows per wave and pass (64)
  constexpr int TPW = RPW / RPT;                        // logit tiles per wave and pass
  constexpr int TQ = DG / 32;                           // W_q tiles (4 rows each) per wave
  static_assert(RPW == 64, "one row per lane in the part sum");

  extern __shared__ uint32_t s_keys[];           // NBmax logits (float bits)
  __shared__ SelectSmem s_sel;
  __shared__ float s_part[kGateRows][4];         // part sums (gate query, then logits)
  __shared__ float s_qg[DG];                     // the gate query
  __shared__ __align__(16) uint16_t s_new[kMaxInlineNew][DG];  // this launch's new entries (read as 16-byte words)
  __shared__ CompressSmem<D, DG, kMaxInlineNew> s_cm;

  const int part = blockIdx.x / p.pairs;
  const int pair = blockIdx.x - part * p.pairs;
  const int r0 = part * p.rows_per_part;          // this workgroup's logit rows
  const int r1 = min(p.NBmax, r0 + p.rows_per_part);
  const int b = pair / p.Hkv;
  const int h = pair - b * p.Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;

  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  int nc0 = p.kcomp_lens[b];
  nc0 = min(min(max(nc0, 0), p.NBmax), L / p.BS);  // cached blocks
  const int nc = min(L / p.BS, nc0 + p.max_new);   // scored: with this launch's entries
  if (p.clear_ctr != nullptr && part == 0 && tid == 0) p.clear_ctr[pair] = 0;
  // this launch's new entries that fall in this workgroup's rows
  const int e0 = max(nc0, r0);
  const int nnew = max(0, min(nc, r1) - e0);
  select_smem_init(s_sel);
  const double wf = rope_freq(tid % (DG / 2), DG, p.log2_theta);

  // ---- new cache entries (blocks completed since the last update), in one
  // pass before anything else is in flight (they are rare: one step in b)
  if (nnew > 0) {
    const uint16_t* keys = p.k_nope + b * p.sb + h * p.sh + static_cast<int64_t>(e0) * p.BS * p.st;
    compress_blocks<D, DG, kMaxInlineNew>(s_cm, keys, p.st, p.BS,
                                          p.w_k + static_cast<int64_t>(h) * DG * 3 * D, wf, e0,
                                          nnew, p.kcomp + (static_cast<int64_t>(pair) * p.NBmax + e0) * DG,
                                          &s_new[0][0]);
  }

  // ---- then all loads: W_q rows and the query heads (first chunk group),
  // then the first pass of cache rows
  const int K = p.G * D;  // W_q row length
  const int nch = (K + 127) / 128;
  const uint16_t* wq = p.w_q + static_cast<int64_t>(h) * DG * K + 32 * (n & 3) + 8 * g;
  const uint16_t* xq =
      p.q_nope + (static_cast<int64_t>(b) * p.Hq + h * p.G) * D + 32 * (n >> 2) + 8 * g;
  uint4 wb[TQ][kQueryChunks], xa[kQueryChunks];
  // The 16 workgroups of a KV head share its W_q rows and run on one XCD
  // (workgroups go round-robin over the 8 XCDs); each sequence starts its
  // waves at a different row group so that they do not all request the
  // same L2 lines at once.  Each row's arithmetic is unchanged.
  const int wr = (w + b) & (kGateThreads / 64 - 1);
  load_query_group<TQ>(wb, xa, wq, xq, 0, nch, K, n, g, wr);

  const uint16_t* kc = p.kcomp + static_cast<int64_t>(pair) * p.NBmax * DG + 32 * n + 8 * g;
  const int rows_scored = max(0, min(nc, r1) - r0);  // rows r0 .. of this workgroup
  const int passes = (rows_scored + kGateRows - 1) / kGateRows;
  const int lim = min(nc0, r1);  // rows read from the cache (the rest: this launch's entries)
  uint4 kv[TPW];
  if (passes > 0) load_rows<TPW, RPT, P, DG>(kv, kc, r0 + w * RPW, lim, n);

  // ---- gate query: y = W_q[h] x, then RoPE at position L-1
  {
    f32x4_t acc[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nch; c0 += kQueryChunks) {
      if (c0 > 0) load_query_group<TQ>(wb, xa, wq, xq, c0, nch, K, n, g, wr);
#pragma unroll
      for (int c = 0; c < kQueryChunks; ++c)
#pragma unroll
        for (int t = 0; t < TQ; ++t) acc[t] = mfma16x16x32(xa[c], wb[t][c], acc[t]);
    }
    if (g == (n & 3)) {
#pragma unroll
      for (int t = 0; t < TQ; ++t) s_part[(wr * TQ + t) * 4 + (n >> 2)][g] = acc[t][0];
    }
  }
  __syncthreads();
  if (tid < DG / 2) {
    const float* lo_row = s_part[tid];
    const float* hi_row = s_part[tid + DG / 2];
    const float ylo = ((lo_row[0] + lo_row[1]) + lo_row[2]) + lo_row[3];
    const float yhi = ((hi_row[0] + hi_row[1]) + hi_row[2]) + hi_row[3];
    float olo, ohi;
    rope_pair(static_cast<double>(L - 1), wf, ylo, yhi, &olo, &ohi);
    s_qg[tid] = olo;
    s_qg[tid + DG / 2] = ohi;
    if (p.q_gate_out != nullptr && part == 0) {
      p.q_gate_out[static_cast<int64_t>(pair) * DG + tid] = olo;
      p.q_gate_out[static_cast<int64_t>(pair) * DG + tid + DG / 2] = ohi;
    }
  }
  __syncthreads();

  // ---- logits
  uint4 qa = make_uint4(0u, 0u, 0u, 0u);
  {
    const int pa = n >> 2;
    const int ca = n & 3;
    if (pa < P && ca < 3) {
      const float* x = s_qg + 32 * pa + 8 * g;
      qa.x = bf16_part(x[0], ca) | (bf16_part(x[1], ca) << 16);
      qa.y = bf16_part(x[2], ca) | (bf16_part(x[3], ca) << 16);
      qa.z = bf16_part(x[4], ca) | (bf16_part(x[5], ca) << 16);
      qa.w = bf16_part(x[6], ca) | (bf16_part(x[7], ca) << 16);
    }
  }
  const bool diag = (g < P) && (g == n % P);
  float* lo = p.logits_out ? p.logits_out + static_cast<int64_t>(pair) * p.NBmax : nullptr;
  for (int pass = 0; pass < passes; ++pass) {
    const int row0 = r0 + pass * kGateRows + w * RPW;  // first row of this wave
    if (pass > 0) load_rows<TPW, RPT, P, DG>(kv, kc, row0, lim, n);
    if (nnew > 0) {  // this launch's entries, from LDS
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int j = row0 + t * RPT + n / P;
        if (j >= e0 && j < e0 + nnew)
          kv[t] = *reinterpret_cast<const uint4*>(&s_new[j - e0][32 * (n % P) + 8 * g]);
      }
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const f32x4_t acc = mfma16x16x32(qa, kv[t], f32x4_t{0.f, 0.f, 0.f, 0.f});
      if (diag) s_part[w * RPW + t * RPT + n / P][g] = (acc[0] + acc[1]) + acc[2];
    }
    wave_lds_order();
    {  // lane l: row row0 + l
      const int j = row0 + lane;
      const float* pp = s_part[w * RPW + lane];
      float z = pp[0];
#pragma unroll
      for (int q = 1; q < P; ++q) z += pp[q];
      z *= p.inv_sqrt_dg;
      if (j < min(nc, r1)) s_keys[j] = __float_as_uint(z);
      if (lo != nullptr && j < r1) lo[j] = (j < nc) ? z : -INFINITY;
    }
    wave_lds_order();  // the next pass rewrites this wave's part sums
  }
  if (lo != nullptr)  // this workgroup's rows past the passes walked above
    for (int j = r0 + passes * kGateRows + tid; j < r1; j += kGateThreads) lo[j] = -INFINITY;
  if (p.block_idx == nullptr) return;
  __syncthreads();
  select_blocks_wg<kGateThreads>(s_keys, s_sel, nc, (L + p.BS - 1) / p.BS, p.mode, p.topk,
                                 p.log_tau, p.mass_target, p.max_sel,
                                 p.block_idx + static_cast<int64_t>(pair) * p.max_sel,
                                 p.num_selected + pair);
}

template <int D, int DG>
void launch_gate_t(const GateParams& p, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((gate_kernel<D, DG>), dim3(grid), dim3(kGateThreads), lds, s, p);
}

}  // namespace


int launch_prep(const seer_dims& d, const PrepArgs& a, void* stream) {
  PrepParams p{};
  p.k_nope = a.k_nope;
  p.w_k = a.w_k;
  p.kcomp_lens = a.kcomp_lens;
  p.kcomp = a.kcomp;
  p.max_new = a.max_new_blocks;
  p.seq_lens = a.seq_lens;
  p.sb = d.kv_stride_b;
  p.sh = d.kv_stride_h;
  p.st = d.kv_stride_t;
  p.Hkv = d.num_kv_heads;
  p.BS = d.block_size;
  p.Lmax = d.max_seq_len;
  p.NBmax = static_cast<int>(nb_max(&d));
  p.log2_theta = std::log2(a.theta);
  const bool bulk = a.max_new_blocks >= kBulkBlocks;
  const int64_t per_pair = bulk ? (a.max_new_blocks + kBulkBlocks - 1) / kBulkBlocks
                                : a.max_new_blocks;
  const int64_t grid = static_cast<int64_t>(d.batch) * d.num_kv_heads * per_pair;
  if (grid > 0x7fffffff) {
    set_error("cache update grid too large");
    return SEER_ERR_UNSUPPORTED;
  }
  if (grid <= 0) return SEER_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int key = (d.head_dim == 128 ? 2 : 0) | (d.d_gate == 128 ? 1 : 0);
  switch (key) {
    case 0: launch_prep_t<64, 64>(p, static_cast<int>(grid), bulk, s); break;
    case 1: launch_prep_t<64, 128>(p, static_cast<int>(grid), bulk, s); break;
    case 2: launch_prep_t<128, 64>(p, static_cast<int>(grid), bulk, s); break;
    default: launch_prep_t<128, 128>(p, static_cast<int>(grid), bulk, s); break;
  }
  return check_launch("cache update launch");
}

int launch_commit(const seer_dims& d, const int32_t* seq_lens, int32_t* kcomp_lens, int max_new,
                  void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(commit_kernel, dim3((d.batch + 255) / 256), dim3(256), 0, s, seq_lens,
                     kcomp_lens, d.batch, d.block_size, d.max_seq_len,
                     static_cast<int>(nb_max(&d)), max_new);
  return check_launch("kcomp commit launch");
}

int launch_gate(const seer_dims& d, const GateArgs& a, void* stream) {
  if (a.max_new < 0 || a.max_new > kMaxInlineNew) {
    set_error("gate launch: too many new cache entries for one launch");
    return SEER_ERR_INVALID_ARG;
  }
  GateParams p{};
  p.q_nope = a.q_nope;
  p.w_q = a.w_q;
  p.q_gate_out = a.q_gate;
  p.k_nope = a.k_nope;
  p.w_k = a.w_k;
  p.sb = d.kv_stride_b;
  p.sh = d.kv_stride_h;
  p.st = d.kv_stride_t;
  p.max_new = a.max_new;
  p.kcomp = a.kcomp;
  p.kcomp_lens = a.kcomp_lens;
  p.seq_lens = a.seq_lens;
  p.logits_out = a.logits_out;
  p.block_idx = a.block_idx;
  p.num_selected = a.num_selected;
  p.clear_ctr = a.clear_counters;
  const int64_t pairs = static_cast<int64_t>(d.batch) * d.num_kv_heads;
  p.pairs = static_cast<int>(pairs);
  p.Hq = d.num_q_heads;
  p.Hkv = d.num_kv_heads;
  p.G = d.num_q_heads / d.num_kv_heads;
  p.BS = d.block_size;
  p.Lmax = d.max_seq_len;
  p.NBmax = static_cast<int>(nb_max(&d));
  p.mode = a.mode;
  p.topk = a.topk;
  p.max_sel = a.max_selected;
  p.log_tau = log_threshold(a.tau);
  p.mass_target = topp_mass_target(a.tau);
  p.inv_sqrt_dg = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d.d_gate)));
  p.log2_theta = std::log2(a.theta);
  // row parts: every one non-empty (rows_per_part a multiple of 64); the
  // selection needs the whole row in one workgroup
  const int nbm = p.NBmax;
  int parts = (a.block_idx != nullptr) ? 1 : std::max(1, std::min(a.row_parts, (nbm + 63) / 64));
  int rpp = ((nbm + parts - 1) / parts + 63) / 64 * 64;
  parts = (nbm + rpp - 1) / rpp;
  p.rows_per_part = rpp;
  const int64_t grid = pairs * parts;
  if (grid > 0x7fffffff) {
    set_error("gate grid too large");
    return SEER_ERR_UNSUPPORTED;
  }
  const size_t lds = static_cast<size_t>(p.NBmax) * sizeof(uint32_t);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int key = (d.head_dim == 128 ? 2 : 0) | (d.d_gate == 128 ? 1 : 0);
  switch (key) {
    case 0: launch_gate_t<64, 64>(p, static_cast<int>(grid), lds, s); break;
    case 1: launch_gate_t<64, 128>(p, static_cast<int>(grid), lds, s); break;
    case 2: launch_gate_t<128, 64>(p, static_cast<int>(grid), lds, s); break;
    default: launch_gate_t<128, 128>(p, static_cast<int>(grid), lds, s); break;
  }
  return check_launch("gate launch");
}

}  // namespace seer
