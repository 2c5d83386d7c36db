// AttnGate kernels of the decode step, for gfx950 (MI355X).
//
// [CP Knowl 1, Knowl 2] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): gate query Q_gate = RoPE(W_q reshape(Q_nope,
// [.., g*d])), compressed keys K_gate = RoPE(W_k [P_max, P_min, P_avg](K_nope)),
// block scores Q_gate K_gate^T / sqrt(d_gate).  [PN key design 1] (papernotes
// page "Sparse Attention Adaptation for Long Reasoning"): one W_q per KV head.
// [CP Knowl 5]: the K Compression Cache gets one entry per newly completed
// block, once every b tokens; top-k or threshold then picks the blocks.
//
// Kernels:
//   prep_kernel    one launch for two kinds of independent tasks:
//                  * gate-query tiles: 16 gate rows x 16 sequences of one KV
//                    head as an MFMA GEMM (W_q read once per step, not once
//                    per sequence), the g*d contraction split over 4 waves
//                    with every load issued up front, then RoPE in float64;
//                  * cache-entry tasks: one newly completed block of one
//                    (sequence, KV head) each (pool, W_k GEMV, RoPE, bf16).
//   gate_kernel    one 512-thread workgroup per (sequence, KV head): all its
//                  cache rows requested at once, block logits in float32,
//                  and -- in the fused step -- the selection, from LDS.
//   commit_kernel  raises kcomp_lens once every new entry is written.
#include <cmath>

#include "gate_dev.hpp"
#include "select_dev.hpp"
#include "seer_internal.h"

namespace seer {

namespace {

RopeFreqs make_freqs(int dg, double theta) {
  RopeFreqs f{};
  for (int i = 0; i < dg / 2; ++i) f.w[i] = std::pow(theta, -2.0 * i / dg);
  return f;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  return SEER_OK;
}

// ------------------------------------------------ gate query + cache entries

struct PrepParams {
  // gate-query tiles (n_query_wgs of them, first in the grid)
  const uint16_t* q_nope;
  const uint16_t* w_q;
  float* q_gate;
  int n_query_wgs;
  // cache-entry tasks (the rest of the grid): entry kcomp_lens[b] + z
  const uint16_t* k_nope;
  const uint16_t* w_k;
  const int32_t* kcomp_lens;
  uint16_t* kcomp;
  int max_new;
  const int32_t* seq_lens;
  int64_t sb, sh, st;
  int B, Hq, Hkv, G, BS, Lmax, NBmax;
  RopeFreqs freqs;
};

constexpr int kQueryStepsPerWave = 16;  // k-steps of 32 per wave: g*d <= 2048

// Gate-query tile t: 16 gate rows (rows i0..i0+7 and their RoPE partners
// i0+DG/2..) x 16 sequences of one KV head as MFMA D = W_q . X.  The 4 waves
// split the g*d contraction; each issues all of its loads before its first
// MFMA; the partial tiles are summed in a fixed order, and wave w rotates
// and stores element w of every lane's accumulator.
template <int D, int DG>
__device__ void query_tile(const PrepParams& p, int t, float (*red)[64][4]) {
  const int RT = DG / 16;
  const int BT = (p.B + 15) / 16;
  const int h = t / (RT * BT);
  const int rt = (t / BT) % RT;
  const int b0 = (t % BT) * 16;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 15;
  const int lq = lane >> 4;
  const int half = DG / 2;
  const int i0 = rt * 8;
  const int K = p.G * D;
  const int KST = K / 32;

  const int bq = b0 + ln;
  const bool bvalid = bq < p.B;
  int L = bvalid ? p.seq_lens[bq] : 1;  // issued early; used by the rotation
  // frequency of the row this lane rotates (element w of its tile column), also early
  const double wf = p.freqs.w[i0 + ((4 * lq + w) & 7)];

  const int arow = (ln < 8) ? (i0 + ln) : (half + i0 + ln - 8);
  const uint16_t* wrow = p.w_q + (static_cast<int64_t>(h) * DG + arow) * K + 8 * lq;
  const uint16_t* xrow = p.q_nope + (static_cast<int64_t>(bvalid ? bq : 0) * p.Hq + h * p.G) * D + 8 * lq;
  const int s0 = w * KST / 4;
  const int s1 = (w + 1) * KST / 4;
  uint4 a[kQueryStepsPerWave], x[kQueryStepsPerWave];
#pragma unroll
  for (int i = 0; i < kQueryStepsPerWave; ++i) {
    const int s = s0 + i;
    a[i] = (s < s1) ? ld16(wrow + 32 * s) : make_uint4(0u, 0u, 0u, 0u);
    x[i] = (s < s1 && bvalid) ? ld16(xrow + 32 * s) : make_uint4(0u, 0u, 0u, 0u);
  }
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kQueryStepsPerWave; ++i)
    if (s0 + i < s1) acc = mfma16x16x32(a[i], x[i], acc);
#pragma unroll
  for (int r = 0; r < 4; ++r) red[w][lane][r] = acc[r];
  __syncthreads();
  // wave w finishes element r = w of every lane: Y[tile row 4*lq + w][sequence b0 + ln]
  const int r = w;
  const float mine = ((red[0][lane][r] + red[1][lane][r]) + red[2][lane][r]) + red[3][lane][r];
  L = min(max(L, 0), p.Lmax);
  const double pos = static_cast<double>(L - 1);
  const float other = __shfl_xor(mine, 32);  // rows m and m^8 sit in lanes l and l^32
  const int m = 4 * lq + r;
  const int fi = i0 + (m & 7);
  const bool first = m < 8;  // this lane holds x_fi (else x_{fi+DG/2})
  float olo, ohi;
  rope_pair(pos, wf, first ? mine : other, first ? other : mine, &olo, &ohi);
  if (bvalid)
    p.q_gate[(static_cast<int64_t>(bq) * p.Hkv + h) * DG + (first ? fi : half + fi)] =
        first ? olo : ohi;
}

template <int D, int DG>
__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
  __shared__ union {
    float red[4][64][4];
    CompressSmem<D, DG> cm;
  } sm;
  const int t = blockIdx.x;
  if (t < p.n_query_wgs) {
    query_tile<D, DG>(p, t, sm.red);
    return;
  }
  const int c = t - p.n_query_wgs;
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
  const uint16_t* keys = p.k_nope + b * p.sb + h * p.sh + static_cast<int64_t>(j) * p.BS * p.st;
  uint16_t* dst = p.kcomp + (static_cast<int64_t>(pair) * p.NBmax + j) * DG;
  compress_block<D, DG>(sm.cm, keys, p.st, p.BS, p.w_k + static_cast<int64_t>(h) * DG * 3 * D,
                        p.freqs, j, dst);
}

__global__ void commit_kernel(const int32_t* seq_lens, int32_t* kcomp_lens, int B, int BS, int Lmax,
                              int NBmax, int max_new) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  kcomp_lens[b] = committed_count(seq_lens[b], kcomp_lens[b], BS, Lmax, NBmax, max_new);
}

// ------------------------------------------------------------------ gate

constexpr int kGateThreads = 512;
constexpr int kGateRows = 512;  // cache rows per prefetch pass

struct GateParams {
  const float* q_gate;          // [B, H_kv, d_gate]
  const uint16_t* kcomp;
  const int32_t* kcomp_lens;
  const int32_t* seq_lens;
  float* logits_out;            // [B, H_kv, NBmax] or null
  int32_t* block_idx;           // select when non-null
  int32_t* num_selected;
  int pending_new;              // entries appended this step, not yet counted
  int Hkv, BS, Lmax, NBmax;
  int mode, topk, max_sel;
  float log_tau;
  float inv_sqrt_dg;
};

// Part m (0, 1, 2) of the exact three-way bf16 split x = q0 + q1 + q2 (+ a
// remainder below 2^-24 |x|): q0 = bf16(x), q1 = bf16(x - q0), q2 =
// bf16(x - q0 - q1).  Each subtraction is exact in float32 (the operands
// agree in their leading bits).
__device__ __forceinline__ uint32_t bf16_part(float x, int m) {
  const uint16_t h0 = f2bf(x);
  const float r1 = x - __uint_as_float(static_cast<uint32_t>(h0) << 16);
  const uint16_t h1 = f2bf(r1);
  const float r2 = r1 - __uint_as_float(static_cast<uint32_t>(h1) << 16);
  const uint16_t h2 = f2bf(r2);
  return m == 0 ? h0 : (m == 1 ? h1 : h2);
}

// One 512-thread workgroup per (sequence, KV head); wave w scores 64 rows of
// each 512-row pass.  A 16-column MFMA tile covers 16/P cache rows split
// into their P = d_gate/32 parts of 32 dims: column n is (row n/P, part
// n%P), so lane l's B operand is the 16 bytes at 64(l%16) + 16(l/16) of
// 1 KiB of consecutive rows -- every load instruction reads one contiguous
// 1 KiB.  A row m = 4p + c holds part p of the float32 gate query's exact
// three-way bf16 split (component c < 3).  The diagonal lanes (lane group
// l/16 == n%P) then receive the part's three component dot products in
// elements 0..2: bf16 x bf16 products are exact in float32 and the three
// components carry 24 bits of the query, so the logits keep float32
// accuracy.  Each row's P part sums meet in LDS and are added in part
// order.  In the fused step the workgroup then selects on the logits
// without them leaving LDS.
template <int DG>
__global__ __launch_bounds__(kGateThreads) void gate_kernel(GateParams p) {
  constexpr int P = DG / 32;                               // 32-dim parts of a row
  constexpr int RPT = 16 / P;                              // rows per MFMA tile
  constexpr int RPW = kGateRows / (kGateThreads / 64);     // rows per wave and pass (64)
  constexpr int TPW = RPW / RPT;                           // tiles per wave and pass
  static_assert(RPW == 64, "one row per lane in the part sum");

  extern __shared__ uint32_t s_keys[];           // NBmax logits (float bits)
  __shared__ SelectSmem s_sel;
  __shared__ float s_part[kGateRows][4];         // part sums of one pass

  const int pair = blockIdx.x;
  const int b = pair / p.Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;

  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  int nc = p.kcomp_lens[b];
  nc = min(min(max(nc, 0), p.NBmax) + p.pending_new, L / p.BS);  // scored blocks
  if (tid < 256) s_sel.hist[tid] = 0;

  const uint16_t* kc = p.kcomp + static_cast<int64_t>(pair) * p.NBmax * DG + 32 * n + 8 * g;
  float* lo = p.logits_out ? p.logits_out + static_cast<int64_t>(pair) * p.NBmax : nullptr;
  const int passes = max(1, (nc + kGateRows - 1) / kGateRows);
  const bool diag = (g < P) && (g == n % P);
  uint4 qa = make_uint4(0u, 0u, 0u, 0u);
  for (int pass = 0; pass < passes; ++pass) {
    const int row0 = pass * kGateRows + w * RPW;  // first row of this wave
    uint4 kv[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int j = row0 + t * RPT + n / P;  // the row this lane's piece belongs to
      kv[t] = (j < nc) ? ld16(kc + static_cast<int64_t>(row0 + t * RPT) * DG)
                       : make_uint4(0u, 0u, 0u, 0u);
    }
    if (pass == 0) {  // the query parts, while the first rows are in flight
      const int pa = n >> 2;
      const int ca = n & 3;
      if (pa < P && ca < 3) {
        const float* qg = p.q_gate + static_cast<int64_t>(pair) * DG + 32 * pa + 8 * g;
        const float4 x0 = *reinterpret_cast<const float4*>(qg);
        const float4 x1 = *reinterpret_cast<const float4*>(qg + 4);
        qa.x = bf16_part(x0.x, ca) | (bf16_part(x0.y, ca) << 16);
        qa.y = bf16_part(x0.z, ca) | (bf16_part(x0.w, ca) << 16);
        qa.z = bf16_part(x1.x, ca) | (bf16_part(x1.y, ca) << 16);
        qa.w = bf16_part(x1.z, ca) | (bf16_part(x1.w, ca) << 16);
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
      if (j < nc) s_keys[j] = __float_as_uint(z);
      if (lo != nullptr && j < p.NBmax) lo[j] = (j < nc) ? z : -INFINITY;
    }
    wave_lds_order();  // the next pass rewrites this wave's part sums
  }
  if (lo != nullptr)  // rows past the passes walked above
    for (int j = passes * kGateRows + tid; j < p.NBmax; j += kGateThreads) lo[j] = -INFINITY;
  if (p.block_idx == nullptr) return;
  __syncthreads();
  select_blocks_wg<kGateThreads>(s_keys, s_sel, nc, (L + p.BS - 1) / p.BS, p.mode, p.topk,
                                 p.log_tau, p.max_sel,
                                 p.block_idx + static_cast<int64_t>(pair) * p.max_sel,
                                 p.num_selected + pair);
}

template <int D, int DG>
void launch_prep_t(const PrepParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((prep_kernel<D, DG>), dim3(grid), dim3(256), 0, s, p);
}

}  // namespace

float log_threshold(float tau);

int launch_prep(const seer_dims& d, const PrepArgs& a, void* stream) {
  PrepParams p{};
  p.q_nope = a.q_nope;
  p.w_q = a.w_q;
  p.q_gate = a.q_gate;
  p.n_query_wgs = a.q_gate ? d.num_kv_heads * (d.d_gate / 16) * ((d.batch + 15) / 16) : 0;
  p.k_nope = a.k_nope;
  p.w_k = a.w_k;
  p.kcomp_lens = a.kcomp_lens;
  p.kcomp = a.kcomp;
  p.max_new = a.max_new_blocks;
  p.seq_lens = a.seq_lens;
  p.sb = d.kv_stride_b;
  p.sh = d.kv_stride_h;
  p.st = d.kv_stride_t;
  p.B = d.batch;
  p.Hq = d.num_q_heads;
  p.Hkv = d.num_kv_heads;
  p.G = d.num_q_heads / d.num_kv_heads;
  p.BS = d.block_size;
  p.Lmax = d.max_seq_len;
  p.NBmax = static_cast<int>(nb_max(&d));
  p.freqs = make_freqs(d.d_gate, a.theta);
  const int64_t cache_wgs = (a.kcomp != nullptr && a.max_new_blocks > 0)
                                ? static_cast<int64_t>(d.batch) * d.num_kv_heads * a.max_new_blocks
                                : 0;
  const int64_t grid = p.n_query_wgs + cache_wgs;
  if (grid > 0x7fffffff) {
    set_error("gate prep grid too large");
    return SEER_ERR_UNSUPPORTED;
  }
  if (grid == 0) return SEER_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int key = (d.head_dim == 128 ? 2 : 0) | (d.d_gate == 128 ? 1 : 0);
  switch (key) {
    case 0: launch_prep_t<64, 64>(p, static_cast<int>(grid), s); break;
    case 1: launch_prep_t<64, 128>(p, static_cast<int>(grid), s); break;
    case 2: launch_prep_t<128, 64>(p, static_cast<int>(grid), s); break;
    default: launch_prep_t<128, 128>(p, static_cast<int>(grid), s); break;
  }
  return check_launch("gate prep launch");
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
  GateParams p{};
  p.q_gate = a.q_gate;
  p.kcomp = a.kcomp;
  p.kcomp_lens = a.kcomp_lens;
  p.seq_lens = a.seq_lens;
  p.logits_out = a.logits_out;
  p.block_idx = a.block_idx;
  p.num_selected = a.num_selected;
  p.pending_new = a.pending_new;
  p.Hkv = d.num_kv_heads;
  p.BS = d.block_size;
  p.Lmax = d.max_seq_len;
  p.NBmax = static_cast<int>(nb_max(&d));
  p.mode = a.mode;
  p.topk = a.topk;
  p.max_sel = a.max_selected;
  p.log_tau = log_threshold(a.tau);
  p.inv_sqrt_dg = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d.d_gate)));
  const int64_t grid = static_cast<int64_t>(d.batch) * d.num_kv_heads;
  if (grid > 0x7fffffff) {
    set_error("gate grid too large");
    return SEER_ERR_UNSUPPORTED;
  }
  const size_t lds = static_cast<size_t>(p.NBmax) * sizeof(uint32_t);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.d_gate == 128)
    hipLaunchKernelGGL(gate_kernel<128>, dim3(grid), dim3(kGateThreads), lds, s, p);
  else
    hipLaunchKernelGGL(gate_kernel<64>, dim3(grid), dim3(kGateThreads), lds, s, p);
  return check_launch("gate launch");
}

}  // namespace seer
