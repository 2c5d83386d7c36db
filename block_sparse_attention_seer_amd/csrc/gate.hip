// AttnGate block scoring for one decode step, for gfx950 (MI355X).
//
// [CP Knowl 1, Knowl 2] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): the query branch maps the g query heads
// of each GQA group, concatenated to g*d values, through one linear layer
// W_q (d_gate x g*d) to one gate query, re-applies RoPE, and scores it
// against the compressed keys as Q_gate K_gate^T / sqrt(d_gate).
// [PN key design 1] (papernotes page "Sparse Attention Adaptation for Long
// Reasoning"): one W_q per KV head.
//
// Two kernels:
//   qgate_kernel   Q_gate[b, h] = RoPE(W_q[h] . concat(q_nope group), L_b - 1)
//                  as one small GEMM per KV head on MFMA (rows of W_q x batch),
//                  reading W_q once per step; RoPE angles in float64.
//   logits_kernel  z[b, h, j] = Q_gate . kcomp[b, h, j] / sqrt(d_gate), float32
//                  VALU dot products, 16-byte coalesced rows of the cache.
#include <cmath>

#include "seer_device.hpp"
#include "seer_internal.h"

namespace seer {

namespace {

struct QgateParams {
  const uint16_t* q_nope;
  const uint16_t* w_q;
  const int32_t* seq_lens;
  float* q_gate;
  int B, Hq, Hkv, G, D, DG, Lmax;
  double theta;
};

// grid (H_kv, d_gate/16, ceil(B/16)), one wave.  The 16 rows of the MFMA
// M-tile are gate rows i0..i0+7 and their RoPE partners i0+DG/2..i0+DG/2+7,
// so each rotation pairs lane l with lane l^32.
__global__ __launch_bounds__(64) void qgate_kernel(QgateParams p) {
  const int h = blockIdx.x;
  const int i0 = blockIdx.y * 8;
  const int bt = blockIdx.z * 16;
  const int lane = threadIdx.x;
  const int ln = lane & 15;
  const int lq = lane >> 4;
  const int half = p.DG >> 1;
  const int K = p.G * p.D;  // multiple of 64

  const int arow = (ln < 8) ? (i0 + ln) : (half + i0 + ln - 8);
  const uint16_t* wrow = p.w_q + (static_cast<int64_t>(h) * p.DG + arow) * K + 8 * lq;
  const int bq = bt + ln;
  const bool bvalid = bq < p.B;
  const uint16_t* xrow =
      p.q_nope + (static_cast<int64_t>(bvalid ? bq : 0) * p.Hq + h * p.G) * p.D + 8 * lq;

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 32) {
    const uint4 a = ld16(wrow + k0);
    const uint4 x = bvalid ? ld16(xrow + k0) : make_uint4(0u, 0u, 0u, 0u);
    acc = mfma16x16x32(a, x, acc);
  }
  // acc[r] = Y[tile row 4*lq + r][batch bt + ln]
  int L = bvalid ? p.seq_lens[bq] : 1;
  L = min(max(L, 0), p.Lmax);
  const double pos = static_cast<double>(L - 1);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float mine = acc[r];
    const float other = __shfl_xor(mine, 32);
    const int m = 4 * lq + r;          // tile row
    const int fi = i0 + (m & 7);       // frequency index
    const double w = pow(p.theta, -2.0 * static_cast<double>(fi) / static_cast<double>(p.DG));
    double sn, cs;
    sincos(pos * w, &sn, &cs);
    double outv;
    int grow;
    if (m < 8) {  // lower half: x_i cos - x_{i+D/2} sin
      outv = static_cast<double>(mine) * cs - static_cast<double>(other) * sn;
      grow = fi;
    } else {      // upper half: x_{i+D/2} cos + x_i sin
      outv = static_cast<double>(mine) * cs + static_cast<double>(other) * sn;
      grow = half + fi;
    }
    if (bvalid) p.q_gate[(static_cast<int64_t>(bq) * p.Hkv + h) * p.DG + grow] = static_cast<float>(outv);
  }
}

struct LogitParams {
  const float* q_gate;
  const uint16_t* kcomp;
  const int32_t* kcomp_lens;
  const int32_t* seq_lens;
  float* logits;
  int Hkv, BS, Lmax, NBmax;
  float inv_sqrt_dg;
};

constexpr int kLogitRowsPerWg = 256;

// grid (B*H_kv, ceil(NBmax/256)), 256 threads.  LPR = DG/8 lanes read one
// 16-byte piece each of a cache row; a wave covers 64/LPR rows per load.
template <int DG>
__global__ __launch_bounds__(256) void logits_kernel(LogitParams p) {
  constexpr int LPR = DG / 8;
  constexpr int RPI = 64 / LPR;                    // rows per wave load
  constexpr int ITER = kLogitRowsPerWg / 4 / RPI;  // loads per lane
  const int pair = blockIdx.x;
  const int b = pair / p.Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c = lane % LPR;
  const int rsub = lane / LPR;

  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  int nc = p.kcomp_lens[b];
  nc = min(max(nc, 0), p.NBmax);
  nc = min(nc, L / p.BS);

  float qv[8];
  {
    const float4* qp = reinterpret_cast<const float4*>(p.q_gate + static_cast<int64_t>(pair) * DG + 8 * c);
    const float4 a = qp[0], bb = qp[1];
    qv[0] = a.x; qv[1] = a.y; qv[2] = a.z; qv[3] = a.w;
    qv[4] = bb.x; qv[5] = bb.y; qv[6] = bb.z; qv[7] = bb.w;
  }
  const int jbase = blockIdx.y * kLogitRowsPerWg + w * (kLogitRowsPerWg / 4) + rsub;
  const uint16_t* kc = p.kcomp + static_cast<int64_t>(pair) * p.NBmax * DG + 8 * c;

  uint4 kv[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int j = jbase + it * RPI;
    kv[it] = (j < nc) ? ld16(kc + static_cast<int64_t>(j) * DG) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int j = jbase + it * RPI;
    const uint4 u = kv[it];
    float s = bf_lo(u.x) * qv[0];
    s = fmaf(bf_hi(u.x), qv[1], s);
    s = fmaf(bf_lo(u.y), qv[2], s);
    s = fmaf(bf_hi(u.y), qv[3], s);
    s = fmaf(bf_lo(u.z), qv[4], s);
    s = fmaf(bf_hi(u.z), qv[5], s);
    s = fmaf(bf_lo(u.w), qv[6], s);
    s = fmaf(bf_hi(u.w), qv[7], s);
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if (c == 0 && j < p.NBmax)
      p.logits[static_cast<int64_t>(pair) * p.NBmax + j] = (j < nc) ? s * p.inv_sqrt_dg : -INFINITY;
  }
}

}  // namespace

int launch_gate(const seer_dims& d, const GateArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = d.num_q_heads / d.num_kv_heads;
  QgateParams qp{a.q_nope, a.w_q, a.seq_lens, a.q_gate, d.batch, d.num_q_heads, d.num_kv_heads,
                 G, d.head_dim, d.d_gate, d.max_seq_len, a.theta};
  dim3 qgrid(d.num_kv_heads, d.d_gate / 16, (d.batch + 15) / 16);
  hipLaunchKernelGGL(qgate_kernel, qgrid, dim3(64), 0, s, qp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("gate query launch: ") + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  const int nbm = static_cast<int>(nb_max(&d));
  LogitParams lp{a.q_gate, a.kcomp, a.kcomp_lens, a.seq_lens, a.logits, d.num_kv_heads,
                 d.block_size, d.max_seq_len, nbm, static_cast<float>(1.0 / std::sqrt(double(d.d_gate)))};
  dim3 lgrid(d.batch * d.num_kv_heads, (nbm + kLogitRowsPerWg - 1) / kLogitRowsPerWg);
  if (d.d_gate == 128)
    hipLaunchKernelGGL(logits_kernel<128>, lgrid, dim3(256), 0, s, lp);
  else
    hipLaunchKernelGGL(logits_kernel<64>, lgrid, dim3(256), 0, s, lp);
  e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("gate logits launch: ") + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  return SEER_OK;
}

}  // namespace seer
