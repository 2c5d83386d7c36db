// Device pieces of the AttnGate shared by the gate kernels and the fused
// decode step, for gfx950 (MI355X).
//
// [CP Knowl 1, Knowl 2] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"):
//   K branch: max / min / average pooling of each non-overlapping b-token
//   block of pre-RoPE keys, concatenated (3d values), mapped by W_k
//   (d_gate x 3d), then RoPE at the block's first-token position.
//   Q branch: the g query heads of a GQA group concatenated (g*d values),
//   mapped by W_q (d_gate x g*d), then RoPE at the query position.
// [CP Knowl 5]: the K Compression Cache stores K_gate, one entry per
// complete block.
#pragma once

#include "seer_device.hpp"

namespace seer {

// RoPE frequencies theta^(-2i/d_gate), i < d_gate/2, formed on the host in
// float64 and passed by value.
struct RopeFreqs {
  double w[64];
};

// Rotate-half RoPE of the pair (lo, hi) = (x_i, x_{i+D/2}) at angle pos*w.
// The angle (up to ~1e5 rad) is formed and reduced to [-pi, pi] in float64
// with a two-part 2*pi (Cody-Waite: each fma forms its product exactly and
// rounds once), so the reduced angle r is good to ~1e-15 rad.  r is then
// split into float parts rh + rl; sin and cos are taken of the small float
// argument rh and corrected to first order in rl (|rl| <= 2^-24 pi, so the
// neglected term is below 1e-14), and the rotation is formed with fused
// multiply-adds in float32.
__device__ __forceinline__ void rope_pair(double pos, double w, float lo, float hi, float* out_lo,
                                          float* out_hi) {
  constexpr double kTwoPiHi = 6.283185307179586;             // 2*pi rounded to double
  constexpr double kTwoPiLo = 2.4492935982947064e-16;         // 2*pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189535;
  const double a = pos * w;
  const double k = rint(a * kInvTwoPi);
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, a));
  const float rh = static_cast<float>(r);
  const float rl = static_cast<float>(r - static_cast<double>(rh));
  float s0, c0;
  sincosf(rh, &s0, &c0);
  const float sn = fmaf(c0, rl, s0);
  const float cs = fmaf(-s0, rl, c0);
  *out_lo = fmaf(lo, cs, -(hi * sn));
  *out_hi = fmaf(hi, cs, lo * sn);
}

// Shared-memory scratch of the cache-entry computation of up to NB blocks.
template <int D, int DG, int NB = 1>
struct CompressSmem {
  static constexpr int CP = D / 2;      // channel pairs
  static constexpr int NTG = 256 / CP;  // token groups
  float red[3][NTG][D];
  float u[NB][3 * D];
  float v[NB][DG];
};

// K Compression Cache entries of blocks j0 .. j0+nblk-1 (nblk <= NB,
// consecutive blocks of one pair; keys points at row 0 of block j0, dst at
// entry j0) computed by the first 256 threads of the workgroup; every thread
// of the workgroup must call this (it contains barriers).  Each block's
// arithmetic is the same for every NB and nblk, so an entry has the same bits
// whichever way the cache is built.
//   pooling, block by block: each (channel pair, token group) thread reduces
//   a strided set of tokens, then threads < D fold the groups in a fixed
//   order;
//   GEMV: wave w of the 256 handles rows w, w+4, ... (loaded 8 rows at a
//   time, each row applied to every block); lanes split the 3d columns and
//   reduce across the wave;
//   RoPE at position j*b (float64 angle), bf16 store (round to nearest even)
//   to dst and, when lds_copy is not null, to LDS ([NB][DG]) as well.
//   wf is this thread's RoPE frequency, theta^(-2(t mod DG/2)/DG) for thread t.
template <int D, int DG, int NB>
__device__ void compress_blocks(CompressSmem<D, DG, NB>& sm, const uint16_t* keys, int64_t st,
                                int BS, const uint16_t* w_k_h, double wf, int j0, int nblk,
                                uint16_t* dst, uint16_t* lds_copy = nullptr) {
  constexpr int CP = CompressSmem<D, DG, NB>::CP;
  constexpr int NTG = CompressSmem<D, DG, NB>::NTG;
  const int tid = threadIdx.x;
  for (int n = 0; n < nblk; ++n) {
    if (tid < 256) {
      const int cp = tid % CP;
      const int tg = tid / CP;
      const uint16_t* base = keys + static_cast<int64_t>(n) * BS * st + 2 * cp;
      float mx0 = -INFINITY, mx1 = -INFINITY, mn0 = INFINITY, mn1 = INFINITY, s0 = 0.f, s1 = 0.f;
      for (int t = tg; t < BS; t += NTG) {
        const uint32_t wv = *reinterpret_cast<const uint32_t*>(base + t * st);
        const float a = bf_lo(wv), bb = bf_hi(wv);
        mx0 = fmaxf(mx0, a); mn0 = fminf(mn0, a); s0 += a;
        mx1 = fmaxf(mx1, bb); mn1 = fminf(mn1, bb); s1 += bb;
      }
      sm.red[0][tg][2 * cp] = mx0; sm.red[0][tg][2 * cp + 1] = mx1;
      sm.red[1][tg][2 * cp] = mn0; sm.red[1][tg][2 * cp + 1] = mn1;
      sm.red[2][tg][2 * cp] = s0;  sm.red[2][tg][2 * cp + 1] = s1;
    }
    __syncthreads();
    if (tid < D) {
      float mx = -INFINITY, mn = INFINITY, sum = 0.f;
#pragma unroll
      for (int g = 0; g < NTG; ++g) {
        mx = fmaxf(mx, sm.red[0][g][tid]);
        mn = fminf(mn, sm.red[1][g][tid]);
        sum += sm.red[2][g][tid];
      }
      sm.u[n][tid] = mx;
      sm.u[n][D + tid] = mn;
      sm.u[n][2 * D + tid] = sum / static_cast<float>(BS);
    }
    __syncthreads();
  }
  if (tid < 256) {
    // rows in groups of kRowsPerGroup, every W_k load of a group in flight
    // before its first use (the per-row arithmetic and order are those of a
    // plain row loop)
    constexpr int kRowsPerGroup = 8;
    constexpr int NQ = (3 * D / 2 + 63) / 64;  // 32-bit words per lane and row
    const int w = tid >> 6;
    const int lane = tid & 63;
    for (int r0 = w; r0 < DG; r0 += 4 * kRowsPerGroup) {
      uint32_t wv[kRowsPerGroup][NQ];
#pragma unroll
      for (int i = 0; i < kRowsPerGroup; ++i) {
        const int r = r0 + 4 * i;
        const uint32_t* row = reinterpret_cast<const uint32_t*>(w_k_h + static_cast<int64_t>(r) * 3 * D);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int q2 = lane + 64 * q;
          wv[i][q] = (r < DG && q2 < 3 * D / 2) ? row[q2] : 0u;
        }
      }
#pragma unroll
      for (int i = 0; i < kRowsPerGroup; ++i) {
        const int r = r0 + 4 * i;
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          if (n < nblk) {
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              const int q2 = lane + 64 * q;
              if (q2 < 3 * D / 2) {
                acc = fmaf(bf_lo(wv[i][q]), sm.u[n][2 * q2], acc);
                acc = fmaf(bf_hi(wv[i][q]), sm.u[n][2 * q2 + 1], acc);
              }
            }
            acc = wave_sum(acc);
            if (lane == 0 && r < DG) sm.v[n][r] = acc;
          }
        }
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nblk * (DG / 2); idx += blockDim.x) {
    const int n = idx / (DG / 2);
    const int i = idx - n * (DG / 2);  // = tid mod DG/2: wf is this row's frequency
    float olo, ohi;
    rope_pair(static_cast<double>(j0 + n) * BS, wf, sm.v[n][i], sm.v[n][i + DG / 2], &olo, &ohi);
    const uint16_t lo = f2bf(olo), hi = f2bf(ohi);
    dst[n * DG + i] = lo;
    dst[n * DG + i + DG / 2] = hi;
    if (lds_copy != nullptr) {
      lds_copy[n * DG + i] = lo;
      lds_copy[n * DG + i + DG / 2] = hi;
    }
  }
}

// One block's entry (compress_blocks with a single block).
template <int D, int DG>
__device__ void compress_block(CompressSmem<D, DG, 1>& sm, const uint16_t* keys, int64_t st,
                               int BS, const uint16_t* w_k_h, double wf, int j, uint16_t* dst,
                               uint16_t* lds_copy = nullptr) {
  compress_blocks<D, DG, 1>(sm, keys, st, BS, w_k_h, wf, j, 1, dst, lds_copy);
}

}  // namespace seer
