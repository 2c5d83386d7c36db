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

// RoPE frequency theta^(-2i/D) of pair i, formed in float64 from log2(theta)
// (the exponent 2i/D is exact for the power-of-two D here).  Computed where
// it is used rather than passed as a table: a table in the kernel arguments
// is loaded by every wave into scalar registers.
__device__ __forceinline__ double rope_freq(int i, int D, double log2_theta) {
  return exp2((-2.0 * static_cast<double>(i) / static_cast<double>(D)) * log2_theta);
}

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
  static_assert(NB >= 1 && NB <= 16, "one MFMA column per block");
  static constexpr int CP = D / 2;      // channel pairs
  static constexpr int NTG = 256 / CP;  // token groups
  float red[2][3][NTG][D];              // pooling partials of two blocks
  float u[NB][3 * D + 4];               // pooled features (rows padded: no bank conflicts)
  float v[NB][DG];                      // W_k u
};

// K Compression Cache entries of blocks j0 .. j0+nblk-1 (nblk <= NB,
// consecutive blocks of one pair; keys points at row 0 of block j0, dst at
// entry j0) computed by the first 256 threads of the workgroup; every thread
// of the workgroup must call this (it contains barriers).  A block's
// arithmetic does not depend on NB or nblk (MFMA columns are independent),
// so an entry has the same bits whichever way the cache is built.
//   pooling, two blocks at a time: each (channel pair, token group) thread
//   loads its strided tokens of both blocks, then reduces them in token
//   order; threads < D fold the groups in a fixed order;
//   GEMV on MFMA: V[row][block] = W_k[row][:] . u[block][:], the blocks as
//   the 16 B-operand columns; max and min features are exact in bf16, the
//   mean enters as three bf16 components against the same W_k columns;
//   RoPE at position j*b (float64 angle), bf16 store (round to nearest even)
//   to dst and, when lds_copy is not null, to LDS ([NB][DG]) as well.
//   wf is this thread's RoPE frequency, theta^(-2(t mod DG/2)/DG) for thread t.
template <int D, int DG, int NB>
__device__ __forceinline__ void compress_blocks(CompressSmem<D, DG, NB>& sm, const uint16_t* keys,
                                                int64_t st, int BS, const uint16_t* w_k_h,
                                                double wf, int j0, int nblk, uint16_t* dst,
                                                uint16_t* lds_copy = nullptr) {
  constexpr int CP = CompressSmem<D, DG, NB>::CP;
  constexpr int NTG = CompressSmem<D, DG, NB>::NTG;
  constexpr int TMAX = 128 / NTG;  // tokens per thread at b <= 128
  const int tid = threadIdx.x;
  for (int n0 = 0; n0 < nblk; n0 += 2) {
    if (tid < 256) {
      const int cp = tid % CP;
      const int tg = tid / CP;
      const int cnt = (BS - tg + NTG - 1) / NTG;  // this thread's tokens of a block
      uint32_t wv[2][TMAX];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        const uint16_t* base = keys + static_cast<int64_t>(n0 + pb) * BS * st + 2 * cp;
#pragma unroll
        for (int i = 0; i < TMAX; ++i)
          wv[pb][i] = (n0 + pb < nblk && i < cnt)
                          ? *reinterpret_cast<const uint32_t*>(base + (tg + NTG * i) * st)
                          : 0u;
      }
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        float mx0 = -INFINITY, mx1 = -INFINITY, mn0 = INFINITY, mn1 = INFINITY, s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < TMAX; ++i) {
          if (i < cnt) {
            const float a = bf_lo(wv[pb][i]), bb = bf_hi(wv[pb][i]);
            mx0 = fmaxf(mx0, a); mn0 = fminf(mn0, a); s0 += a;
            mx1 = fmaxf(mx1, bb); mn1 = fminf(mn1, bb); s1 += bb;
          }
        }
        sm.red[pb][0][tg][2 * cp] = mx0; sm.red[pb][0][tg][2 * cp + 1] = mx1;
        sm.red[pb][1][tg][2 * cp] = mn0; sm.red[pb][1][tg][2 * cp + 1] = mn1;
        sm.red[pb][2][tg][2 * cp] = s0;  sm.red[pb][2][tg][2 * cp + 1] = s1;
      }
    }
    __syncthreads();
    if (tid < D) {
      for (int pb = 0; pb < 2 && n0 + pb < nblk; ++pb) {
        float mx = -INFINITY, mn = INFINITY, sum = 0.f;
#pragma unroll
        for (int g = 0; g < NTG; ++g) {
          mx = fmaxf(mx, sm.red[pb][0][g][tid]);
          mn = fminf(mn, sm.red[pb][1][g][tid]);
          sum += sm.red[pb][2][g][tid];
        }
        sm.u[n0 + pb][tid] = mx;
        sm.u[n0 + pb][D + tid] = mn;
        sm.u[n0 + pb][2 * D + tid] = sum / static_cast<float>(BS);
      }
    }
    __syncthreads();
  }
  if (tid < 256) {
    constexpr int TW = DG / 64;  // 16-row tiles per wave
    constexpr int KS1 = D / 32;  // k-steps per feature section
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 15;  // A row / B column (block)
    const int g = lane >> 4;
    uint4 a[TW][3 * KS1];  // this lane's W_k pieces: row (w*TW + t)*16 + n
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const uint16_t* row = w_k_h + static_cast<int64_t>((w * TW + t) * 16 + n) * 3 * D + 8 * g;
#pragma unroll
      for (int s = 0; s < 3 * KS1; ++s) a[t][s] = ld16(row + 32 * s);
    }
    f32x4_t acc[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 5 * KS1; ++s) {  // max, min, then the mean's three components
      const int sec = s / KS1;
      const int as = (sec < 2 ? sec : 2) * KS1 + s % KS1;  // W_k k-step
      uint4 bop = make_uint4(0u, 0u, 0u, 0u);
      if (n < nblk) {
        const float* x = &sm.u[n][32 * as + 8 * g];
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = sec < 2 ? f2bf(x[i]) : bf16_part(x[i], sec - 2);
        bop = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16));
      }
#pragma unroll
      for (int t = 0; t < TW; ++t) acc[t] = mfma16x16x32(a[t][as], bop, acc[t]);
    }
    if (n < nblk) {
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.v[n][(w * TW + t) * 16 + 4 * g + r] = acc[t][r];
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
