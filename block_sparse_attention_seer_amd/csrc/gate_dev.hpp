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

// Shared-memory scratch of the cache-entry computation of up to NB blocks:
// the pooled features (max and min as bf16 bits -- the max or min of bf16
// keys is one of them -- and the float32 mean as its three bf16 parts, the
// MFMA B operands as they are), then, in the same bytes once every wave has
// read them, V = W_k u.
template <int D, int DG, int NB = 1>
struct alignas(16) CompressSmem {  // 16-byte aligned: the MFMA operands are read as 16-byte LDS words
  static_assert(NB >= 1 && NB <= 32, "up to two 16-column MFMA tiles of blocks");
  struct Pooled {
    uint16_t mx[NB][D + 8];  // rows padded (16-byte aligned, fewer bank conflicts)
    uint16_t mn[NB][D + 8];
    uint16_t mean[3][NB][D + 8];  // the mean's exact three-way bf16 split
  };
  union {
    Pooled u;
    float v[NB][DG];
  };
};

// Max, min and mean over the b keys of each block n = n0, n0 + nstep, ...
// < nblk (block n's rows start at keys + n*b*st), by one wave: lane l reads
// the 16-byte chunk l % (D/8) (8 channels) of tokens l / (D/8) + i*Q,
// i = 0, 1, ... (Q = 64 / (D/8) token groups; a wave instruction reads Q
// whole key rows), reduces them in i order, then the Q groups are folded by
// butterfly exchanges (offsets D/8, 2 D/8, ...); every lane ends with the
// same sums.  The loads of the next batch of kPoolBatch tokens per lane
// (possibly of the next block) are in flight while a batch is reduced.  The lanes of
// group 0 write block n's max and min (bf16 bits) and the three bf16 parts of
// sum / b to u.
// Max and min are taken on order keys of the bf16 bit patterns, two
// channels per 32-bit word with packed 16-bit integer max / min: for a bf16
// pattern x read as int16, key(x) = x ^ ((x >> 15) & 0x7fff) orders like the
// values (negative patterns get their magnitude bits flipped; -0 sorts just
// below +0), and key(key(x)) = x.  The max or min of bf16 values is one of
// them, so no float conversion is needed.  The sums are float32.
typedef short pool_s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ pool_s16x2 bf16x2_order_key(uint32_t w) {
  const pool_s16x2 x = __builtin_bit_cast(pool_s16x2, w);
  return x ^ ((x >> 15) & static_cast<short>(0x7fff));
}

template <int D>
struct PoolAcc {
  pool_s16x2 kmx[4], kmn[4];  // order keys of channels (2k, 2k + 1)
  float sm[8];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      kmx[k] = pool_s16x2{static_cast<short>(-32768), static_cast<short>(-32768)};
      kmn[k] = pool_s16x2{32767, 32767};
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) sm[k] = 0.f;
  }
};

constexpr int kPoolBatch = 4;  // 16-byte loads in flight per lane and buffer

template <int D>
__device__ __forceinline__ void pool_load(uint4 (&buf)[kPoolBatch], const uint16_t* keys,
                                          int64_t st, int BS, int n, int bt) {
  constexpr int CH = D / 8;
  constexpr int Q = 64 / CH;
  const int lane = threadIdx.x & 63;
  const uint16_t* base = keys + static_cast<int64_t>(n) * BS * st +
                         static_cast<int64_t>(lane / CH) * st + 8 * (lane % CH);
  // every lane has b / Q tokens per block, a multiple of the batch for the
  // block sizes built (64 and 128): the loads need no bounds test
  const uint16_t* p = base + static_cast<int64_t>(bt) * kPoolBatch * Q * st;
  const int64_t step = static_cast<int64_t>(Q) * st;
#pragma unroll
  for (int i = 0; i < kPoolBatch; ++i) buf[i] = ld16_stream(p + i * step);
}

template <int D>
__device__ __forceinline__ void pool_reduce(PoolAcc<D>& acc, const uint4 (&buf)[kPoolBatch]) {
#pragma unroll
  for (int i = 0; i < kPoolBatch; ++i) {
    const uint32_t w4[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const pool_s16x2 key = bf16x2_order_key(w4[k]);
      acc.kmx[k] = __builtin_elementwise_max(acc.kmx[k], key);
      acc.kmn[k] = __builtin_elementwise_min(acc.kmn[k], key);
      acc.sm[2 * k] += bf_lo(w4[k]);
      acc.sm[2 * k + 1] += bf_hi(w4[k]);
    }
  }
}

template <int D>
__device__ __forceinline__ void pool_finish(PoolAcc<D>& acc, int BS, uint16_t* mx_row,
                                            uint16_t* mn_row, uint16_t* m0_row, uint16_t* m1_row,
                                            uint16_t* m2_row) {
  constexpr int CH = D / 8;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = CH; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t omx = __shfl_xor(__builtin_bit_cast(uint32_t, acc.kmx[k]), off);
      const uint32_t omn = __shfl_xor(__builtin_bit_cast(uint32_t, acc.kmn[k]), off);
      acc.kmx[k] = __builtin_elementwise_max(acc.kmx[k], __builtin_bit_cast(pool_s16x2, omx));
      acc.kmn[k] = __builtin_elementwise_min(acc.kmn[k], __builtin_bit_cast(pool_s16x2, omn));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc.sm[k] = acc.sm[k] + __shfl_xor(acc.sm[k], off);
  }
  if (lane < CH) {
    const int c = lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // the key map is its own inverse: back to bf16 bits
      reinterpret_cast<uint32_t*>(mx_row)[4 * c + k] =
          __builtin_bit_cast(uint32_t, bf16x2_order_key(__builtin_bit_cast(uint32_t, acc.kmx[k])));
      reinterpret_cast<uint32_t*>(mn_row)[4 * c + k] =
          __builtin_bit_cast(uint32_t, bf16x2_order_key(__builtin_bit_cast(uint32_t, acc.kmn[k])));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float x = acc.sm[k] / static_cast<float>(BS);
      m0_row[8 * c + k] = static_cast<uint16_t>(bf16_part(x, 0));
      m1_row[8 * c + k] = static_cast<uint16_t>(bf16_part(x, 1));
      m2_row[8 * c + k] = static_cast<uint16_t>(bf16_part(x, 2));
    }
  }
}

template <int D, int DG, int NB>
__device__ __forceinline__ void pool_blocks_wave(const uint16_t* keys, int64_t st, int BS,
                                                 int n0, int nstep, int nblk,
                                                 typename CompressSmem<D, DG, NB>::Pooled& u) {
  constexpr int CH = D / 8;
  constexpr int Q = 64 / CH;
  const int nbat = (BS / Q + kPoolBatch - 1) / kPoolBatch;  // batches per block (wave-uniform)
  const int nmine = n0 < nblk ? (nblk - n0 + nstep - 1) / nstep : 0;
  const int total = nmine * nbat;
  if (total == 0) return;
  PoolAcc<D> acc;
  acc.reset();
  uint4 b0[kPoolBatch], b1[kPoolBatch];
  pool_load<D>(b0, keys, st, BS, n0, 0);
  for (int k = 0; k < total; k += 2) {
    // batch k in b0; batch k + 1 (if any) loaded into b1 before reducing b0
    const int n_k = n0 + (k / nbat) * nstep, bt_k = k % nbat;
    if (k + 1 < total)
      pool_load<D>(b1, keys, st, BS, n0 + ((k + 1) / nbat) * nstep, (k + 1) % nbat);
    pool_reduce<D>(acc, b0);
    if (bt_k == nbat - 1) {
      pool_finish<D>(acc, BS, u.mx[n_k], u.mn[n_k], u.mean[0][n_k], u.mean[1][n_k],
                     u.mean[2][n_k]);
      acc.reset();
    }
    if (k + 1 >= total) break;
    const int n_k1 = n0 + ((k + 1) / nbat) * nstep, bt_k1 = (k + 1) % nbat;
    if (k + 2 < total)
      pool_load<D>(b0, keys, st, BS, n0 + ((k + 2) / nbat) * nstep, (k + 2) % nbat);
    pool_reduce<D>(acc, b1);
    if (bt_k1 == nbat - 1) {
      pool_finish<D>(acc, BS, u.mx[n_k1], u.mn[n_k1], u.mean[0][n_k1], u.mean[1][n_k1],
                     u.mean[2][n_k1]);
      acc.reset();
    }
  }
}

// K Compression Cache entries of blocks j0 .. j0+nblk-1 (nblk <= NB,
// consecutive blocks of one pair; keys points at row 0 of block j0, dst at
// entry j0) computed by the first 256 threads of the workgroup; every thread
// of the workgroup must call this (it contains barriers).  A block's
// arithmetic does not depend on NB or nblk (MFMA columns are independent),
// so an entry has the same bits whichever way the cache is built.
//   pooling: wave w of the first four takes blocks w, w + 4, ... (one block
//   at a time per wave, pool_blocks_wave), with no barrier until all are
//   pooled;
//   GEMV on MFMA: V[row][block] = W_k[row][:] . u[block][:], the blocks as
//   B-operand columns (16 per tile); max and min features are exact in bf16, the
//   mean enters as three bf16 components against the same W_k columns;
//   RoPE at position j*b (float64 angle), bf16 store (round to nearest even)
//   to dst and, when lds_copy is not null, to LDS ([NB][DG]) as well.
//   wf is this thread's RoPE frequency, theta^(-2(t mod DG/2)/DG) for thread t.
template <int D, int DG, int NB>
__device__ __forceinline__ void compress_blocks(CompressSmem<D, DG, NB>& sm, const uint16_t* keys,
                                                int64_t st, int BS, const uint16_t* w_k_h,
                                                double wf, int j0, int nblk, uint16_t* dst,
                                                uint16_t* lds_copy = nullptr) {
  constexpr int TW = DG / 64;          // 16-row tiles per wave
  constexpr int NCT = (NB + 15) / 16;  // 16-column tiles of blocks
  constexpr int KS1 = D / 32;          // k-steps per feature section
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;  // A row; B column (block) n + 16 ct
  const int g = lane >> 4;
  if (tid < 256) pool_blocks_wave<D, DG, NB>(keys, st, BS, w, 4, nblk, sm.u);
  __syncthreads();
  f32x4_t acc[TW][NCT];
  if (tid < 256) {
    const uint16_t* wrow[TW];  // this lane's W_k rows (w*TW + t)*16 + n
#pragma unroll
    for (int t = 0; t < TW; ++t)
      wrow[t] = w_k_h + static_cast<int64_t>((w * TW + t) * 16 + n) * 3 * D + 8 * g;
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // k-steps in the order max, min, then the mean's three parts (each
    // against the mean's W_k columns); W_k is read one feature section at a
    // time, the next section's pieces requested before this one's products
    uint4 a[TW][KS1], an[TW][KS1];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int k = 0; k < KS1; ++k) a[t][k] = ld16(wrow[t] + 32 * k);
#pragma unroll
    for (int sec = 0; sec < 3; ++sec) {
      if (sec < 2) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
          for (int k = 0; k < KS1; ++k) an[t][k] = ld16(wrow[t] + 32 * ((sec + 1) * KS1 + k));
      }
#pragma unroll
      for (int part = 0; part < (sec < 2 ? 1 : 3); ++part) {
#pragma unroll
        for (int k = 0; k < KS1; ++k) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const int nb = n + 16 * ct;
            uint4 bop = make_uint4(0u, 0u, 0u, 0u);
            if (nb < nblk) {
              const uint16_t* src = sec == 0 ? sm.u.mx[nb]
                                  : sec == 1 ? sm.u.mn[nb]
                                             : sm.u.mean[part][nb];
              bop = *reinterpret_cast<const uint4*>(src + 32 * k + 8 * g);
            }
#pragma unroll
            for (int t = 0; t < TW; ++t) acc[t][ct] = mfma16x16x32(a[t][k], bop, acc[t][ct]);
          }
        }
      }
      if (sec < 2) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
          for (int k = 0; k < KS1; ++k) a[t][k] = an[t][k];
      }
    }
  }
  __syncthreads();  // every wave has read the pooled features: V takes their place
  if (tid < 256) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int nb = n + 16 * ct;
      if (nb < nblk) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.v[nb][(w * TW + t) * 16 + 4 * g + r] = acc[t][ct][r];
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
