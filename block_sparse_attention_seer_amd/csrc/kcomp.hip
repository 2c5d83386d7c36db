// K Compression Cache update, for gfx950 (MI355X).
//
// [CP Knowl 5] (chapterpal page "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning"): the cache holds the compressed keys
// K_gate and is updated once every b new tokens by passing the latest b keys
// through the pooling and linear layers.  [CP Knowl 1, Knowl 2]: pooling is
// non-overlapping with kernel = stride = b; max, min and average outputs are
// concatenated (3d values) and mapped by W_k (d_gate x 3d); RoPE is then
// applied at the position of the block's first token.
//
// One workgroup per (sequence, KV head, new block): pool the block's b x d
// keys (coalesced 4-byte pieces, then an LDS reduction), run the 3d -> d_gate
// GEMV with one wave per row set (coalesced W_k rows, wave reductions),
// rotate in float64 and store bf16 (round to nearest even).  A second tiny
// kernel raises kcomp_lens once every entry is in place, so concurrent
// workgroups never see a half-updated count.
#include <cmath>

#include "seer_device.hpp"
#include "seer_internal.h"

namespace seer {

namespace {

struct KcompParams {
  const uint16_t* k_nope;
  const uint16_t* w_k;
  const int32_t* seq_lens;
  const int32_t* kcomp_lens;
  uint16_t* kcomp;
  int64_t sb, sh;
  int st;
  int Hkv, BS, Lmax, NBmax, max_new;
  double theta;
};

template <int D, int DG>
__global__ __launch_bounds__(256) void kcomp_kernel(KcompParams p) {
  constexpr int CP = D / 2;       // channel pairs
  constexpr int NTG = 256 / CP;   // token groups
  __shared__ float s_red[3][NTG][D];
  __shared__ float s_u[3 * D];
  __shared__ float s_v[DG];

  const int pair = blockIdx.x;
  const int b = pair / p.Hkv;
  const int h = pair - b * p.Hkv;
  int L = p.seq_lens[b];
  L = min(max(L, 0), p.Lmax);
  const int nb = L / p.BS;
  int c = p.kcomp_lens[b];
  c = min(max(c, 0), p.NBmax);
  const int j = c + static_cast<int>(blockIdx.y);
  if (j >= nb) return;

  const int tid = threadIdx.x;
  // ---- pooling
  {
    const int cp = tid % CP;
    const int tg = tid / CP;
    const uint16_t* base = p.k_nope + b * p.sb + h * p.sh + static_cast<int64_t>(j) * p.BS * p.st + 2 * cp;
    float mx0 = -INFINITY, mx1 = -INFINITY, mn0 = INFINITY, mn1 = INFINITY, s0 = 0.f, s1 = 0.f;
    for (int t = tg; t < p.BS; t += NTG) {
      const uint32_t wv = *reinterpret_cast<const uint32_t*>(base + t * p.st);
      const float a = bf_lo(wv), bb = bf_hi(wv);
      mx0 = fmaxf(mx0, a); mn0 = fminf(mn0, a); s0 += a;
      mx1 = fmaxf(mx1, bb); mn1 = fminf(mn1, bb); s1 += bb;
    }
    s_red[0][tg][2 * cp] = mx0; s_red[0][tg][2 * cp + 1] = mx1;
    s_red[1][tg][2 * cp] = mn0; s_red[1][tg][2 * cp + 1] = mn1;
    s_red[2][tg][2 * cp] = s0;  s_red[2][tg][2 * cp + 1] = s1;
  }
  __syncthreads();
  if (tid < D) {
    float mx = -INFINITY, mn = INFINITY, sm = 0.f;
#pragma unroll
    for (int g = 0; g < NTG; ++g) {
      mx = fmaxf(mx, s_red[0][g][tid]);
      mn = fminf(mn, s_red[1][g][tid]);
      sm += s_red[2][g][tid];
    }
    s_u[tid] = mx;
    s_u[D + tid] = mn;
    s_u[2 * D + tid] = sm / static_cast<float>(p.BS);
  }
  __syncthreads();

  // ---- v = W_k[h] . u : wave w handles rows w, w+4, ...
  {
    const int w = tid >> 6;
    const int lane = tid & 63;
    const uint16_t* wk = p.w_k + static_cast<int64_t>(h) * DG * 3 * D;
    for (int r = w; r < DG; r += 4) {
      const uint32_t* row = reinterpret_cast<const uint32_t*>(wk + static_cast<int64_t>(r) * 3 * D);
      float acc = 0.f;
      for (int q2 = lane; q2 < 3 * D / 2; q2 += 64) {
        const uint32_t wv = row[q2];
        acc = fmaf(bf_lo(wv), s_u[2 * q2], acc);
        acc = fmaf(bf_hi(wv), s_u[2 * q2 + 1], acc);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
      if (lane == 0) s_v[r] = acc;
    }
  }
  __syncthreads();

  // ---- RoPE at the block's first token, bf16 store
  if (tid < DG / 2) {
    const int i = tid;
    const double w = pow(p.theta, -2.0 * static_cast<double>(i) / static_cast<double>(DG));
    double sn, cs;
    sincos(static_cast<double>(j) * p.BS * w, &sn, &cs);
    const double lo = s_v[i], hi = s_v[i + DG / 2];
    const float olo = static_cast<float>(lo * cs - hi * sn);
    const float ohi = static_cast<float>(hi * cs + lo * sn);
    uint16_t* dst = p.kcomp + ((static_cast<int64_t>(pair) * p.NBmax) + j) * DG;
    dst[i] = f2bf(olo);
    dst[i + DG / 2] = f2bf(ohi);
  }
}

__global__ void kcomp_commit_kernel(const int32_t* seq_lens, int32_t* kcomp_lens, int B, int BS,
                                    int Lmax, int NBmax, int max_new) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int L = seq_lens[b];
  L = min(max(L, 0), Lmax);
  const int nb = L / BS;
  int c = kcomp_lens[b];
  c = min(max(c, 0), NBmax);
  const int nw = min(nb, c + max_new);
  if (nw > c) kcomp_lens[b] = nw;
  else if (kcomp_lens[b] != c) kcomp_lens[b] = c;  // clamp an out-of-range count
}

}  // namespace

int launch_kcomp(const seer_dims& d, const KcompArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  KcompParams p{a.k_nope, a.w_k, a.seq_lens, a.kcomp_lens, a.kcomp, d.kv_stride_b, d.kv_stride_h,
                static_cast<int>(d.kv_stride_t), d.num_kv_heads, d.block_size, d.max_seq_len,
                static_cast<int>(nb_max(&d)), a.max_new_blocks, a.theta};
  dim3 grid(d.batch * d.num_kv_heads, a.max_new_blocks);
  const int key = (d.head_dim == 128 ? 2 : 0) | (d.d_gate == 128 ? 1 : 0);
  switch (key) {
    case 0: hipLaunchKernelGGL((kcomp_kernel<64, 64>), grid, dim3(256), 0, s, p); break;
    case 1: hipLaunchKernelGGL((kcomp_kernel<64, 128>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((kcomp_kernel<128, 64>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((kcomp_kernel<128, 128>), grid, dim3(256), 0, s, p); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("kcomp launch: ") + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  hipLaunchKernelGGL(kcomp_commit_kernel, dim3((d.batch + 255) / 256), dim3(256), 0, s,
                     a.seq_lens, a.kcomp_lens, d.batch, d.block_size, d.max_seq_len,
                     static_cast<int>(nb_max(&d)), a.max_new_blocks);
  e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("kcomp commit launch: ") + hipGetErrorString(e));
    return SEER_ERR_HIP;
  }
  return SEER_OK;
}

}  // namespace seer
