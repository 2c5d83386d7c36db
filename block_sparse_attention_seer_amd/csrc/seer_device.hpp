// Device-side helpers shared by the gfx950 kernels of libseer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seer {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 halves of a packed 32-bit word, widened exactly to float.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}
// Two floats -> packed bf16 pair (lo, hi).
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies
// A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16]; it receives
// D[4*(l/16) + r][l%16] in element r.
__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-byte and 8-byte global loads.
__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// Order-preserving map of a float to an unsigned key (larger float, larger
// key).  -0 is mapped like +0 and NaN below every number.
__device__ __forceinline__ uint32_t float_key(float z) {
  if (z != z) return 0u;
  z = z + 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of K Compression Cache entries after an update that may append up
// to max_new blocks: min(floor(L/b), c + max_new), never below the clamped
// old count c.
__device__ __forceinline__ int committed_count(int L, int c, int BS, int Lmax, int NBmax,
                                               int max_new) {
  L = min(max(L, 0), Lmax);
  c = min(max(c, 0), NBmax);
  const int nw = min(L / BS, c + max_new);
  return nw > c ? nw : c;
}

}  // namespace seer
