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
// Two floats -> packed bf16 pair (lo, hi), one v_cvt_pk_bf16_f32 (the same
// rounding as f2bf on each).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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

// An 8-byte load marked non-temporal (`global_load ... nt`), for data read
// once per call that nothing waits on first: the decode's V rows.  Such loads
// do not allocate in the Infinity Cache, which keeps it and its allocation
// bandwidth for other traffic.  On MI355X they cost latency, so the K rows,
// which every chunk's scores wait on, use ordinary loads: streaming V only
// was measured faster than streaming both at every size from batch 1 at 8k
// tokens (latency-bound) to batch 64 at 64k (bandwidth-bound).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld8_stream(const uint16_t* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// The same for 16 bytes: keys read once by the cache build.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Part m (0, 1, 2) of the exact three-way bf16 split x = q0 + q1 + q2 (+ a
// remainder below 2^-24 |x|): q0 = bf16(x), q1 = bf16(x - q0), q2 =
// bf16(x - q0 - q1).  Each subtraction is exact in float32 (the operands
// agree in their leading bits).  bf16 x bf16 products are exact in float32,
// so an MFMA over the three parts keeps float32 accuracy.
__device__ __forceinline__ uint32_t bf16_part(float x, int m) {
  const uint16_t h0 = f2bf(x);
  const float r1 = x - __uint_as_float(static_cast<uint32_t>(h0) << 16);
  const uint16_t h1 = f2bf(r1);
  const float r2 = r1 - __uint_as_float(static_cast<uint32_t>(h1) << 16);
  const uint16_t h2 = f2bf(r2);
  return m == 0 ? h0 : (m == 1 ? h1 : h2);
}

// Order-preserving map of a float to an unsigned key (larger float, larger
// key).  -0 is mapped like +0 and NaN below every number.
__device__ __forceinline__ uint32_t float_key(float z) {
  if (z != z) return 0u;
  z = z + 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- cross-lane steps through DPP (a VALU operand modifier, no LDS round
// trip as with ds_bpermute).  GFX9 dpp_ctrl encodings.
enum : int {
  kDppXor1 = 0xB1,          // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,          // quad_perm [2,3,0,1]
  kDppRowShr = 0x110,       // + n: lane i reads lane i-n of its 16-lane row
  kDppRowMirror = 0x140,    // lane i reads lane 15-i of its row
  kDppHalfMirror = 0x141,   // lane i reads lane 7-i of its 8-lane half row
  kDppRowBcast15 = 0x142,   // lane 15 of the previous row
  kDppRowBcast31 = 0x143,   // lane 31
};

// Lane value moved by DPP control CTRL; lanes masked off or whose source
// lies outside the row read `fill`.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ int dpp_i32(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, ROW_MASK, BANK_MASK, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v), 0));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(dpp_i32<CTRL>(static_cast<int>(v), 0));
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane of a group
// receives the same value (each step adds two equal-ordered partial sums).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  if (N == 16) v += dpp_f32<kDppRowMirror>(v);
  return v;
}

__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes of a wave, the same value in every lane: 16-lane
// row sums, then the four rows in order.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return ((lane_f32(v, 0) + lane_f32(v, 16)) + lane_f32(v, 32)) + lane_f32(v, 48);
}

// Maximum / minimum over a wave (exact, so the order does not matter).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp_f32<kDppXor1>(v));
  v = fminf(v, dpp_f32<kDppXor2>(v));
  v = fminf(v, dpp_f32<kDppHalfMirror>(v));
  v = fminf(v, dpp_f32<kDppRowMirror>(v));
  return fminf(fminf(lane_f32(v, 0), lane_f32(v, 16)), fminf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppRowMirror>(v));
  return max(max(lane_u32(v, 0), lane_u32(v, 16)), max(lane_u32(v, 32), lane_u32(v, 48)));
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = min(v, dpp_u32<kDppXor1>(v));
  v = min(v, dpp_u32<kDppXor2>(v));
  v = min(v, dpp_u32<kDppHalfMirror>(v));
  v = min(v, dpp_u32<kDppRowMirror>(v));
  return min(min(lane_u32(v, 0), lane_u32(v, 16)), min(lane_u32(v, 32), lane_u32(v, 48)));
}

// ---- butterfly steps across 16- and 32-lane halves without an LDS round
// trip.  v_permlane32_swap exchanges the upper 32 lanes of its first operand
// with the lower 32 lanes of its second; given the same value twice, every
// lane l then holds the values of lanes l & ~32 (first result) and l | 32
// (second result).  v_permlane16_swap does the same between the even and odd
// 16-lane rows, for lanes l & ~16 and l | 16.  A commutative combination of
// the two values is the step "combine with lane l ^ 16 (or 32)", with the
// same bits as that step taken through ds_bpermute.
struct LanePair {
  uint32_t lo, hi;  // the values of lanes l & ~XOR and l | XOR
};
template <int XOR>
__device__ __forceinline__ LanePair lanes_xor(uint32_t v) {
  static_assert(XOR == 16 || XOR == 32, "16- or 32-lane halves");
  if constexpr (XOR == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return LanePair{r[0], r[1]};
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return LanePair{r[0], r[1]};
  }
}
template <int XOR>
__device__ __forceinline__ float max_xor(float v) {
  const LanePair r = lanes_xor<XOR>(__float_as_uint(v));
  return fmaxf(__uint_as_float(r.lo), __uint_as_float(r.hi));
}
template <int XOR>
__device__ __forceinline__ float sum_xor(float v) {
  const LanePair r = lanes_xor<XOR>(__float_as_uint(v));
  return __uint_as_float(r.lo) + __uint_as_float(r.hi);
}

// Orders the LDS accesses of one wave: the ones before complete before the
// ones after (a wave's LDS operations are performed in issue order; this
// keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele within
// each row, then row 0's total into row 1 (and row 2's into row 3), then
// the first two rows' total into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp_i32<kDppRowShr + 1>(v, 0);
  v += dpp_i32<kDppRowShr + 2>(v, 0);
  v += dpp_i32<kDppRowShr + 4>(v, 0);
  v += dpp_i32<kDppRowShr + 8>(v, 0);
  v += dpp_i32<kDppRowBcast15, 0xa>(v, 0);
  v += dpp_i32<kDppRowBcast31, 0xc>(v, 0);
  return v;
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
