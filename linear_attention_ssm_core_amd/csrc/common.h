// Device helpers shared by the gfx950 kernels of libgdn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Global-memory pointers.  A pointer read from memory (an array of per-sequence
// state pointers, say) is not known to the compiler to address global memory, so
// its accesses become FLAT instructions, which also count against the LDS/scalar
// counter and make the compiler wait for every outstanding memory operation at
// the next wait.  Casting to the global address space keeps them vector-memory
// operations.
template <typename T>
using gptr = __attribute__((address_space(1))) T *;
template <typename T>
__device__ __forceinline__ gptr<T> to_global(T *p) {
  return (gptr<T>)p;
}

// ---- scalar element access for the two activation dtypes --------------------
__device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16 *p, size_t i) { return (float)p[i]; }
__device__ __forceinline__ void st(float *p, size_t i, float v) { p[i] = v; }
// float -> bf16 conversion rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ void st(bf16 *p, size_t i, float v) { p[i] = (bf16)v; }

// x / (1 + e^-x), with the hardware reciprocal (about 1 ulp) instead of an IEEE
// division (a dozen instructions); e^-x -> inf gives 0, e^-x -> 0 gives x.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
// 1 / sqrt(x) on the hardware (about 1 ulp); x > 0 here (an epsilon is added).
__device__ __forceinline__ float rsqrt_hw(float x) { return __builtin_amdgcn_rsqf(x); }

// One DPP lane move within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum over each aligned group of N lanes (N = 1, 2, 4, 8 or 16), in every lane of the
// group: swaps within pairs and quads, then the half-row and row mirrors (which pair
// the two quads of an 8-lane half and the two halves of a 16-lane row).
template <int N>
__device__ __forceinline__ float sum_lanes(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "groups of up to 16 lanes");
  if (N >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if (N >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if (N >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if (N >= 16) v += dpp_f<0x140>(v); // row_mirror
  return v;
}

// Sum over all 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Sum over the lanes that share (lane mod span); span is a power of two <= 64.
template <int SPAN>
__device__ __forceinline__ float sum_across_groups(float v) {
#pragma unroll
  for (int off = SPAN; off < kWave; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Sum over the first SPAN lanes' groups: lanes l and l^off for off < SPAN.
template <int SPAN>
__device__ __forceinline__ float sum_within_span(float v) {
#pragma unroll
  for (int off = SPAN / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---- bf16 hi/lo split of an fp32 value --------------------------------------
// hi = x rounded to bf16, lo = (x - hi) rounded to bf16, so hi + lo carries about
// 16 significant bits; products of split operands are taken as
// hi*hi + hi*lo + lo*hi (the lo*lo term is below 2^-16 relative).
__device__ __forceinline__ void split_bf16(float x, bf16 &hi, bf16 &lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}
// The same split of two values as packed words (element 0 in the low half), with
// one packed conversion per pair (widening a bf16 back to fp32 is exact: it only
// appends zero bits).
struct Split2 {
  uint32_t hi, lo;
};
__device__ __forceinline__ Split2 split_bf16_2(float x0, float x1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float floatx2 __attribute__((ext_vector_type(2)));
  const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{x0, x1}, bf16x2));
  const float f0 = __builtin_bit_cast(float, hb << 16), f1 = __builtin_bit_cast(float, hb & 0xffff0000u);
  return {hb, __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{x0 - f0, x1 - f1}, bf16x2))};
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16) on the matrix cores.
// Lane l holds A row (l % 16), B column (l % 16), and the 8 k-elements of group
// (l / 16); D lane l holds column (l % 16), rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ floatx4 mfma16(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace gdn
