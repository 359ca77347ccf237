// Device-side helpers shared by the ARL2 kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16, row-major M x K): lane l holds A[l % 32][8 * (l / 32) + j], j = 0..7
//   B (16 x 32, K x N):           lane l holds B[8 * (l / 32) + j][l % 32], j = 0..7
//   C (32 x 32):                  lane l, register i holds C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32]
// A C block therefore gives every lane one column and 16 rows.  When a C block is reused
// as an MFMA operand whose contraction runs over those rows, the 16 rows of lane l are read
// as the k-indices of two consecutive k-steps: k-step h, element j <-> row
// 16 h + 8 (j / 4) + 4 (l / 32) + j % 4.  Any operand paired with such a fragment uses the
// same row order; this is a permutation of the contraction index and leaves sums unchanged.
//
// v_mfma_f32_16x16x32_bf16 (the state write's per-token products):
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + j], j = 0..7
//   B (32 x 16): lane l holds B[8 * (l / 16) + j][l % 16]
//   C (16 x 16): lane l, register i holds C[4 * (l / 16) + i][l % 16]
// Two C blocks stacked over rows (rows 0-15, then 16-31) serve as one 32-deep operand of a
// contraction over those rows: element j of lane l <-> row 16 (j / 4) + 4 (l / 16) + j % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arl2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}

// 16-byte global load of 8 bf16 values (caller guarantees 16-byte alignment).
__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Row of the 32x32 C block held in register i of lane l.
__device__ __forceinline__ int c_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Value of x in the lane 32 apart (l ^ 32).
__device__ __forceinline__ float other_half(float x, int lane) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// An fp32 value as bf16 hi + bf16 lo, hi + lo = x to about 16 mantissa bits.
struct Bf16Pair {
  bf16 hi, lo;
};
__device__ __forceinline__ Bf16Pair split_bf16(float x) {
  const bf16 hi = (bf16)x;
  return {hi, (bf16)(x - (float)hi)};
}

}  // namespace arl2
