// cdna4.hpp -- gfx950 (CDNA4) building blocks: bf16 vector types, the bf16
// MFMA builtins, LDS transpose reads and bf16 conversion.
//
// Operand layouts of the 32x32x16 bf16 MFMA (one 64-lane wavefront; lane l,
// half h = l / 32, column c = l % 32), checked on the device:
//   A (32 x 16, M x K): lane holds A[c][8h + e], e = 0..7
//   B (16 x 32, K x N): lane holds B[8h + e][c], e = 0..7
//   C (32 x 32):        lane holds C[8a + 4h + b][c] in register 4a + b (a, b = 0..3)
// ds_read_tr16_b64 (LDS transpose read of 16-bit elements): inside each group
// of 16 lanes, view the 16 8-byte chunks the lanes address as a 4 x 16 matrix
// whose row r is the chunks of lanes 4r..4r+3 in order; lane i receives
// column i of that matrix (its four rows, in order).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;  // 16 raw bytes
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 8-byte LDS transpose read (see the header comment for the lane mapping).
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 concat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round-to-nearest-even float -> bf16.
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

__device__ __forceinline__ float from_bf16(bf16 x) { return (float)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace fa
