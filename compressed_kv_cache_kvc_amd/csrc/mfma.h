// CDNA4 (gfx950) matrix-core fragments used by the assignment and attention kernels.
//
// v_mfma_f32_32x32x16_bf16 computes D = A B + C for A: 32x16 (M x K), B: 16x32
// (K x N), C/D: 32x32 fp32.  Operand layout per 64-lane wavefront, lane l:
//   A: row i = l % 32, columns k = 8*(l / 32) .. +7   (8 bf16 in 4 VGPRs)
//   B: column j = l % 32, rows k = 8*(l / 32) .. +7
//   D: column j = l % 32, rows i = 8*(v / 4) + 4*(l / 32) + (v % 4) for v = 0..15
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }
__device__ __forceinline__ uint4 as_uint4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x8 as_f16x8(uint4 w) { return __builtin_bit_cast(f16x8, w); }

// Same layout as mfma32, fp16 operands (v_mfma_f32_32x32x16_f16, same rate as bf16).
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Round two fp32 values to fp16 (nearest even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {lo, hi};
  f16x2 h = __builtin_convertvector(f, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Round two fp32 values to bf16 (nearest even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

}  // namespace kvc
