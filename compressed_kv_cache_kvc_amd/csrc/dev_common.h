// Device helpers: storage-type loads and the fp32 -> fp16 directed conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

struct bf16_t { uint16_t bits; };  // storage tag for bf16 arrays

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Load N consecutive storage elements starting at p (16-byte aligned) as fp32.
template <int N>
__device__ __forceinline__ void load_row(const bf16_t* p, float (&v)[N]) {
  static_assert(N % 8 == 0, "bf16 rows are loaded 8 at a time");
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    uint4 w = q[i];
    v[8 * i + 0] = bf16_lo(w.x); v[8 * i + 1] = bf16_hi(w.x);
    v[8 * i + 2] = bf16_lo(w.y); v[8 * i + 3] = bf16_hi(w.y);
    v[8 * i + 4] = bf16_lo(w.z); v[8 * i + 5] = bf16_hi(w.z);
    v[8 * i + 6] = bf16_lo(w.w); v[8 * i + 7] = bf16_hi(w.w);
  }
}

template <int N>
__device__ __forceinline__ void load_row(const float* p, float (&v)[N]) {
  static_assert(N % 4 == 0, "fp32 rows are loaded 4 at a time");
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    float4 w = q[i];
    v[4 * i + 0] = w.x; v[4 * i + 1] = w.y; v[4 * i + 2] = w.z; v[4 * i + 3] = w.w;
  }
}

// fp32 -> fp16 bit pattern rounded toward +inf (up = true) or toward -inf
// (up = false), with results beyond the fp16 range saturated to +-65504 (out of
// the codec's contract): the exact value's nearest fp16 neighbour on that side
// (11 significant bits, smallest normal 2^-14, subnormal quantum 2^-24; a tiny
// nonzero input goes to +-2^-24 or to a signed zero).  Done by the conversion
// instruction: the round-mode fields of the MODE register (bits 0-1 for fp32,
// 2-3 for fp16 and fp64; 1 = toward +inf, 2 = toward -inf, 0 = nearest even)
// are set for the one conversion and set back to nearest even in the same
// statement, with wait states on both sides of the conversion.  The input is
// first clamped to +-65504, which gives the saturation.
__device__ __forceinline__ uint32_t f32_to_f16_directed(float f, bool up) {
  const float c = __builtin_amdgcn_fmed3f(f, -65504.0f, 65504.0f);
  uint32_t r;
  if (up)
    asm volatile(
        "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 5\n\ts_nop 1\n\tv_cvt_f16_f32 %0, %1\n\ts_nop 4\n\t"
        "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 0"
        : "=v"(r)
        : "v"(c));
  else
    asm volatile(
        "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 10\n\ts_nop 1\n\tv_cvt_f16_f32 %0, %1\n\ts_nop 4\n\t"
        "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 0"
        : "=v"(r)
        : "v"(c));
  return r & 0xffffu;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(h)));
}

}  // namespace kvc
