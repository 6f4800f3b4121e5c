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

// fp32 -> fp16 bit pattern, rounding the magnitude up (toward +inf for positive
// values) when `toward_pos_inf` matches the sign convention below.  Written from
// the IEEE-754 binary16 definition: 11 significant bits, smallest normal 2^-14,
// subnormal quantum 2^-24.  up = true rounds toward +inf, up = false toward -inf.
// Results beyond the fp16 range saturate to +-65504 (out of the codec's contract).
__device__ __forceinline__ uint32_t f32_to_f16_directed(float f, bool up) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = u >> 31;
  const uint32_t a = u & 0x7fffffffu;
  const bool mag_up = (up != (sign != 0));  // round the magnitude away from zero?
  if (a == 0) return sign << 15;
  uint32_t bits;
  if (a < 0x00800000u) {                    // fp32 subnormal: far below half the fp16 quantum
    bits = mag_up ? 1u : 0u;
  } else {
    const int e = int(a >> 23) - 127;       // value = m * 2^(e - 23), m in [2^23, 2^24)
    const uint32_t m = (a & 0x007fffffu) | 0x00800000u;
    const int qe = max(e - 10, -24);        // exponent of the fp16 quantum at this magnitude
    const int sh = qe - (e - 23);           // >= 13
    uint32_t R, rem;
    if (sh >= 32) { R = 0; rem = m; }
    else { R = m >> sh; rem = m & ((1u << sh) - 1u); }
    if (rem != 0 && mag_up) R += 1;
    // R * 2^qe with R <= 2048; the field layout absorbs a carry into the exponent
    bits = (R < 1024u) ? R : (uint32_t(qe + 24) << 10) + R;
    if (bits > 0x7bffu) bits = 0x7bffu;     // saturate at 65504
  }
  return (sign << 15) | bits;
}

// The same directed rounding by the conversion instruction: the round-mode
// fields of the MODE register (bits 0-1 for fp32, 2-3 for fp16 and fp64; 1 =
// toward +inf, 2 = toward -inf, 0 = nearest even) are set for the one
// conversion and set back to nearest even in the same statement, with wait
// states on both sides of the conversion.  The input is first clamped to
// +-65504, so that results saturate there as above.
__device__ __forceinline__ uint32_t f32_to_f16_directed_hw(float f, bool up) {
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
