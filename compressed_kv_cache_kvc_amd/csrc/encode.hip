// Residual encode: r = x - c[id] (or its coefficients in a reduced basis), then the
// per-group affine min/max quantizer with fp16 scale and zero-point, packed.
// Sources: TempoKV, section 3.1 Eq. 1 (quantizer) and section 3.3 Eq. 2 (residual
// against a prediction, here the assigned centre); NanoKV, Figure 4b (residual
// coefficients quantized and packed).
//
// Bit-exactness: every fp32 operation is written with an explicit rounding
// intrinsic (__fsub_rn, __fmul_rn, __fdiv_rn, __fadd_rn), so no multiply-add is
// fused and the sequence matches the stated operation order.
#include "kvc_internal.h"
#include "dev_common.h"
#include "mfma.h"

namespace kvc {
namespace {

// Quantize one group held by one thread and return its (scale | zero << 16) word;
// q receives the integer codes.
template <int G, int BITS>
__device__ __forceinline__ uint32_t quantize_group(const float (&r)[G], uint32_t (&q)[G]) {
  float mn = r[0], mx = r[0];
#pragma unroll
  for (int i = 1; i < G; ++i) { mn = fminf(mn, r[i]); mx = fmaxf(mx, r[i]); }
  uint32_t z16 = f32_to_f16_directed(mn, /*up=*/false);
  if ((z16 & 0x7fffu) == 0) z16 = 0;                     // zero offset stored as +0
  const float z = f16_bits_to_f32(z16);
  constexpr float L = float((1 << BITS) - 1);
  const float s32 = __fdiv_rn(__fsub_rn(mx, z), L);
  uint32_t s16 = f32_to_f16_directed(s32, /*up=*/true);
  if ((s16 & 0x7fffu) == 0) s16 = 0;
  const float s = f16_bits_to_f32(s16);
  if (s16 == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) q[i] = 0;
  } else {
    const float inv = __fdiv_rn(1.0f, s);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float t = rintf(__fmul_rn(__fsub_rn(r[i], z), inv));
      t = fminf(fmaxf(t, 0.0f), L);
      q[i] = static_cast<uint32_t>(t);
    }
  }
  return s16 | (z16 << 16);
}

// Full-dimensional encode: one thread per (token, channel group) of head
// blockIdx.y (the arrays start at the launch's first head).
template <typename T, int D, int G, int BITS>
__global__ __launch_bounds__(256) void encode_kernel(const T* __restrict__ x, const T* __restrict__ cent,
                                                     const uint8_t* __restrict__ ids, int C, int64_t n,
                                                     uint8_t* __restrict__ codes, uint32_t* __restrict__ meta) {
  constexpr int NG = D / G;
  constexpr int ROW_BYTES = D * BITS / 8;
  constexpr int CHUNK_WORDS = G * BITS / 32;  // 32-bit words of codes per group
  static_assert((NG & (NG - 1)) == 0, "groups per row: a power of two");
  const int64_t item = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;   // (token, group) within the head
  if (item >= n * NG) return;
  const int g = int(item) & (NG - 1);
  const int64_t h = blockIdx.y;
  const int64_t tok = h * n + (item >> __builtin_ctz(NG));   // h * n + j
  const int id = ids[tok];

  float xv[G], cv[G], r[G];
  load_row<G>(x + tok * D + g * G, xv);
  load_row<G>(cent + (h * C + id) * D + g * G, cv);
#pragma unroll
  for (int i = 0; i < G; ++i) r[i] = __fsub_rn(xv[i], cv[i]);

  uint32_t q[G];
  const uint32_t m = quantize_group<G, BITS>(r, q);

  uint32_t w[CHUNK_WORDS];
  constexpr int PER_WORD = 32 / BITS;
#pragma unroll
  for (int k = 0; k < CHUNK_WORDS; ++k) {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < PER_WORD; ++i) acc |= q[k * PER_WORD + i] << (BITS * i);
    w[k] = acc;
  }
  uint8_t* dst = codes + tok * ROW_BYTES + g * (G * BITS / 8);
  if constexpr (CHUNK_WORDS == 1) {
    *reinterpret_cast<uint32_t*>(dst) = w[0];
  } else if constexpr (CHUNK_WORDS == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
    static_assert(CHUNK_WORDS == 4, "unsupported chunk");
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  meta[tok * NG + g] = m;
}

// 16-bit residuals (no quantizer, no metadata): r = fl32(x - c[id]) rounded to
// fp16 nearest-even, stored per element in channel order.  One thread per
// (token, 8 channels), one 16-byte store.
template <typename T, int D>
__global__ __launch_bounds__(256) void encode_raw_kernel(const T* __restrict__ x, const T* __restrict__ cent,
                                                         const uint8_t* __restrict__ ids, int C, int64_t n,
                                                         uint8_t* __restrict__ codes) {
  constexpr int NG = D / 8;
  const int64_t item = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;   // (token, 8 channels) within the head
  if (item >= n * NG) return;
  const int g = int(item) & (NG - 1);
  const int64_t h = blockIdx.y;
  const int64_t tok = h * n + (item >> __builtin_ctz(NG));
  const int id = ids[tok];
  float xv[8], cv[8];
  load_row<8>(x + tok * D + g * 8, xv);
  load_row<8>(cent + (h * C + id) * D + g * 8, cv);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_f16x2(__fsub_rn(xv[2 * i], cv[2 * i]), __fsub_rn(xv[2 * i + 1], cv[2 * i + 1]));
  *reinterpret_cast<uint4*>(codes + tok * (D * 2) + g * 16) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Low-dimensional encode: coefficients a = U^T r of each token in a rank-R basis,
// then the same quantizer over groups of G coefficients.  A workgroup takes 64
// tokens per pass; a thread computes 4 consecutive coefficients of TT tokens
// (register tiling: one basis read and TT residual reads feed 4*TT products),
// each coefficient summed over the channels in ascending order from +0 with the
// product and the sum rounded separately.  The basis of the head and the
// residual rows of the pass (transposed, channel-major) are staged in LDS; the
// G/4 threads of a coefficient group are adjacent lanes.
template <typename T, int D, int R, int G, int BITS>
__global__ __launch_bounds__(256) void encode_lowdim_kernel(const T* __restrict__ x, const T* __restrict__ cent,
                                                            const uint8_t* __restrict__ ids, int C, int64_t n,
                                                            const float* __restrict__ basis,
                                                            int tokens_per_block,
                                                            uint8_t* __restrict__ codes,
                                                            uint32_t* __restrict__ meta) {
  constexpr int TP = 64;                       // tokens per pass
  constexpr int KQ = R / 4;                    // threads per token (4 coefficients each)
  constexpr int TS = 256 / KQ;                 // token slots per pass
  constexpr int TT = TP / TS;                  // tokens per thread
  constexpr int SR = TP + 1;                   // padded row of the transposed residuals
  constexpr int NG = R / G;
  constexpr int ROW_BYTES = R * BITS / 8;
  constexpr int GL = G / 4;                    // lanes of one coefficient group
  static_assert(TS * TT == TP && KQ <= 64, "thread layout");
  __shared__ __attribute__((aligned(16))) float sU[D * R];
  __shared__ float sR[D * SR];
  const int h = blockIdx.y;
  const int64_t j0 = int64_t(blockIdx.x) * tokens_per_block;
  const float* Uh = basis + int64_t(h) * D * R;
  for (int i = threadIdx.x; i < D * R / 4; i += 256)
    reinterpret_cast<float4*>(sU)[i] = reinterpret_cast<const float4*>(Uh)[i];

  const int kq = threadIdx.x % KQ;             // coefficients 4kq .. 4kq+3
  const int ts = threadIdx.x / KQ;             // tokens ts*TT .. ts*TT + TT-1 of the pass
  for (int p = 0; p < tokens_per_block; p += TP) {
    __syncthreads();
    // residual rows of the pass, r = fl32(x - c[id]), stored channel-major
    for (int e = threadIdx.x; e < TP * (D / 8); e += 256) {
      const int c8 = e % (D / 8);
      const int t = e / (D / 8);
      const int64_t j = j0 + p + t;
      float rv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (j < n) {
        const int64_t tok = int64_t(h) * n + j;
        const int id = ids[tok];
        float xv[8], cv[8];
        load_row<8>(x + tok * D + c8 * 8, xv);
        load_row<8>(cent + (int64_t(h) * C + id) * D + c8 * 8, cv);
#pragma unroll
        for (int i = 0; i < 8; ++i) rv[i] = __fsub_rn(xv[i], cv[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) sR[(c8 * 8 + i) * SR + t] = rv[i];
    }
    __syncthreads();
    float a[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int c = 0; c < 4; ++c) a[tt][c] = 0.0f;
#pragma unroll 4
    for (int i = 0; i < D; ++i) {
      const float4 u = *reinterpret_cast<const float4*>(&sU[i * R + 4 * kq]);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const float r = sR[i * SR + ts * TT + tt];
        a[tt][0] = __fadd_rn(a[tt][0], __fmul_rn(u.x, r));
        a[tt][1] = __fadd_rn(a[tt][1], __fmul_rn(u.y, r));
        a[tt][2] = __fadd_rn(a[tt][2], __fmul_rn(u.z, r));
        a[tt][3] = __fadd_rn(a[tt][3], __fmul_rn(u.w, r));
      }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      // group min / max across the GL lanes holding the group's coefficients
      float mn = fminf(fminf(a[tt][0], a[tt][1]), fminf(a[tt][2], a[tt][3]));
      float mx = fmaxf(fmaxf(a[tt][0], a[tt][1]), fmaxf(a[tt][2], a[tt][3]));
#pragma unroll
      for (int off = 1; off < GL; off <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 64));
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      }
      uint32_t z16 = f32_to_f16_directed(mn, false);
      if ((z16 & 0x7fffu) == 0) z16 = 0;
      const float z = f16_bits_to_f32(z16);
      constexpr float L = float((1 << BITS) - 1);
      uint32_t s16 = f32_to_f16_directed(__fdiv_rn(__fsub_rn(mx, z), L), true);
      if ((s16 & 0x7fffu) == 0) s16 = 0;
      const float s = f16_bits_to_f32(s16);
      uint32_t bits = 0;
      if (s16 != 0) {
        const float inv = __fdiv_rn(1.0f, s);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float t = rintf(__fmul_rn(__fsub_rn(a[tt][c], z), inv));
          bits |= static_cast<uint32_t>(fminf(fmaxf(t, 0.0f), L)) << (BITS * c);
        }
      }
      const int64_t j = j0 + p + ts * TT + tt;
      if (j < n) {
        const int64_t tok = int64_t(h) * n + j;
        uint8_t* crow = codes + tok * ROW_BYTES;
        if constexpr (BITS == 2) crow[kq] = static_cast<uint8_t>(bits);
        else reinterpret_cast<uint16_t*>(crow)[kq] = static_cast<uint16_t>(bits);
        if (kq % GL == 0) meta[tok * NG + kq / GL] = s16 | (z16 << 16);
      }
    }
  }
}

template <typename T, int D, int G, int BITS>
hipError_t run_full(int heads, int64_t n, const void* x, int C, const void* cent, const uint8_t* ids,
                    uint8_t* codes, uint16_t* meta, hipStream_t st) {
  if (heads == 0 || n == 0) return hipSuccess;
  const int64_t blocks = (n * (D / G) + 255) / 256;
  // the grid's second dimension takes the heads, at most 65535 per launch
  for (int h0 = 0; h0 < heads; h0 += 65535) {
    const int hc = heads - h0 < 65535 ? heads - h0 : 65535;
    hipLaunchKernelGGL((encode_kernel<T, D, G, BITS>), dim3(unsigned(blocks), unsigned(hc)), dim3(256), 0, st,
                       static_cast<const T*>(x) + int64_t(h0) * n * D, static_cast<const T*>(cent) + int64_t(h0) * C * D,
                       ids + int64_t(h0) * n, C, n, codes + int64_t(h0) * n * (D * BITS / 8),
                       reinterpret_cast<uint32_t*>(meta) + int64_t(h0) * n * (D / G));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D, int R, int G, int BITS>
hipError_t run_lowdim(int heads, int64_t n, const void* x, int C, const void* cent, const uint8_t* ids,
                      const float* basis, uint8_t* codes, uint16_t* meta, hipStream_t st) {
  if (n == 0 || heads == 0) return hipSuccess;
  const int tpb = 128;
  const int64_t bx = (n + tpb - 1) / tpb;
  // the grid's second dimension takes the heads, at most 65535 per launch
  for (int h0 = 0; h0 < heads; h0 += 65535) {
    const int hc = heads - h0 < 65535 ? heads - h0 : 65535;
    hipLaunchKernelGGL((encode_lowdim_kernel<T, D, R, G, BITS>), dim3(unsigned(bx), unsigned(hc)), dim3(256),
                       0, st, static_cast<const T*>(x) + int64_t(h0) * n * D, static_cast<const T*>(cent) + int64_t(h0) * C * D,
                       ids + int64_t(h0) * n, C, n, basis + int64_t(h0) * D * R, tpb,
                       codes + int64_t(h0) * n * (R * BITS / 8), reinterpret_cast<uint32_t*>(meta) + int64_t(h0) * n * (R / G));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D>
hipError_t dispatch_full(int heads, int64_t n, const void* x, int C, const void* cent, const uint8_t* ids,
                         int bits, int group, uint8_t* codes, uint16_t* meta, hipStream_t st) {
  if (bits == 16) {
    if (heads == 0 || n == 0) return hipSuccess;
    const int64_t blocks = (n * (D / 8) + 255) / 256;
    for (int h0 = 0; h0 < heads; h0 += 65535) {
      const int hc = heads - h0 < 65535 ? heads - h0 : 65535;
      hipLaunchKernelGGL((encode_raw_kernel<T, D>), dim3(unsigned(blocks), unsigned(hc)), dim3(256), 0, st,
                         static_cast<const T*>(x) + int64_t(h0) * n * D, static_cast<const T*>(cent) + int64_t(h0) * C * D,
                         ids + int64_t(h0) * n, C, n, codes + int64_t(h0) * n * (D * 2));
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (group == 16 && bits == 2) return run_full<T, D, 16, 2>(heads, n, x, C, cent, ids, codes, meta, st);
  if (group == 16 && bits == 4) return run_full<T, D, 16, 4>(heads, n, x, C, cent, ids, codes, meta, st);
  if (group == 32 && bits == 2) return run_full<T, D, 32, 2>(heads, n, x, C, cent, ids, codes, meta, st);
  if (group == 32 && bits == 4) return run_full<T, D, 32, 4>(heads, n, x, C, cent, ids, codes, meta, st);
  return hipErrorInvalidValue;
}

template <typename T, int R>
hipError_t dispatch_lowdim(int heads, int64_t n, const void* x, int C, const void* cent, const uint8_t* ids,
                           const float* basis, int bits, int group, uint8_t* codes, uint16_t* meta,
                           hipStream_t st) {
  if (group == 16 && bits == 2) return run_lowdim<T, 128, R, 16, 2>(heads, n, x, C, cent, ids, basis, codes, meta, st);
  if (group == 16 && bits == 4) return run_lowdim<T, 128, R, 16, 4>(heads, n, x, C, cent, ids, basis, codes, meta, st);
  if (group == 32 && bits == 2) return run_lowdim<T, 128, R, 32, 2>(heads, n, x, C, cent, ids, basis, codes, meta, st);
  if (group == 32 && bits == 4) return run_lowdim<T, 128, R, 32, 4>(heads, n, x, C, cent, ids, basis, codes, meta, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C,
                         const void* cent, const uint8_t* ids, const float* basis, int rank,
                         int bits, int group, uint8_t* codes, uint16_t* meta, hipStream_t st) {
  if (basis == nullptr) {
    if (dt == KVC_BF16 && dim == 128) return dispatch_full<bf16_t, 128>(heads, n, x, C, cent, ids, bits, group, codes, meta, st);
    if (dt == KVC_BF16 && dim == 64) return dispatch_full<bf16_t, 64>(heads, n, x, C, cent, ids, bits, group, codes, meta, st);
    if (dt == KVC_F32 && dim == 128) return dispatch_full<float, 128>(heads, n, x, C, cent, ids, bits, group, codes, meta, st);
    if (dt == KVC_F32 && dim == 64) return dispatch_full<float, 64>(heads, n, x, C, cent, ids, bits, group, codes, meta, st);
    return hipErrorInvalidValue;
  }
  if (dim != 128) return hipErrorInvalidValue;
  if (dt == KVC_BF16 && rank == 32) return dispatch_lowdim<bf16_t, 32>(heads, n, x, C, cent, ids, basis, bits, group, codes, meta, st);
  if (dt == KVC_BF16 && rank == 64) return dispatch_lowdim<bf16_t, 64>(heads, n, x, C, cent, ids, basis, bits, group, codes, meta, st);
  if (dt == KVC_F32 && rank == 32) return dispatch_lowdim<float, 32>(heads, n, x, C, cent, ids, basis, bits, group, codes, meta, st);
  if (dt == KVC_F32 && rank == 64) return dispatch_lowdim<float, 64>(heads, n, x, C, cent, ids, basis, bits, group, codes, meta, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
