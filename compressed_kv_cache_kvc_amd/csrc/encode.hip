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

// Full-dimensional encode: one thread per (token, channel group).
template <typename T, int D, int G, int BITS>
__global__ __launch_bounds__(256) void encode_kernel(const T* __restrict__ x, const T* __restrict__ cent,
                                                     const uint8_t* __restrict__ ids, int C, int64_t n,
                                                     int64_t total_items, uint8_t* __restrict__ codes,
                                                     uint32_t* __restrict__ meta) {
  constexpr int NG = D / G;
  constexpr int ROW_BYTES = D * BITS / 8;
  constexpr int CHUNK_WORDS = G * BITS / 32;  // 32-bit words of codes per group
  const int64_t item = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= total_items) return;
  const int g = int(item % NG);
  const int64_t tok = item / NG;               // h * n + j
  const int64_t h = tok / n;
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

// Low-dimensional encode: coefficients a = U^T r of each token in a rank-R basis,
// then the same quantizer over groups of G coefficients.  One thread per
// (token, coefficient); R consecutive lanes hold one token.  The basis of the
// head and the residual rows of the batch are staged in LDS.
template <typename T, int D, int R, int G, int BITS>
__global__ __launch_bounds__(256) void encode_lowdim_kernel(const T* __restrict__ x, const T* __restrict__ cent,
                                                            const uint8_t* __restrict__ ids, int C, int64_t n,
                                                            const float* __restrict__ basis,
                                                            int tokens_per_block,
                                                            uint8_t* __restrict__ codes,
                                                            uint32_t* __restrict__ meta) {
  constexpr int TPB = 256 / R;                 // tokens per pass
  constexpr int NG = R / G;
  constexpr int ROW_BYTES = R * BITS / 8;
  __shared__ float sU[D * R];
  __shared__ float sR[TPB][D + 4];
  const int h = blockIdx.y;
  const int64_t j0 = int64_t(blockIdx.x) * tokens_per_block;
  const float* Uh = basis + int64_t(h) * D * R;
  for (int i = threadIdx.x; i < D * R; i += 256) sU[i] = Uh[i];

  const int k = threadIdx.x % R;               // coefficient index
  const int tl = threadIdx.x / R;              // token within the pass
  for (int p = 0; p < tokens_per_block; p += TPB) {
    __syncthreads();
    // stage residual rows: each thread produces D*TPB/256 = D/R channels
    for (int e = threadIdx.x; e < TPB * (D / 8); e += 256) {
      const int t = e / (D / 8);
      const int c8 = e % (D / 8);
      const int64_t j = j0 + p + t;
      if (j < n) {
        const int64_t tok = int64_t(h) * n + j;
        const int id = ids[tok];
        float xv[8], cv[8];
        load_row<8>(x + tok * D + c8 * 8, xv);
        load_row<8>(cent + (int64_t(h) * C + id) * D + c8 * 8, cv);
#pragma unroll
        for (int i = 0; i < 8; ++i) sR[t][c8 * 8 + i] = __fsub_rn(xv[i], cv[i]);
      }
    }
    __syncthreads();
    const int64_t j = j0 + p + tl;
    // a_k = sum_i fl(U[i][k] * r[i]), i ascending, from +0
    float a = 0.0f;
#pragma unroll 8
    for (int i = 0; i < D; ++i) a = __fadd_rn(a, __fmul_rn(sU[i * R + k], sR[tl][i]));

    // group min / max across the G lanes holding the group's coefficients
    float mn = a, mx = a;
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
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
    uint32_t q = 0;
    if (s16 != 0) {
      const float inv = __fdiv_rn(1.0f, s);
      float t = rintf(__fmul_rn(__fsub_rn(a, z), inv));
      q = static_cast<uint32_t>(fminf(fmaxf(t, 0.0f), L));
    }
    // pack 32/BITS consecutive coefficients into one word by an OR reduction
    constexpr int PER_WORD = 32 / BITS;
    uint32_t wbits = q << (BITS * (k % PER_WORD));
#pragma unroll
    for (int off = 1; off < PER_WORD; off <<= 1) wbits |= __shfl_xor(wbits, off, 64);
    if (j < n) {
      const int64_t tok = int64_t(h) * n + j;
      if (k % PER_WORD == 0)
        reinterpret_cast<uint32_t*>(codes + tok * ROW_BYTES)[k / PER_WORD] = wbits;
      if (k % G == 0) meta[tok * NG + k / G] = s16 | (z16 << 16);
    }
  }
}

template <typename T, int D, int G, int BITS>
hipError_t run_full(int heads, int64_t n, const void* x, int C, const void* cent, const uint8_t* ids,
                    uint8_t* codes, uint16_t* meta, hipStream_t st) {
  const int64_t items = int64_t(heads) * n * (D / G);
  if (items == 0) return hipSuccess;
  const int64_t blocks = (items + 255) / 256;
  hipLaunchKernelGGL((encode_kernel<T, D, G, BITS>), dim3(unsigned(blocks)), dim3(256), 0, st,
                     static_cast<const T*>(x), static_cast<const T*>(cent), ids, C, n, items, codes,
                     reinterpret_cast<uint32_t*>(meta));
  return hipGetLastError();
}

template <typename T, int D, int R, int G, int BITS>
hipError_t run_lowdim(int heads, int64_t n, const void* x, int C, const void* cent, const uint8_t* ids,
                      const float* basis, uint8_t* codes, uint16_t* meta, hipStream_t st) {
  if (n == 0 || heads == 0) return hipSuccess;
  const int tpb = 128;
  const int64_t bx = (n + tpb - 1) / tpb;
  hipLaunchKernelGGL((encode_lowdim_kernel<T, D, R, G, BITS>), dim3(unsigned(bx), unsigned(heads)), dim3(256),
                     0, st, static_cast<const T*>(x), static_cast<const T*>(cent), ids, C, n, basis, tpb,
                     codes, reinterpret_cast<uint32_t*>(meta));
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_full(int heads, int64_t n, const void* x, int C, const void* cent, const uint8_t* ids,
                         int bits, int group, uint8_t* codes, uint16_t* meta, hipStream_t st) {
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
