// Predictive residual coding of the cache over latent frames (TempoKV, section
// 3.3, Eqs. 2-4 and "Anchor frames"): each key is predicted from the keys of the
// same spatial token in the two previous frames as they were reconstructed
// (Eq. 3; the first frame after the anchor has its own coefficients), each value
// from the reconstructed key of the same token through a dense D x D map plus the
// previous frame's reconstructed value (Eq. 4); only the residual against the
// prediction is quantized (Eq. 2), with the group quantizer of the centre codec.
// The anchor frame (frame 0) is coded without prediction.
//
// A reconstruction depends on the reconstructions of earlier frames, so the
// frames of a token are walked in order, while the spatial tokens of a frame are
// independent: one wavefront per (head, spatial token) walks the call's frames,
// keeping the reconstructed history (two key frames, one value frame) in
// registers; lane l holds channels l*PER .. l*PER + PER - 1.  A group's minimum
// and maximum come from shuffles over its lanes; the dense map W is staged in LDS
// transposed, so the lanes read consecutive words, and the reconstructed key
// reaches every lane one channel at a time through readlane.
//
// Every fp32 operation is written with an explicit rounding intrinsic, in one
// fixed order:
//   k_tilde = ((beta_k + A1*k1) + A2*k2)          (A2 term only with two key frames)
//   v_tilde = (beta_v + W[c][0]*k_hat[0] + ... + W[c][D-1]*k_hat[D-1]) + A_v*v1
//   r = x - x_tilde;  x_hat = x_tilde + (q*s + z)
// so the codes are unique and a decode reproduces the encoder's reconstruction
// bit for bit.
#include "kvc_internal.h"
#include "dev_common.h"
#include "mfma.h"

namespace kvc {
namespace {

struct TempoArgs {
  const void* k;           // encode: [H][n_frames*S][D] keys (storage dtype)
  const void* v;
  const float* prm;        // [H][7D + D*D]
  uint8_t* k_codes;        // [H][n_frames*S][D*KB/8]
  uint32_t* k_meta;        // [H][n_frames*S][D/G] (scale | zero << 16)
  uint8_t* v_codes;
  uint32_t* v_meta;
  float* state;            // [H][S][3][D]: K_hat[f-1], K_hat[f-2], V_hat[f-1]
  uint16_t* k_hat;         // decode: [H][n_frames*S][D] fp16
  uint16_t* v_hat;
  int S;
  int first_frame;
  int n_frames;
};

constexpr int kTempoWaves = 16;          // spatial tokens (wavefronts) per workgroup

template <typename T, int PER>
__device__ __forceinline__ void load_lane(const T* row, int lane, float (&x)[PER]) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (PER == 2) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
      x[0] = bf16_lo(w);
      x[1] = bf16_hi(w);
    } else {
      x[0] = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(row)[lane]) << 16);
    }
  } else {
    if constexpr (PER == 2) {
      const float2 w = reinterpret_cast<const float2*>(row)[lane];
      x[0] = w.x;
      x[1] = w.y;
    } else {
      x[0] = reinterpret_cast<const float*>(row)[lane];
    }
  }
}

// Quantize the residual r (this lane's PER channels) by groups of G channels
// spread over G/PER lanes; returns the group's (scale | zero << 16) and the codes.
// Same operations as the centre codec's quantizer, with the group's minimum and
// maximum gathered across lanes.
template <int G, int BITS, int PER>
__device__ __forceinline__ uint32_t quantize_lanes(const float (&r)[PER], uint32_t (&q)[PER]) {
  float mn = r[0], mx = r[0];
#pragma unroll
  for (int i = 1; i < PER; ++i) { mn = fminf(mn, r[i]); mx = fmaxf(mx, r[i]); }
#pragma unroll
  for (int o = 1; o < G / PER; o <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, 64));
    mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  }
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
    for (int i = 0; i < PER; ++i) q[i] = 0;
  } else {
    const float inv = __fdiv_rn(1.0f, s);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float t = rintf(__fmul_rn(__fsub_rn(r[i], z), inv));
      t = fminf(fmaxf(t, 0.0f), L);
      q[i] = static_cast<uint32_t>(t);
    }
  }
  return s16 | (z16 << 16);
}

// r_hat = q*s + z (q*s is exact in fp32; one rounding of the sum)
template <int PER>
__device__ __forceinline__ void dequant_lane(const uint32_t (&q)[PER], uint32_t m, float (&rh)[PER]) {
  const float s = f16_bits_to_f32(m & 0xffffu), z = f16_bits_to_f32(m >> 16);
#pragma unroll
  for (int i = 0; i < PER; ++i) rh[i] = __fadd_rn(__fmul_rn(float(q[i]), s), z);
}

// Packed codes of one row: lane l's PER codes occupy bits BITS*PER*(l % LW) of
// 32-bit word l / LW (channel c at bit BITS*(c mod 32/BITS) of word c/(32/BITS),
// the byte layout of the codec).  Lanes l % LW == 0 write the words.
template <int BITS, int PER>
__device__ __forceinline__ void store_codes(uint8_t* row, int lane, const uint32_t (&q)[PER]) {
  constexpr int BL = BITS * PER, LW = 32 / BL;
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) w |= q[i] << (BITS * i);
  w <<= BL * (lane % LW);
#pragma unroll
  for (int o = 1; o < LW; o <<= 1) w |= __shfl_xor(w, o, 64);
  if (lane % LW == 0) reinterpret_cast<uint32_t*>(row)[lane / LW] = w;
}

template <int BITS, int PER>
__device__ __forceinline__ void load_codes(const uint8_t* row, int lane, uint32_t (&q)[PER]) {
  constexpr int BL = BITS * PER, LW = 32 / BL;
  const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane / LW] >> (BL * (lane % LW));
#pragma unroll
  for (int i = 0; i < PER; ++i) q[i] = (w >> (BITS * i)) & ((1u << BITS) - 1u);
}

template <typename T, int D, int KB, int VB, int G, bool DECODE>
__global__ __launch_bounds__(64 * kTempoWaves, 8) void tempo_kernel(TempoArgs a) {
  constexpr int PER = D / 64;
  constexpr int NP = 7 * D + D * D;
  __shared__ float sWt[D * D];                       // sWt[j * D + c] = W[c][j]
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* P = a.prm + int64_t(h) * NP;
  for (int idx = threadIdx.x; idx < D * D; idx += 64 * kTempoWaves) {
    const int c = idx / D, j = idx % D;              // reads run along a row of W
    sWt[j * D + c] = P[7 * D + idx];
  }
  __syncthreads();
  const int s = blockIdx.x * kTempoWaves + wave;
  if (s >= a.S) return;                              // wave-uniform; no barrier follows

  float bk1[PER], ak1[PER], bk2[PER], ak21[PER], ak22[PER], bv[PER], av[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = lane * PER + i;
    bk1[i] = P[c]; ak1[i] = P[D + c]; bk2[i] = P[2 * D + c]; ak21[i] = P[3 * D + c]; ak22[i] = P[4 * D + c];
    bv[i] = P[5 * D + c]; av[i] = P[6 * D + c];
  }
  float* st = a.state + (int64_t(h) * a.S + s) * 3 * D + lane * PER;
  float k1[PER], k2[PER], v1[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    k1[i] = a.first_frame > 0 ? st[i] : 0.f;
    k2[i] = a.first_frame > 0 ? st[D + i] : 0.f;
    v1[i] = a.first_frame > 0 ? st[2 * D + i] : 0.f;
  }
  const int64_t rows = int64_t(a.n_frames) * a.S;
  for (int f = 0; f < a.n_frames; ++f) {
    const int t = a.first_frame + f;
    const int64_t row = int64_t(h) * rows + int64_t(f) * a.S + s;
    // ---- keys (Eq. 3)
    float kt[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (t == 0) kt[i] = 0.f;
      else if (t == 1) kt[i] = __fadd_rn(bk1[i], __fmul_rn(ak1[i], k1[i]));
      else kt[i] = __fadd_rn(__fadd_rn(bk2[i], __fmul_rn(ak21[i], k1[i])), __fmul_rn(ak22[i], k2[i]));
    }
    uint32_t q[PER];
    uint32_t m;
    if constexpr (!DECODE) {
      float x[PER], r[PER];
      load_lane<T, PER>(static_cast<const T*>(a.k) + row * D, lane, x);
#pragma unroll
      for (int i = 0; i < PER; ++i) r[i] = __fsub_rn(x[i], kt[i]);
      m = quantize_lanes<G, KB, PER>(r, q);
      store_codes<KB, PER>(a.k_codes + row * (D * KB / 8), lane, q);
      if (lane % (G / PER) == 0) a.k_meta[row * (D / G) + lane * PER / G] = m;
    } else {
      load_codes<KB, PER>(a.k_codes + row * (D * KB / 8), lane, q);
      m = a.k_meta[row * (D / G) + lane * PER / G];
    }
    float kh[PER], rh[PER];
    dequant_lane<PER>(q, m, rh);
#pragma unroll
    for (int i = 0; i < PER; ++i) kh[i] = __fadd_rn(kt[i], rh[i]);
    // ---- values (Eq. 4)
    float vt[PER];
    if (t == 0) {
#pragma unroll
      for (int i = 0; i < PER; ++i) vt[i] = 0.f;
    } else {
      float acc[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = bv[i];
#pragma unroll 4
      for (int jl = 0; jl < 64; ++jl) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int j = jl * PER + e;               // input channel, ascending
          const float kj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(kh[e]), jl));
          const float* wr = &sWt[j * D + lane * PER];
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] = __fadd_rn(acc[i], __fmul_rn(wr[i], kj));
        }
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) vt[i] = __fadd_rn(acc[i], __fmul_rn(av[i], v1[i]));
    }
    if constexpr (!DECODE) {
      float x[PER], r[PER];
      load_lane<T, PER>(static_cast<const T*>(a.v) + row * D, lane, x);
#pragma unroll
      for (int i = 0; i < PER; ++i) r[i] = __fsub_rn(x[i], vt[i]);
      m = quantize_lanes<G, VB, PER>(r, q);
      store_codes<VB, PER>(a.v_codes + row * (D * VB / 8), lane, q);
      if (lane % (G / PER) == 0) a.v_meta[row * (D / G) + lane * PER / G] = m;
    } else {
      load_codes<VB, PER>(a.v_codes + row * (D * VB / 8), lane, q);
      m = a.v_meta[row * (D / G) + lane * PER / G];
    }
    float vh[PER];
    dequant_lane<PER>(q, m, rh);
#pragma unroll
    for (int i = 0; i < PER; ++i) vh[i] = __fadd_rn(vt[i], rh[i]);
    if constexpr (DECODE) {
      // reconstructions as fp16 (nearest even), the precision of the attention tiles
      if constexpr (PER == 2) {
        reinterpret_cast<uint32_t*>(a.k_hat + row * D)[lane] = pack_f16x2(kh[0], kh[1]);
        reinterpret_cast<uint32_t*>(a.v_hat + row * D)[lane] = pack_f16x2(vh[0], vh[1]);
      } else {
        a.k_hat[row * D + lane] = static_cast<uint16_t>(pack_f16x2(kh[0], 0.f) & 0xffffu);
        a.v_hat[row * D + lane] = static_cast<uint16_t>(pack_f16x2(vh[0], 0.f) & 0xffffu);
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      k2[i] = k1[i];
      k1[i] = kh[i];
      v1[i] = vh[i];
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    st[i] = k1[i];
    st[D + i] = k2[i];
    st[2 * D + i] = v1[i];
  }
}

template <typename T, int D, bool DECODE>
hipError_t pick_tempo(const TempoArgs& a, int heads, int kb, int vb, int g, hipStream_t st) {
  const dim3 grid(unsigned((a.S + kTempoWaves - 1) / kTempoWaves), unsigned(heads));
#define KVC_TEMPO(KB_, VB_, G_)                                                                             \
  if (kb == KB_ && vb == VB_ && g == G_) {                                                                  \
    hipLaunchKernelGGL((tempo_kernel<T, D, KB_, VB_, G_, DECODE>), grid, dim3(64 * kTempoWaves), 0, st, a); \
    return hipGetLastError();                                                                               \
  }
  KVC_TEMPO(2, 2, 16) KVC_TEMPO(2, 4, 16) KVC_TEMPO(4, 2, 16) KVC_TEMPO(4, 4, 16)
  KVC_TEMPO(2, 2, 32) KVC_TEMPO(2, 4, 32) KVC_TEMPO(4, 2, 32) KVC_TEMPO(4, 4, 32)
#undef KVC_TEMPO
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_tempo(bool decode, int heads, int S, int first_frame, int n_frames, int dim, kvc_dtype dt,
                        const void* k, const void* v, const float* prm, int kb, int vb, int g, uint8_t* k_codes,
                        uint16_t* k_meta, uint8_t* v_codes, uint16_t* v_meta, float* state, uint16_t* k_hat,
                        uint16_t* v_hat, hipStream_t st) {
  if (heads == 0 || S == 0 || n_frames == 0) return hipSuccess;
  TempoArgs a;
  a.k = k;
  a.v = v;
  a.prm = prm;
  a.k_codes = k_codes;
  a.k_meta = reinterpret_cast<uint32_t*>(k_meta);
  a.v_codes = v_codes;
  a.v_meta = reinterpret_cast<uint32_t*>(v_meta);
  a.state = state;
  a.k_hat = k_hat;
  a.v_hat = v_hat;
  a.S = S;
  a.first_frame = first_frame;
  a.n_frames = n_frames;
  if (decode) {
    if (dim == 128) return pick_tempo<bf16_t, 128, true>(a, heads, kb, vb, g, st);
    if (dim == 64) return pick_tempo<bf16_t, 64, true>(a, heads, kb, vb, g, st);
    return hipErrorInvalidValue;
  }
  if (dt == KVC_BF16) {
    if (dim == 128) return pick_tempo<bf16_t, 128, false>(a, heads, kb, vb, g, st);
    if (dim == 64) return pick_tempo<bf16_t, 64, false>(a, heads, kb, vb, g, st);
  } else {
    if (dim == 128) return pick_tempo<float, 128, false>(a, heads, kb, vb, g, st);
    if (dim == 64) return pick_tempo<float, 64, false>(a, heads, kb, vb, g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvc
