// Principal-subspace logit compensation of the remaining key error (PSAC;
// QuantWM, section 4.2, Eqs. 13-17): the queries' second-moment matrix
// M = E[q q^T], its top-r eigenvectors U_r (the principal query subspace), and the
// kept coefficients C = (K - K_hat_0) U_r of each key's quantization error.  The
// attention kernel adds (U_r^T q) . c to every logit (attend.hip).
#include "kvc_internal.h"
#include "dev_common.h"
#include "mfma.h"

namespace kvc {
namespace {

// M <- (n_prev * M + sum_i q_i q_i^T) / (n_prev + n_q) for one 32 x 32 tile of
// one head (fp32 queries): 256 threads, thread t owns row 32*bi + t/8 and columns 32*bj +
// 4*(t%8) .. +3; the queries pass through LDS 64 rows at a time, and each output
// sums over the queries in increasing order (fp32 multiply-adds).
template <typename T, int D>
__global__ __launch_bounds__(256) void query_moments_kernel(const T* __restrict__ q, int64_t n_q, int64_t n_prev,
                                                            float* __restrict__ m) {
  constexpr int NT = D / 32;
  __shared__ float sa[64][33], sb[64][33];
  const int h = blockIdx.y;
  const int bi = blockIdx.x / NT, bj = blockIdx.x % NT;
  const int t = threadIdx.x;
  const int row = t / 8, c0 = 4 * (t % 8);
  const T* qh = q + int64_t(h) * n_q * D;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i0 = 0; i0 < n_q; i0 += 64) {
    __syncthreads();
    // 64 rows x 32 channels of each block: 2048 values, 8 per thread
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e = t + 256 * k;
      const int r = e / 32, c = e % 32;
      const int64_t qi = i0 + r;
      float a = 0.f, b = 0.f;
      if (qi < n_q) {
        const T* rowp = qh + qi * D;
        if constexpr (sizeof(T) == 2) {
          a = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(rowp)[bi * 32 + c]) << 16);
          b = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(rowp)[bj * 32 + c]) << 16);
        } else {
          a = reinterpret_cast<const float*>(rowp)[bi * 32 + c];
          b = reinterpret_cast<const float*>(rowp)[bj * 32 + c];
        }
      }
      sa[r][c] = a;
      sb[r][c] = b;
    }
    __syncthreads();
    const int nr = n_q - i0 < 64 ? int(n_q - i0) : 64;
    for (int r = 0; r < nr; ++r) {
      const float a = sa[r][row];
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(a, sb[r][c0 + k], acc[k]);
    }
  }
  float* mh = m + int64_t(h) * D * D;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float* dst = mh + int64_t(bi * 32 + row) * D + bj * 32 + c0 + k;
    double tot = double(acc[k]);
    if (n_prev > 0) tot += double(*dst) * double(n_prev);
    *dst = float(tot / double(n_prev + n_q));
  }
}

// bf16 queries: the 32 x 32 tile (bi, bj) of sum_i q_i q_i^T on the matrix cores:
// A = Q^T rows (channels 32*bi ..), B = Q columns (channels 32*bj ..), the
// contraction over 16 queries per v_mfma_f32_32x32x16_bf16 (products of bf16
// values are exact in fp32).  Eight wavefronts per tile, each walking its own
// blocks of 64 queries (block w, w + 8, ...) through its own LDS rows (32
// channels, 64 B, so the transposing reads of 4 rows hit distinct banks) with no
// barrier in the loop; the operands come from ds_read_b64_tr_b16, A and B in the
// same query order.  The eight partial tiles are added in wavefront order.
typedef short mom_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) mom_s16x4 mom_lds_s16x4;
__device__ __forceinline__ uint2 mom_read_tr16(const uint16_t* p) {
  const mom_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((mom_lds_s16x4*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, v);
}

template <int D>
__global__ __launch_bounds__(512) void query_moments_mfma_kernel(const bf16_t* __restrict__ q, int64_t n_q,
                                                                 int64_t n_prev, float* __restrict__ m) {
  constexpr int NT = D / 32;
  constexpr int W = 8;                         // wavefronts per tile
  __shared__ __attribute__((aligned(16))) uint16_t sa[W][64 * 32], sb[W][64 * 32];
  __shared__ float red[W][16][64];             // partial tiles, [wave][v][lane]
  const int h = blockIdx.y;
  const int bi = blockIdx.x / NT, bj = blockIdx.x % NT;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint16_t* qh = reinterpret_cast<const uint16_t*>(q) + int64_t(h) * n_q * D;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  // transposing reads: lane s supplies query row 4*(s >> 5) + ((s >> 2) & 3) (+8
  // for the second read, +16*kk per product) and channels 16*((s >> 4) & 1) +
  // 4*(s & 3) .. +3; lane l receives channel l % 32 of its 4 queries
  const int trow = 4 * (lane >> 5) + ((lane >> 2) & 3);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  for (int64_t i0 = int64_t(w) * 64; i0 < n_q; i0 += W * 64) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {              // 64 rows x 4 chunks of 8 channels
      const int e = lane + 64 * k;
      const int r = e / 4, c8 = (e % 4) * 8;
      uint4 wa = make_uint4(0, 0, 0, 0), wb = make_uint4(0, 0, 0, 0);
      if (i0 + r < n_q) {
        wa = *reinterpret_cast<const uint4*>(qh + (i0 + r) * D + bi * 32 + c8);
        wb = *reinterpret_cast<const uint4*>(qh + (i0 + r) * D + bj * 32 + c8);
      }
      *reinterpret_cast<uint4*>(&sa[w][r * 32 + c8]) = wa;
      *reinterpret_cast<uint4*>(&sb[w][r * 32 + c8]) = wb;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {           // 16 queries per product
      const uint16_t* pa = &sa[w][(kk * 16 + trow) * 32 + tcol];
      const uint16_t* pb = &sb[w][(kk * 16 + trow) * 32 + tcol];
      const uint2 alo = mom_read_tr16(pa), ahi = mom_read_tr16(pa + 8 * 32);
      const uint2 blo = mom_read_tr16(pb), bhi = mom_read_tr16(pb + 8 * 32);
      acc = mfma32(as_bf16x8(make_uint4(alo.x, alo.y, ahi.x, ahi.y)),
                   as_bf16x8(make_uint4(blo.x, blo.y, bhi.x, bhi.y)), acc);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) red[w][v][lane] = acc[v];
  __syncthreads();
  if (w != 0) return;
  // lane: column j = lane % 32, rows i = 8*(v/4) + 4*(lane/32) + v%4
  float* mh = m + int64_t(h) * D * D;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    double tot = 0.0;
#pragma unroll
    for (int u = 0; u < W; ++u) tot += double(red[u][v][lane]);
    const int i = bi * 32 + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
    const int j = bj * 32 + lane % 32;
    float* dst = mh + int64_t(i) * D + j;
    if (n_prev > 0) tot += double(*dst) * double(n_prev);
    *dst = float(tot / double(n_prev + n_q));
  }
}

// Eigen-decomposition of the symmetric R x R matrix a (row-major, overwritten)
// by cyclic Jacobi rotations; eigenvectors in the columns of v.  One thread; the
// index loops are unrolled so that a and v stay in registers.
template <int R>
__device__ void jacobi_eig(float (&a)[R][R], float (&v)[R][R]) {
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) v[i][j] = i == j ? 1.f : 0.f;
  for (int sweep = 0; sweep < 30; ++sweep) {
    float off = 0.f, diag = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      diag += a[i][i] * a[i][i];
#pragma unroll
      for (int j = i + 1; j < R; ++j) off += a[i][j] * a[i][j];
    }
    if (off <= 1e-14f * diag) break;          // off-diagonal at fp32 rounding level
#pragma unroll
    for (int p = 0; p < R; ++p)
#pragma unroll
      for (int qq = p + 1; qq < R; ++qq) {
        if (a[p][qq] == 0.f) continue;
        // rotation that zeroes a[p][qq] (the standard symmetric Schur step)
        const float theta = 0.5f * (a[qq][qq] - a[p][p]) / a[p][qq];
        const float tt = (theta >= 0.f ? 1.f : -1.f) / (fabsf(theta) + sqrtf(theta * theta + 1.f));
        const float c = 1.f / sqrtf(tt * tt + 1.f), s = tt * c;
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const float akp = a[k][p], akq = a[k][qq];
          a[k][p] = c * akp - s * akq;
          a[k][qq] = s * akp + c * akq;
        }
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const float apk = a[p][k], aqk = a[qq][k];
          a[p][k] = c * apk - s * aqk;
          a[qq][k] = s * apk + c * aqk;
        }
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const float vkp = v[k][p], vkq = v[k][qq];
          v[k][p] = c * vkp - s * vkq;
          v[k][qq] = s * vkp + c * vkq;
        }
      }
  }
}

// Sum of a float over the 64 lanes, the same in every lane, in a fixed order:
// neighbours (DPP quad permutations), the other half of each group of 8 and of
// each row of 16 (DPP mirrors), then across rows and halves (permlane swaps).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);     // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);     // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);    // row_half_mirror
  v += dpp_f32<0x140>(v);    // row_mirror
  {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Top-R eigenvectors of one head's M by subspace iteration: V <- orth(M V),
// n_iter times (modified Gram-Schmidt by one wavefront), then Rayleigh-Ritz:
// the R x R matrix V^T M V is diagonalized and V rotated onto its eigenvectors,
// largest eigenvalue first; each column's largest component is made positive.
// The start is u_prev (warm) or a fixed dense pattern.
template <int D, int R>
__global__ __launch_bounds__(256) void psac_basis_kernel(const float* __restrict__ m, int n_iter,
                                                         const float* __restrict__ u_prev, float* __restrict__ u,
                                                         float* __restrict__ lam) {
  __shared__ float sm[D][D + 1];
  __shared__ __attribute__((aligned(16))) float sv[D][R], sw[D][R];
  __shared__ float st[R][R];
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  const float* mh = m + int64_t(h) * D * D;
  {                                           // M into LDS: all loads issued first
    constexpr int PER = D * D / 4 / 256;
    float4 w[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) w[k] = reinterpret_cast<const float4*>(mh)[t + 256 * k];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = 4 * (t + 256 * k);
      sm[e / D][e % D] = w[k].x; sm[e / D][e % D + 1] = w[k].y;
      sm[e / D][e % D + 2] = w[k].z; sm[e / D][e % D + 3] = w[k].w;
    }
  }
  for (int e = t; e < D * R; e += 256) {
    const int i = e / R, k = e % R;
    sv[i][k] = u_prev ? u_prev[int64_t(h) * D * R + e]
                      : __sinf(0.37f * float(i + 1) * float(k + 1) + 0.11f * float(k)) + (i == k ? 1.f : 0.f);
  }
  __syncthreads();
  auto multiply = [&]() {                     // sw = M sv: a thread per (row, 4 columns)
    static_assert(R == 8 && D * 2 <= 256, "two threads per row");
    if (t < 2 * D) {
      const int i = t >> 1, k0 = (t & 1) * 4;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      for (int j = 0; j < D; ++j) {
        const float mij = sm[i][j];
        const float4 vj = *reinterpret_cast<const float4*>(&sv[j][k0]);
        a0 = fmaf(mij, vj.x, a0); a1 = fmaf(mij, vj.y, a1);
        a2 = fmaf(mij, vj.z, a2); a3 = fmaf(mij, vj.w, a3);
      }
      *reinterpret_cast<float4*>(&sw[i][k0]) = make_float4(a0, a1, a2, a3);
    }
    __syncthreads();
  };
  auto orthonormalize = [&]() {               // sv = columns of sw, Gram-Schmidt (wave 0)
    if (t < 64) {
      for (int k = 0; k < R; ++k) {
        for (int j = 0; j < k; ++j) {
          float d = 0.f;
          for (int i = t; i < D; i += 64) d += sv[i][j] * sw[i][k];
          d = wave_sum_f32(d);
          for (int i = t; i < D; i += 64) sw[i][k] -= d * sv[i][j];
        }
        float nn = 0.f;
        for (int i = t; i < D; i += 64) nn += sw[i][k] * sw[i][k];
        nn = wave_sum_f32(nn);
        const float inv = nn > 0.f ? 1.f / sqrtf(nn) : 0.f;
        for (int i = t; i < D; i += 64) sv[i][k] = sw[i][k] * inv;
      }
    }
    __syncthreads();
  };
  // orthonormal start
  for (int e = t; e < D * R; e += 256) sw[e / R][e % R] = sv[e / R][e % R];
  __syncthreads();
  orthonormalize();
  for (int it = 0; it < n_iter; ++it) {
    multiply();
    orthonormalize();
  }
  // Rayleigh-Ritz
  multiply();
  if (t < R * R) {
    const int a = t / R, b = t % R;
    float acc = 0.f;
    for (int i = 0; i < D; ++i) acc = fmaf(sv[i][a], sw[i][b], acc);
    st[a][b] = acc;
  }
  __syncthreads();
  __shared__ float sy[R][R], sy0[R][R], sdiag[R];
  if (t == 0) {                                // static indices only: a and y stay in registers
    float a[R][R], y[R][R];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < R; ++j) a[i][j] = 0.5f * (st[i][j] + st[j][i]);
    jacobi_eig<R>(a, y);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      sdiag[i] = a[i][i];
#pragma unroll
      for (int j = 0; j < R; ++j) sy0[j][i] = y[j][i];
    }
  }
  __syncthreads();
  if (t < R) {                                 // by eigenvalue, largest first (ties: lower index first)
    const float ev = sdiag[t];
    int rank = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) rank += (sdiag[j] > ev || (sdiag[j] == ev && j < t)) ? 1 : 0;
    lam[int64_t(h) * R + rank] = ev;
#pragma unroll
    for (int j = 0; j < R; ++j) sy[j][rank] = sy0[j][t];
  }
  __syncthreads();
  for (int e = t; e < D * R; e += 256) {       // U = V Y
    const int i = e / R, k = e % R;
    float acc = 0.f;
    for (int j = 0; j < R; ++j) acc = fmaf(sv[i][j], sy[j][k], acc);
    sw[i][k] = acc;
  }
  __syncthreads();
  if (t < R) {                                 // sign: the largest component positive
    int arg = 0;
    float best = -1.f;
    for (int i = 0; i < D; ++i)
      if (fabsf(sw[i][t]) > best) { best = fabsf(sw[i][t]); arg = i; }
    const float sg = sw[arg][t] < 0.f ? -1.f : 1.f;
    for (int i = 0; i < D; ++i) u[int64_t(h) * D * R + i * R + t] = sg * sw[i][t];
  }
}

// C = (x - x_hat_0) U_r per token: x_hat_0 = c[id] + q*s + z (fp32), the error's
// coefficients summed over the channels in increasing order, stored as fp16.
// One thread per token; U_r of the head in LDS.
template <typename T, int D, int G, int BITS>
__global__ __launch_bounds__(256) void psac_coeffs_kernel(const T* __restrict__ x, const T* __restrict__ cent,
                                                          const uint8_t* __restrict__ ids,
                                                          const uint8_t* __restrict__ codes,
                                                          const uint32_t* __restrict__ meta, int C, int64_t n,
                                                          const float* __restrict__ u, uint16_t* __restrict__ coef) {
  constexpr int R = kPsacRank;
  __shared__ float su[D][R];
  const int h = blockIdx.y;
  for (int e = threadIdx.x; e < D * R; e += 256) su[e / R][e % R] = u[int64_t(h) * D * R + e];
  __syncthreads();
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j >= n) return;
  const int64_t tok = int64_t(h) * n + j;
  const int id = ids[tok];
  const T* xr = x + tok * D;
  const T* cr = cent + (int64_t(h) * C + id) * D;
  const uint8_t* qr = codes + tok * (D * BITS / 8);
  const uint32_t* mr = meta + tok * (D / G);
  float acc[R];
#pragma unroll
  for (int k = 0; k < R; ++k) acc[k] = 0.f;
  for (int g = 0; g < D / G; ++g) {
    const uint32_t mw = mr[g];
    const float s = f16_bits_to_f32(mw & 0xffffu), z = f16_bits_to_f32(mw >> 16);
    for (int i = 0; i < G; i += 8) {
      float xv[8], cv[8];
      load_row<8>(xr + g * G + i, xv);
      load_row<8>(cr + g * G + i, cv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = g * G + i + e;
        const uint32_t qv = (uint32_t(qr[(c * BITS) / 8]) >> ((c * BITS) % 8)) & ((1u << BITS) - 1u);
        const float xh = cv[e] + fmaf(float(qv), s, z);
        const float err = xv[e] - xh;
#pragma unroll
        for (int k = 0; k < R; ++k) acc[k] = fmaf(err, su[c][k], acc[k]);
      }
    }
  }
  uint32_t w[R / 2];
#pragma unroll
  for (int k = 0; k < R / 2; ++k) w[k] = pack_f16x2(acc[2 * k], acc[2 * k + 1]);
  *reinterpret_cast<uint4*>(coef + tok * R) = make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename T, int D>
hipError_t coeffs_bits(int heads, int64_t n, const void* x, const void* cent, const uint8_t* ids,
                       const uint8_t* codes, const uint16_t* meta, int C, int bits, int group, const float* u,
                       uint16_t* coef, hipStream_t st) {
  const dim3 grid(unsigned((n + 255) / 256), unsigned(heads));
#define KVC_COEF(G_, B_)                                                                                        \
  if (group == G_ && bits == B_) {                                                                              \
    hipLaunchKernelGGL((psac_coeffs_kernel<T, D, G_, B_>), grid, dim3(256), 0, st, static_cast<const T*>(x),    \
                       static_cast<const T*>(cent), ids, codes, reinterpret_cast<const uint32_t*>(meta), C, n, u, \
                       coef);                                                                                   \
    return hipGetLastError();                                                                                   \
  }
  KVC_COEF(16, 2) KVC_COEF(16, 4) KVC_COEF(32, 2) KVC_COEF(32, 4)
#undef KVC_COEF
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_query_moments(int heads, int64_t n_q, int dim, kvc_dtype dt, const void* q, int64_t n_prev,
                                float* m, hipStream_t st) {
  if (heads == 0 || n_q == 0) return hipSuccess;
  const int nt = dim / 32;
  const dim3 grid(unsigned(nt * nt), unsigned(heads));
#define KVC_MOM(T, D) \
  hipLaunchKernelGGL((query_moments_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(q), n_q, n_prev, m)
  if (dt == KVC_BF16) {
    if (dim == 128)
      hipLaunchKernelGGL((query_moments_mfma_kernel<128>), grid, dim3(512), 0, st, static_cast<const bf16_t*>(q), n_q,
                         n_prev, m);
    else
      hipLaunchKernelGGL((query_moments_mfma_kernel<64>), grid, dim3(512), 0, st, static_cast<const bf16_t*>(q), n_q,
                         n_prev, m);
  } else {
    if (dim == 128) KVC_MOM(float, 128); else KVC_MOM(float, 64);
  }
#undef KVC_MOM
  return hipGetLastError();
}

hipError_t launch_psac_basis(int heads, int dim, const float* m, int n_iter, const float* u_prev, float* u,
                             float* lam, hipStream_t st) {
  if (heads == 0) return hipSuccess;
  if (dim == 128)
    hipLaunchKernelGGL((psac_basis_kernel<128, kPsacRank>), dim3(unsigned(heads)), dim3(256), 0, st, m, n_iter,
                       u_prev, u, lam);
  else
    hipLaunchKernelGGL((psac_basis_kernel<64, kPsacRank>), dim3(unsigned(heads)), dim3(256), 0, st, m, n_iter,
                       u_prev, u, lam);
  return hipGetLastError();
}

hipError_t launch_psac_coeffs(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, const void* cent,
                              const uint8_t* ids, const uint8_t* codes, const uint16_t* meta, int bits, int group,
                              const float* u, uint16_t* coef, hipStream_t st) {
  if (heads == 0 || n == 0) return hipSuccess;
  if (dt == KVC_BF16 && dim == 128) return coeffs_bits<bf16_t, 128>(heads, n, x, cent, ids, codes, meta, C, bits, group, u, coef, st);
  if (dt == KVC_BF16 && dim == 64) return coeffs_bits<bf16_t, 64>(heads, n, x, cent, ids, codes, meta, C, bits, group, u, coef, st);
  if (dt == KVC_F32 && dim == 128) return coeffs_bits<float, 128>(heads, n, x, cent, ids, codes, meta, C, bits, group, u, coef, st);
  if (dt == KVC_F32 && dim == 64) return coeffs_bits<float, 64>(heads, n, x, cent, ids, codes, meta, C, bits, group, u, coef, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
