// Nearest-centre assignment (QuantWM, section 4.1: each token goes to its nearest
// centroid) and the k-means centre update (NanoKV, Table 4: two K-means iterations).
//
// bf16 tokens: the scores s_c = ||c||^2 - 2 x.c of a 32-centre by 32-token tile
// come from v_mfma_f32_32x32x16_bf16 (products of bf16 values are exact in fp32;
// the accumulator starts at ||c||^2 and the token fragment is pre-scaled by -2,
// which is exact).  Each lane keeps the best score, its index and the second-best
// score.  When the top-2 gap is not larger than a bound on the fp32 rounding error
// of the scores, the token is re-scored exactly: fp64 sums of (x_i - c_i)^2 over
// all centres, ties to the lowest index.  fp32 tokens always take that fp64 path.
#include "kvc_internal.h"
#include "dev_common.h"
#include "mfma.h"

namespace kvc {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void centroid_norms_kernel(const T* __restrict__ cent, int64_t total,
                                                             float* __restrict__ norms) {
  const int64_t item = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= total) return;
  float s = 0.f;
#pragma unroll
  for (int c8 = 0; c8 < D / 8; ++c8) {
    float v[8];
    load_row<8>(cent + item * D + c8 * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(v[i], v[i], s);
  }
  norms[item] = s;
}

// Exact fp64 squared distance between a token row (global) and a centre row.
template <typename T, int D>
__device__ __forceinline__ double exact_dist(const T* __restrict__ xr, const T* __restrict__ cr) {
  double d = 0.0;
#pragma unroll 4
  for (int c8 = 0; c8 < D / 8; ++c8) {
    float xv[8], cv[8];
    load_row<8>(xr + c8 * 8, xv);
    load_row<8>(cr + c8 * 8, cv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double t = double(xv[i]) - double(cv[i]);
      d = __dadd_rn(d, __dmul_rn(t, t));
    }
  }
  return d;
}

// Wave-wide argmin of (dist, index) with ties to the lower index.
__device__ __forceinline__ void wave_argmin(double& best, int& bi) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double od = __shfl_xor(best, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (od < best || (od == best && oi < bi)) { best = od; bi = oi; }
  }
}

// Exact assignment of one token by the whole wave (lanes take centres lane, lane+64, ...).
template <typename T, int D>
__device__ __forceinline__ int exact_assign_token(const T* __restrict__ xr, const T* __restrict__ centh, int C,
                                                  int lane) {
  double best = INFINITY;
  int bi = 0x7fffffff;
  for (int c = lane; c < C; c += 64) {
    const double d = exact_dist<T, D>(xr, centh + int64_t(c) * D);
    if (d < best) { best = d; bi = c; }
  }
  wave_argmin(best, bi);
  return bi;
}

// fp32 tokens: every token assigned exactly; one wave per token.
template <typename T, int D>
__global__ __launch_bounds__(256) void assign_exact_kernel(const T* __restrict__ x, const T* __restrict__ cent,
                                                           int C, int64_t n, uint8_t* __restrict__ ids) {
  const int lane = threadIdx.x % 64;
  const int64_t j = int64_t(blockIdx.x) * 4 + threadIdx.x / 64;
  const int h = blockIdx.y;
  if (j >= n) return;
  const int bi = exact_assign_token<T, D>(x + (int64_t(h) * n + j) * D, cent + int64_t(h) * C * D, C, lane);
  if (lane == 0) ids[int64_t(h) * n + j] = static_cast<uint8_t>(bi);
}

__device__ __forceinline__ uint32_t scale_m2_bf16x2(uint32_t w) {
  // multiply both bf16 halves by -2 (exact for finite values away from the range limits)
  return pack_bf16x2(-2.f * bf16_lo(w), -2.f * bf16_hi(w));
}

template <int D>
__global__ __launch_bounds__(256) void assign_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ cent,
                                                          const float* __restrict__ norms, int C, int64_t n,
                                                          uint8_t* __restrict__ ids) {
  constexpr int ROWP = D + 8;          // padded LDS row (bf16 elements): conflict-free fragment reads
  constexpr int KC = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sC[256 * ROWP];
  __shared__ __attribute__((aligned(16))) float sN[256];

  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = tid / 64;
  const int half = lane / 32;
  const int col = lane % 32;
  const int nblk = (C + 31) / 32;
  const int rows = nblk * 32;
  const bf16_t* centh = cent + int64_t(h) * C * D;

  for (int e = tid; e < rows * (D / 8); e += 256) {
    const int row = e / (D / 8);
    const int c8 = e % (D / 8);
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row < C) w = *reinterpret_cast<const uint4*>(centh + int64_t(row) * D + c8 * 8);
    *reinterpret_cast<uint4*>(&sC[row * ROWP + c8 * 8]) = w;
  }
  for (int c = tid; c < rows; c += 256) sN[c] = c < C ? norms[int64_t(h) * C + c] : INFINITY;
  float cmax = 0.f;
  for (int c = lane; c < C; c += 64) cmax = fmaxf(cmax, norms[int64_t(h) * C + c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, 64));

  // token fragments (B operand), pre-scaled by -2, and ||x||^2
  const int64_t tok0 = int64_t(blockIdx.x) * 256 + wave * 64;
  bf16x8 xb[2][KC];
  float xx[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int64_t tok = tok0 + cb * 32 + col;
    const bool valid = tok < n;
    float s = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (valid) w = *reinterpret_cast<const uint4*>(x + (int64_t(h) * n + tok) * D + kc * 16 + half * 8);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = fmaf(bf16_lo(ww[i]), bf16_lo(ww[i]), s);
        s = fmaf(bf16_hi(ww[i]), bf16_hi(ww[i]), s);
      }
      xb[cb][kc] = as_bf16x8(make_uint4(scale_m2_bf16x2(w.x), scale_m2_bf16x2(w.y), scale_m2_bf16x2(w.z),
                                        scale_m2_bf16x2(w.w)));
    }
    xx[cb] = s + __shfl_xor(s, 32, 64);
  }
  __syncthreads();

  float b1[2] = {INFINITY, INFINITY}, b2[2] = {INFINITY, INFINITY};
  int i1[2] = {0, 0};
  for (int blk = 0; blk < nblk; ++blk) {
    f32x16 nc;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 t = *reinterpret_cast<const float4*>(&sN[blk * 32 + 8 * g4 + 4 * half]);
      nc[4 * g4 + 0] = t.x; nc[4 * g4 + 1] = t.y; nc[4 * g4 + 2] = t.z; nc[4 * g4 + 3] = t.w;
    }
    f32x16 acc0 = nc, acc1 = nc;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&sC[(blk * 32 + col) * ROWP + kc * 16 + half * 8]));
      acc0 = mfma32(a, xb[0][kc], acc0);
      acc1 = mfma32(a, xb[1][kc], acc1);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int cidx = blk * 32 + 8 * (v / 4) + 4 * half + (v % 4);
      {
        const float s = acc0[v];
        const bool lt = s < b1[0];
        b2[0] = fminf(b2[0], fmaxf(b1[0], s));
        b1[0] = lt ? s : b1[0];
        i1[0] = lt ? cidx : i1[0];
      }
      {
        const float s = acc1[v];
        const bool lt = s < b1[1];
        b2[1] = fminf(b2[1], fmaxf(b1[1], s));
        b1[1] = lt ? s : b1[1];
        i1[1] = lt ? cidx : i1[1];
      }
    }
  }

  const float err_scale = float(4 * D + 8) * 5.9604645e-08f;  // (4D + 8) * 2^-24
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float ob1 = __shfl_xor(b1[cb], 32, 64);
    const float ob2 = __shfl_xor(b2[cb], 32, 64);
    const int oi1 = __shfl_xor(i1[cb], 32, 64);
    const float nb2 = fminf(fmaxf(b1[cb], ob1), fminf(b2[cb], ob2));
    const bool other = ob1 < b1[cb] || (ob1 == b1[cb] && oi1 < i1[cb]);
    const float nb1 = other ? ob1 : b1[cb];
    int id = other ? oi1 : i1[cb];
    const int64_t tok = tok0 + cb * 32 + col;
    const bool valid = tok < n;
    const float thr = err_scale * (xx[cb] + 2.f * cmax);
    const bool flag = valid && half == 0 && !(nb2 - nb1 > thr);  // also catches NaN
    uint64_t mask = __ballot(flag);
    while (mask) {
      const int b = __builtin_ctzll(mask);
      mask &= mask - 1;
      const int64_t t = tok0 + cb * 32 + b;
      const int e = exact_assign_token<bf16_t, D>(x + (int64_t(h) * n + t) * D, centh, C, lane);
      if (lane == b) id = e;
    }
    if (valid && half == 0) ids[int64_t(h) * n + tok] = static_cast<uint8_t>(id);
  }
}

// ------------------------------------------------------------------------------ k-means update
// Round an fp64 value to the binary format with P significand bits and an 8-bit
// exponent (bf16: P = 8, fp32: P = 24), nearest-even, with gradual underflow.
// Returns the bit pattern (in the low 16 or 32 bits).  Written from the IEEE-754
// definition of the formats.
template <int P>
__device__ __forceinline__ uint32_t f64_to_bits_rne(double d) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(d));
  const uint32_t sign = uint32_t(u >> 63);
  const uint64_t a = u & 0x7fffffffffffffffull;
  constexpr int SIGN_SHIFT = P + 7;           // bf16: 15, fp32: 31
  constexpr int QMIN = -125 - P;              // quantum of the subnormals: 2^-133 / 2^-149
  if (a == 0) return sign << SIGN_SHIFT;
  const int e = int(a >> 52) - 1023;          // value = m * 2^(e - 52), m in [2^52, 2^53)
  if (e < -1022) return sign << SIGN_SHIFT;   // fp64 subnormal: rounds to zero in the target
  const uint64_t m = (a & 0x000fffffffffffffull) | 0x0010000000000000ull;
  const int qe = max(e - (P - 1), QMIN);
  const int sh = qe - (e - 52);               // >= 53 - P
  uint64_t R;
  if (sh >= 64) {
    R = 0;                                     // far below half a quantum
  } else {
    R = m >> sh;
    const uint64_t rem = m & ((uint64_t(1) << sh) - 1);
    const uint64_t halfq = uint64_t(1) << (sh - 1);
    if (rem > halfq || (rem == halfq && (R & 1))) R += 1;
  }
  const uint32_t bits = (R < (uint64_t(1) << (P - 1))) ? uint32_t(R)
                                                       : (uint32_t(qe - QMIN) << (P - 1)) + uint32_t(R);
  return (sign << SIGN_SHIFT) | bits;
}

// One wavefront per (head, CPW consecutive centres).  The ids are scanned in
// chunks of 1024 tokens (16 consecutive tokens per lane); the members of the
// wave's centres are listed in token order in LDS through a prefix sum over the
// lanes, then their rows are added in fp64, eight row loads in flight at a time.
// The order of the additions is fixed, so the result is deterministic; each
// centre becomes the mean (one fp64 division) rounded to nearest even in the
// storage type, and a centre without members keeps its value.
template <typename T, int D, int CPW>
__global__ __launch_bounds__(256) void kmeans_update_kernel(const T* __restrict__ x, T* __restrict__ cent,
                                                            const uint8_t* __restrict__ ids, int C, int64_t n) {
  constexpr int PER = D / 64;                 // channels per lane
  constexpr int BATCH = 8;
  static_assert(CPW <= 16, "centre offsets are stored in 4 bits");
  __shared__ uint32_t s_list[4][1024];        // per wave: (token in chunk << 4) | centre offset
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int c0 = (blockIdx.x * 4 + wave) * CPW;
  const int h = blockIdx.y;
  if (c0 >= C) return;                        // wave-uniform; the kernel has no block barrier
  const uint8_t* idh = ids + int64_t(h) * n;
  const T* xh = x + int64_t(h) * n * D;
  double acc[CPW][PER];
  int cnt[CPW];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    cnt[k] = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[k][i] = 0.0;
  }
  uint32_t* list = s_list[wave];
  for (int64_t j0 = 0; j0 < n; j0 += 1024) {
    uint32_t m = 0;                           // members among this lane's 16 tokens
    uint64_t sel = 0;                         // their centre offsets, 4 bits each
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int64_t j = j0 + 16 * lane + k;
      const int d = j < n ? int(idh[j]) - c0 : -1;
      if (d >= 0 && d < CPW) {
        m |= 1u << k;
        sel |= uint64_t(d) << (4 * k);
      }
    }
    // exclusive prefix of the member counts over the lanes (token order is lane-major)
    const int own = __popc(m);
    int pre = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(pre, off, 64);
      if (lane >= off) pre += t;
    }
    const int total = __shfl(pre, 63, 64);
    int pos = pre - own;
    uint32_t mm = m;
    while (mm) {
      const int k = __builtin_ctz(mm);
      mm &= mm - 1;
      list[pos++] = (uint32_t(16 * lane + k) << 4) | uint32_t((sel >> (4 * k)) & 15u);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int b0 = 0; b0 < total; b0 += BATCH) {
      uint32_t e[BATCH];
      float v[BATCH][PER];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        e[u] = __builtin_amdgcn_readfirstlane(b0 + u < total ? list[b0 + u] : 0u);
        const T* row = xh + (j0 + (e[u] >> 4)) * D;
        if (b0 + u < total) {
#pragma unroll
          for (int i = 0; i < PER; ++i) {
            if constexpr (sizeof(T) == 2)
              v[u][i] = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(row)[lane * PER + i]) << 16);
            else
              v[u][i] = reinterpret_cast<const float*>(row)[lane * PER + i];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        if (b0 + u < total) {
          const int ci = int(e[u] & 15u);
#pragma unroll
          for (int k = 0; k < CPW; ++k) {
            if (k == ci) {
              ++cnt[k];
#pragma unroll
              for (int i = 0; i < PER; ++i) acc[k][i] = __dadd_rn(acc[k][i], double(v[u][i]));
            }
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();          // the list is rewritten by the next chunk
  }
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    const int c = c0 + k;
    if (c >= C || cnt[k] == 0) continue;      // empty cluster keeps its centre
    T* dst = cent + (int64_t(h) * C + c) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const double mean = __ddiv_rn(acc[k][i], double(cnt[k]));
      if constexpr (sizeof(T) == 2)
        reinterpret_cast<uint16_t*>(dst)[lane * PER + i] = static_cast<uint16_t>(f64_to_bits_rne<8>(mean));
      else
        reinterpret_cast<uint32_t*>(dst)[lane * PER + i] = f64_to_bits_rne<24>(mean);
    }
  }
}

}  // namespace

hipError_t launch_centroid_norms(int heads, int C, int dim, kvc_dtype dt, const void* cent, float* norms,
                                 hipStream_t st) {
  const int64_t total = int64_t(heads) * C;
  if (total == 0) return hipSuccess;
  const unsigned blocks = unsigned((total + 255) / 256);
  if (dt == KVC_BF16 && dim == 128)
    hipLaunchKernelGGL((centroid_norms_kernel<bf16_t, 128>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const bf16_t*>(cent), total, norms);
  else if (dt == KVC_BF16 && dim == 64)
    hipLaunchKernelGGL((centroid_norms_kernel<bf16_t, 64>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const bf16_t*>(cent), total, norms);
  else if (dt == KVC_F32 && dim == 128)
    hipLaunchKernelGGL((centroid_norms_kernel<float, 128>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(cent), total, norms);
  else if (dt == KVC_F32 && dim == 64)
    hipLaunchKernelGGL((centroid_norms_kernel<float, 64>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(cent), total, norms);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_assign(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, const void* cent,
                         const float* norms, uint8_t* ids, hipStream_t st) {
  if (heads == 0 || n == 0) return hipSuccess;
  if (dt == KVC_BF16) {
    const dim3 grid(unsigned((n + 255) / 256), unsigned(heads));
    if (dim == 128)
      hipLaunchKernelGGL((assign_mfma_kernel<128>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(cent), norms, C, n, ids);
    else if (dim == 64)
      hipLaunchKernelGGL((assign_mfma_kernel<64>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(cent), norms, C, n, ids);
    else
      return hipErrorInvalidValue;
  } else {
    const dim3 grid(unsigned((n + 3) / 4), unsigned(heads));
    if (dim == 128)
      hipLaunchKernelGGL((assign_exact_kernel<float, 128>), grid, dim3(256), 0, st, static_cast<const float*>(x),
                         static_cast<const float*>(cent), C, n, ids);
    else if (dim == 64)
      hipLaunchKernelGGL((assign_exact_kernel<float, 64>), grid, dim3(256), 0, st, static_cast<const float*>(x),
                         static_cast<const float*>(cent), C, n, ids);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D, int CPW>
hipError_t run_kmeans_update(int heads, int64_t n, const void* x, int C, void* cent, const uint8_t* ids,
                             hipStream_t st) {
  const dim3 grid(unsigned((C + 4 * CPW - 1) / (4 * CPW)), unsigned(heads));
  hipLaunchKernelGGL((kmeans_update_kernel<T, D, CPW>), grid, dim3(256), 0, st, static_cast<const T*>(x),
                     static_cast<T*>(cent), ids, C, n);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t pick_cpw(int heads, int64_t n, const void* x, int C, void* cent, const uint8_t* ids, hipStream_t st) {
  // one centre per wavefront while that gives at most ~16k wavefronts; beyond
  // that, eight centres share a wavefront and its scan of the ids
  if (int64_t(heads) * C <= 16384) return run_kmeans_update<T, D, 1>(heads, n, x, C, cent, ids, st);
  return run_kmeans_update<T, D, 8>(heads, n, x, C, cent, ids, st);
}

hipError_t launch_kmeans_update(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, void* cent,
                                const uint8_t* ids, hipStream_t st) {
  if (heads == 0 || n == 0) return hipSuccess;
  if (dt == KVC_BF16 && dim == 128) return pick_cpw<bf16_t, 128>(heads, n, x, C, cent, ids, st);
  if (dt == KVC_BF16 && dim == 64) return pick_cpw<bf16_t, 64>(heads, n, x, C, cent, ids, st);
  if (dt == KVC_F32 && dim == 128) return pick_cpw<float, 128>(heads, n, x, C, cent, ids, st);
  if (dt == KVC_F32 && dim == 64) return pick_cpw<float, 64>(heads, n, x, C, cent, ids, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
