// Nearest-centre assignment (QuantWM, section 4.1: each token goes to its nearest
// centroid) and the k-means centre update (NanoKV, Table 4: two K-means iterations).
//
// bf16 tokens: the nearest centre maximises t_c = x.c - ||c||^2 / 2, which is
// -1/2 times ||c||^2 - 2 x.c (||x - c||^2 less the token's own norm).  The scores
// of a 32-centre by 32-token tile come from v_mfma_f32_32x32x16_bf16 (products of
// bf16 values are exact in fp32; the accumulator starts at -||c||^2 / 2, an exact
// halving, and the token fragment is the raw token, so every intermediate is
// exactly -1/2 of the one for ||c||^2 - 2 x.c and so is its rounding error).  Each
// lane keeps the best score, its index and the second-best score.  When the top-2
// gap is not larger than a bound on the fp32 rounding error of the scores, the
// token is re-scored exactly: fp64 sums of (x_i - c_i)^2 over all centres, ties to
// the lowest index.  fp32 tokens always take that fp64 path.
#include "kvc_internal.h"
#include "dev_common.h"
#include "mfma.h"

namespace kvc {
namespace {

// acc + lo^2 + hi^2 for the two bf16 values of a word (v_dot2_f32_bf16: the
// products are exact in fp32)
__device__ __forceinline__ float sq2_bf16(uint32_t w, float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 v = __builtin_bit_cast(b2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
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


template <int D>
__global__ __launch_bounds__(256) void assign_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ cent,
                                                          int C, int64_t n, uint8_t* __restrict__ ids) {
  constexpr int ROWP = D + 8;          // padded LDS row (bf16 elements): conflict-free fragment reads
  constexpr int KC = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sC[256 * ROWP];
  __shared__ __attribute__((aligned(16))) float sN[256];
  __shared__ __attribute__((aligned(16))) uint16_t sX[4][D];   // a flagged token's row, per wavefront

  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = tid / 64;
  const int half = lane / 32;
  const int col = lane % 32;
  const int nblk = (C + 31) / 32;
  const int rows = nblk * 32;
  const bf16_t* centh = cent + int64_t(h) * C * D;

  // the centre table into LDS: all of a thread's loads are issued before the
  // first store (a fixed, unrolled trip count), so their latencies overlap
  {
    constexpr int PER_T = 256 * (D / 8) / 256;
    uint4 w[PER_T];
#pragma unroll
    for (int it = 0; it < PER_T; ++it) {
      const int e = tid + it * 256;
      const int row = e / (D / 8);
      const int c8 = e % (D / 8);
      w[it] = make_uint4(0, 0, 0, 0);
      if (row < C) w[it] = *reinterpret_cast<const uint4*>(centh + int64_t(row) * D + c8 * 8);
    }
#pragma unroll
    for (int it = 0; it < PER_T; ++it) {
      const int e = tid + it * 256;
      const int row = e / (D / 8);
      const int c8 = e % (D / 8);
      if (row < rows) *reinterpret_cast<uint4*>(&sC[row * ROWP + c8 * 8]) = w[it];
    }
  }
  __syncthreads();
  // -||c||^2 / 2 with ||c||^2 in fp32, channel pairs in order (v_dot2_f32_bf16);
  // padding rows score -inf
  {
    float sn = -INFINITY;
    if (tid < C) {
      sn = 0.f;
#pragma unroll
      for (int c8 = 0; c8 < D / 8; ++c8) {
        const uint4 w = *reinterpret_cast<const uint4*>(&sC[tid * ROWP + c8 * 8]);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sn = sq2_bf16(ww[i], sn);
        }
      }
      sn *= -0.5f;
    }
    if (tid < rows) sN[tid] = sn;
  }
  __syncthreads();
  float cmax = 0.f;                    // max ||c||^2
  for (int c = lane; c < C; c += 64) cmax = fmaxf(cmax, -2.f * sN[c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, 64));

  for (int round = 0; round < kAssignRounds; ++round) {
  // token fragments (B operand) and ||x||^2
  const int64_t tok0 = (int64_t(blockIdx.x) * kAssignRounds + round) * 256 + wave * 64;
  if (tok0 >= n) break;                // wave-uniform; no barrier follows
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
        s = sq2_bf16(ww[i], s);
      }
      xb[cb][kc] = as_bf16x8(w);
    }
    xx[cb] = s + __shfl_xor(s, 32, 64);
  }

  // best and second-best score per token; the index of the best is kept without
  // this lane's row offset 4*half (a wave-uniform code, added after the scan)
  float b1[2] = {-INFINITY, -INFINITY}, b2[2] = {-INFINITY, -INFINITY};
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
    // strictly greater: on equal scores the earlier (lower) centre stays; the
    // second best is the median of (best, second, new)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int code = blk * 32 + 8 * (v / 4) + (v % 4);
      {
        const float sc = acc0[v];
        const bool gt = sc > b1[0];
        b2[0] = __builtin_amdgcn_fmed3f(b1[0], b2[0], sc);
        b1[0] = gt ? sc : b1[0];
        i1[0] = gt ? code : i1[0];
      }
      {
        const float sc = acc1[v];
        const bool gt = sc > b1[1];
        b2[1] = __builtin_amdgcn_fmed3f(b1[1], b2[1], sc);
        b1[1] = gt ? sc : b1[1];
        i1[1] = gt ? code : i1[1];
      }
    }
  }
  i1[0] += 4 * half;
  i1[1] += 4 * half;

  // Bound on the difference of the rounding errors of two scores.  A score sums
  // D exact products and -n_c/2 in fp32 (in any order: at most D roundings), and
  // n_c = ||c||^2 itself comes from at most D roundings, so
  // |err(t_c)| <= g (n_c + ||x|| sqrt(n_c)) with g = D 2^-24 (1 + 2^-16), using
  // |x.c| <= ||x|| ||c||; a gap of two scores is then off by at most
  // 2 g (cmax + ||x|| sqrt(cmax)), below (2D + 4) 2^-24 (cmax + ||x|| sqrt(cmax)).
  const float err_scale = float(2 * D + 4) * 5.9604645e-08f;   // (2D + 4) * 2^-24
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float ob1 = __shfl_xor(b1[cb], 32, 64);
    const float ob2 = __shfl_xor(b2[cb], 32, 64);
    const int oi1 = __shfl_xor(i1[cb], 32, 64);
    const float nb2 = fmaxf(fminf(b1[cb], ob1), fmaxf(b2[cb], ob2));
    const bool other = ob1 > b1[cb] || (ob1 == b1[cb] && oi1 < i1[cb]);
    const float nb1 = other ? ob1 : b1[cb];
    int id = other ? oi1 : i1[cb];
    const int64_t tok = tok0 + cb * 32 + col;
    const bool valid = tok < n;
    const float thr = err_scale * (cmax + sqrtf(xx[cb] * cmax));
    const bool flag = valid && half == 0 && !(nb1 - nb2 > thr);  // also catches NaN
    uint64_t mask = __ballot(flag);
    if (mask) {
      // The true nearest centre of a flagged token is among the centres whose
      // computed score is within thr of the best one.  Those candidates are found
      // by scoring this token half once more, then re-scored exactly (fp64,
      // dimensions spread over the lanes, a fixed reduction order), ties to the
      // lowest index.
      const float lim = nb1 - thr;
      uint32_t cm[8];                 // candidate bits of block blk: 16 per lane
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) cm[blk] = 0;
      // two blocks at a time (two independent accumulation chains); the second of
      // a pair past the last block reads rows of the 256-row table that are never
      // used and is discarded
#pragma unroll
      for (int bp = 0; bp < 4; ++bp) {
        if (2 * bp >= nblk) break;
        f32x16 acc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4 t = *reinterpret_cast<const float4*>(&sN[(2 * bp + u) * 32 + 8 * g4 + 4 * half]);
            acc[u][4 * g4 + 0] = t.x; acc[u][4 * g4 + 1] = t.y; acc[u][4 * g4 + 2] = t.z; acc[u][4 * g4 + 3] = t.w;
          }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 a = as_bf16x8(
                *reinterpret_cast<const uint4*>(&sC[((2 * bp + u) * 32 + col) * ROWP + kc * 16 + half * 8]));
            acc[u] = mfma32(a, xb[cb][kc], acc[u]);
          }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t bits = 0;
#pragma unroll
          for (int v = 0; v < 16; ++v) bits |= (acc[u][v] >= lim ? 1u : 0u) << v;
          if (2 * bp + u < nblk) cm[2 * bp + u] = bits;
        }
      }
      constexpr int PERL = D / 64;    // dimensions per lane in the exact re-scoring
      while (mask) {
        const int b = __builtin_ctzll(mask);
        mask &= mask - 1;
        const int64_t t = tok0 + cb * 32 + b;
        const bf16_t* xr = x + (int64_t(h) * n + t) * D;
        // the token's row from the two lanes that hold it (fragments of 8
        // dimensions), through this wavefront's LDS row (LDS operations of one
        // wavefront complete in order)
        if (col == b) {
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            *reinterpret_cast<uint4*>(&sX[wave][kc * 16 + half * 8]) = as_uint4(xb[cb][kc]);
        }
        double xd[PERL];
#pragma unroll
        for (int i = 0; i < PERL; ++i) xd[i] = double(__uint_as_float(uint32_t(sX[wave][lane * PERL + i]) << 16));
        double best = INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
          if (blk >= nblk) break;
          const uint32_t w0 = __builtin_amdgcn_readlane(cm[blk], b);
          const uint32_t w1 = __builtin_amdgcn_readlane(cm[blk], b + 32);
          uint32_t both = w0 | (w1 << 16);   // bit v: row 8*(v/4) + v%4 (+4 for the high half)
          while (both) {
            const int bit = __builtin_ctz(both);
            both &= both - 1;
            const int v = bit & 15, hh = bit >> 4;
            const int ci = blk * 32 + 8 * (v / 4) + 4 * hh + (v % 4);
            double part = 0.0;
#pragma unroll
            for (int i = 0; i < PERL; ++i) {
              const double cv = double(__uint_as_float(uint32_t(sC[ci * ROWP + lane * PERL + i]) << 16));
              const double dlt = xd[i] - cv;
              part = __dadd_rn(part, __dmul_rn(dlt, dlt));
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) part = __dadd_rn(part, __shfl_xor(part, o, 64));
            if (part < best || (part == best && ci < bi)) { best = part; bi = ci; }
          }
        }
        int e = bi;
        if (bi == 0x7fffffff)           // no candidate (non-finite scores): score every centre exactly
          e = exact_assign_token<bf16_t, D>(xr, centh, C, lane);
        if (lane == b) id = e;
      }
    }
    if (valid && half == 0) ids[int64_t(h) * n + tok] = static_cast<uint8_t>(id);
  }
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

// One wavefront per (head, centre): the members' rows are added in fp64 in token
// order.  The head's ids pass through LDS in chunks of kScanChunk tokens, shared
// by the workgroup's four wavefronts; each wavefront finds its centre's members 64
// ids at a time (a ballot; slots in token order by mbcnt), lists up to 64 of them
// in LDS and then adds their rows in that order with BATCH row loads in flight.
// The order of the additions is fixed, so the result is deterministic; the centre
// becomes the mean (one fp64 division) rounded to nearest even in the storage
// type, and a centre without members keeps its value.
template <typename T, int D>
__global__ __launch_bounds__(256) void kmeans_update_kernel(const T* __restrict__ x, T* __restrict__ cent,
                                                            const uint8_t* __restrict__ ids, int C, int64_t n) {
  constexpr int PER = D / 64;                 // channels per lane
  constexpr int WPR = PER * int(sizeof(T)) / 4 > 0 ? PER * int(sizeof(T)) / 4 : 1;   // 32-bit words per lane and row
  constexpr int BATCH = 64 / WPR < 64 ? 64 / WPR : 64;   // rows in flight (64 registers of raw words)
  __shared__ __attribute__((aligned(16))) uint8_t sid[kScanChunk];
  __shared__ int slist[4][256];
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int c = blockIdx.x * 4 + wave;
  const int h = blockIdx.y;
  const bool active = c < C;                  // wave-uniform; every wavefront takes the barriers
  const uint8_t* idh = ids + int64_t(h) * n;
  const T* xh = x + int64_t(h) * n * D + lane * PER;
  double acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0;
  int64_t cnt = 0;
  int nl = 0;                                 // members listed, not yet added
  // lane's channels of a row
  auto load_raw = [&](const T* row, uint32_t (&w)[WPR]) {
    if constexpr (sizeof(T) == 2 && PER == 1) w[0] = reinterpret_cast<const uint16_t*>(row)[0];
    else {
#pragma unroll
      for (int q = 0; q < WPR; ++q) w[q] = reinterpret_cast<const uint32_t*>(row)[q];
    }
  };
  auto value = [&](const uint32_t (&w)[WPR], int i) -> float {
    if constexpr (sizeof(T) == 2) {
      if constexpr (PER == 1) return __uint_as_float(w[0] << 16);
      else return (i & 1) ? bf16_hi(w[i / 2]) : bf16_lo(w[i / 2]);
    } else {
      return __uint_as_float(w[i]);
    }
  };
  auto flush = [&]() {                        // add the listed rows, in list order
    for (int u0 = 0; u0 < nl; u0 += BATCH) {
      uint32_t w[BATCH][WPR];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int j = slist[wave][u0 + u < nl ? u0 + u : nl - 1];
        load_raw(xh + int64_t(j) * D, w[u]);
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (u0 + u < nl) {
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] = __dadd_rn(acc[i], double(value(w[u], i)));
        }
    }
    nl = 0;
  };
  for (int64_t c0 = 0; c0 < n; c0 += kScanChunk) {
    const int len = int(n - c0 < kScanChunk ? n - c0 : kScanChunk);
    __syncthreads();                          // the previous chunk is scanned
    if (((reinterpret_cast<uintptr_t>(idh + c0)) & 3) == 0) {
      const int len4 = len / 4;
      for (int i = threadIdx.x; i < len4; i += 256)
        reinterpret_cast<uint32_t*>(sid)[i] = reinterpret_cast<const uint32_t*>(idh + c0)[i];
      for (int i = 4 * len4 + threadIdx.x; i < len; i += 256) sid[i] = idh[c0 + i];
    } else {
      for (int i = threadIdx.x; i < len; i += 256) sid[i] = idh[c0 + i];
    }
    __syncthreads();
    if (active) {
      // Windows of 256 ids, four ids (one 32-bit word) per lane, lane l holding
      // ids 4l..4l+3; four windows read at once, then taken in token order.  A
      // byte equal to c is flagged exactly: with x = word ^ (c in every byte),
      // ((x & 0x7f..) + 0x7f..) | x has its top bit clear only in zero bytes
      // (no carry crosses a byte).  Flags past the end of the chunk are dropped.
      const uint32_t cc = uint32_t(c) * 0x01010101u;
      auto rank_of = [](uint64_t m) {
        return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
      };
      for (int p0 = 0; p0 < len; p0 += 1024) {
        uint32_t wv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int p = p0 + 256 * k + 4 * lane;
          wv[k] = p < len ? reinterpret_cast<const uint32_t*>(sid)[p >> 2] : 0u;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int p = p0 + 256 * k + 4 * lane;
          const uint32_t x = wv[k] ^ cc;
          uint32_t z = ~(((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;
          const int rem = len - p;
          if (rem < 4) z &= rem <= 0 ? 0u : (0x80808080u >> (8 * (4 - rem)));
          if (__ballot(z != 0u)) {
            // members of this window: lane prefix of the per-lane counts (0..4)
            // from three ballots of the count's bits
            const int k1 = __popc(z);
            const uint64_t b0 = __ballot(k1 & 1), b1 = __ballot(k1 & 2), b2 = __ballot(k1 & 4);
            const int tot = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
            if (nl + tot > 64) flush();
            int pos = nl + rank_of(b0) + 2 * rank_of(b1) + 4 * rank_of(b2);
            for (uint32_t zz = z; zz != 0u; zz &= zz - 1u) slist[wave][pos++] = int(c0 + p + (__builtin_ctz(zz) >> 3));
            nl += tot;
            cnt += tot;
          }
        }
      }
    }
  }
  if (!active) return;
  flush();
  if (cnt == 0) return;                       // empty cluster keeps its centre
  T* dst = cent + (int64_t(h) * C + c) * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const double mean = __ddiv_rn(acc[i], double(cnt));
    if constexpr (sizeof(T) == 2)
      reinterpret_cast<uint16_t*>(dst)[i] = static_cast<uint16_t>(f64_to_bits_rne<8>(mean));
    else
      reinterpret_cast<uint32_t*>(dst)[i] = f64_to_bits_rne<24>(mean);
  }
}

}  // namespace

hipError_t launch_assign(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, const void* cent,
                         uint8_t* ids, hipStream_t st) {
  if (heads == 0 || n == 0) return hipSuccess;
  if (dt == KVC_BF16) {
    const dim3 grid(unsigned((n + 256 * kAssignRounds - 1) / (256 * kAssignRounds)), unsigned(heads));
    if (dim == 128)
      hipLaunchKernelGGL((assign_mfma_kernel<128>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(cent), C, n, ids);
    else if (dim == 64)
      hipLaunchKernelGGL((assign_mfma_kernel<64>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(cent), C, n, ids);
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

template <typename T, int D>
hipError_t run_kmeans_update(int heads, int64_t n, const void* x, int C, void* cent, const uint8_t* ids,
                             hipStream_t st) {
  hipLaunchKernelGGL((kmeans_update_kernel<T, D>), dim3(unsigned((C + 3) / 4), unsigned(heads)), dim3(256), 0, st,
                     static_cast<const T*>(x), static_cast<T*>(cent), ids, C, n);
  return hipGetLastError();
}

size_t kmeans_update_workspace(int heads, int64_t n, int C) {
  (void)heads;
  (void)n;
  (void)C;
  return 256;                                 // reserved; the update keeps its lists in LDS
}

hipError_t launch_kmeans_update(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, void* cent,
                                const uint8_t* ids, void* ws, hipStream_t st) {
  (void)ws;
  if (heads == 0 || n == 0) return hipSuccess;
  if (n >= (int64_t(1) << 31)) return hipErrorInvalidValue;   // token indices are 32-bit in the lists
  if (dt == KVC_BF16 && dim == 128) return run_kmeans_update<bf16_t, 128>(heads, n, x, C, cent, ids, st);
  if (dt == KVC_BF16 && dim == 64) return run_kmeans_update<bf16_t, 64>(heads, n, x, C, cent, ids, st);
  if (dt == KVC_F32 && dim == 128) return run_kmeans_update<float, 128>(heads, n, x, C, cent, ids, st);
  if (dt == KVC_F32 && dim == 64) return run_kmeans_update<float, 64>(heads, n, x, C, cent, ids, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
