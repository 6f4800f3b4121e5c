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
// token is re-scored exactly: fp64 sums of (x_i - c_i)^2 over the centres whose
// score lies within the bound of the best, ties to the lowest index.  fp32 tokens
// always take an fp64 path over all centres.
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

// max(a, b) as one v_max_f32: a key (a score with index bits in its low mantissa
// bits) is built by integer operations, and fmaxf would first canonicalize it as
// a possible signalling NaN, one more instruction per score.  NaN keys need no
// care: a token with a non-finite value fails the gap test through its bound.
__device__ __forceinline__ float key_max(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
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
  // no finite distance (a token with a NaN or an infinite value): the lowest
  // index, as the first minimum of an all-NaN or all-infinite row
  return bi == 0x7fffffff ? 0 : bi;
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


constexpr int kFlagCap = 128;          // flagged tokens a wavefront holds before resolving them

// A workgroup stages its head's centre table once and then scores `rounds`
// consecutive blocks of 256 tokens against it (the launch picks the number of
// rounds so that the table staging is amortized while the grid still fills the
// chip).
template <int D>
__global__ __launch_bounds__(256, 2) void assign_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ cent,
                                                          int C, int64_t n, int rounds, uint8_t* __restrict__ ids) {
  constexpr int ROWP = D + 8;          // padded LDS row (bf16 elements): conflict-free fragment reads
  constexpr int KC = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sC[256 * ROWP];
  __shared__ __attribute__((aligned(16))) float sN[256];
  __shared__ int sFt[4][kFlagCap];     // per wavefront: flagged tokens waiting for the exact pass
  __shared__ float sFl[4][kFlagCap];   // and their candidate limits (best score - bound)

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
  // padding rows score -FLT_MAX (finite: their keys, with index bits in the low
  // mantissa bits, must not turn into NaNs as -inf would)
  {
    float sn = -3.40282347e+38f;
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

  // The flagged-token pass: tokens whose top-2 gap is within the rounding bound
  // wait in a per-wavefront LDS list; when the list could not take another
  // round's tokens, and after the last round, they are resolved 32 at a time: one
  // more scoring pass over all centres (the same products, so the same fp32
  // scores) marks each token's candidates, and every lane pair re-scores its
  // token's candidates in fp64 (each lane over its 64 dimensions, the two halves
  // added in a fixed order), ties to the lowest index.
  auto flush = [&](int nfl) {
    for (int base = 0; base < nfl; base += 32) {
      const int k = base + col;
      const bool has = k < nfl;
      const int64_t t = sFt[wave][has ? k : base];
      const float lim = has ? sFl[wave][k] : __builtin_nanf("");   // no candidates for idle lanes
      bf16x8 xf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        xf[kc] = as_bf16x8(*reinterpret_cast<const uint4*>(x + (int64_t(h) * n + t) * D + kc * 16 + half * 8));
      uint32_t cm[8];                 // candidate bits of block blk: 16 per lane (this lane's rows)
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
            const float4 tt = *reinterpret_cast<const float4*>(&sN[(2 * bp + u) * 32 + 8 * g4 + 4 * half]);
            acc[u][4 * g4 + 0] = tt.x; acc[u][4 * g4 + 1] = tt.y; acc[u][4 * g4 + 2] = tt.z; acc[u][4 * g4 + 3] = tt.w;
          }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 a = as_bf16x8(
                *reinterpret_cast<const uint4*>(&sC[((2 * bp + u) * 32 + col) * ROWP + kc * 16 + half * 8]));
            acc[u] = mfma32(a, xf[kc], acc[u]);
          }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t bits = 0;
#pragma unroll
          for (int v = 0; v < 16; ++v) bits |= (acc[u][v] >= lim ? 1u : 0u) << v;
          if (2 * bp + u < nblk) cm[2 * bp + u] = bits;
        }
      }
      // both lanes of a pair walk the union of their candidates in the same order
      // (bit v of the low half: row 8*(v/4) + v%4, of the high half: the same + 4),
      // so they run the loop in step and can exchange partial sums
      double best = INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        if (blk >= nblk) break;
        const uint32_t other = __shfl_xor(cm[blk], 32, 64);
        uint32_t both = half ? (other | (cm[blk] << 16)) : (cm[blk] | (other << 16));
        while (both) {
          const int bit = __builtin_ctz(both);
          both &= both - 1;
          const int v = bit & 15, hh = bit >> 4;
          const int ci = blk * 32 + 8 * (v / 4) + 4 * hh + (v % 4);
          double part = 0.0;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            const uint4 cw = *reinterpret_cast<const uint4*>(&sC[ci * ROWP + kc * 16 + half * 8]);
            const uint4 xw = as_uint4(xf[kc]);
            const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w}, ca[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const double d0 = double(bf16_lo(xa[i])) - double(bf16_lo(ca[i]));
              const double d1 = double(bf16_hi(xa[i])) - double(bf16_hi(ca[i]));
              part = __dadd_rn(part, __dmul_rn(d0, d0));
              part = __dadd_rn(part, __dmul_rn(d1, d1));
            }
          }
          const double opart = __shfl_xor(part, 32, 64);
          const double full = half ? __dadd_rn(opart, part) : __dadd_rn(part, opart);
          if (full < best || (full == best && ci < bi)) { best = full; bi = ci; }
        }
      }
      // no finite candidate (a token with a non-finite value): score every centre
      // exactly, the whole wavefront per token
      uint64_t lost = __ballot(has && half == 0 && bi == 0x7fffffff);
      while (lost) {
        const int b = __builtin_ctzll(lost);
        lost &= lost - 1;
        const int64_t tb = sFt[wave][base + b];
        const int e = exact_assign_token<bf16_t, D>(x + (int64_t(h) * n + tb) * D, centh, C, lane);
        if (lane == b) bi = e;       // 0 when no distance is finite
      }
      if (has && half == 0) ids[int64_t(h) * n + t] = static_cast<uint8_t>(bi);
    }
  };

  int nfl = 0;                         // tokens in this wavefront's list (wave-uniform)
  for (int round = 0;; ++round) {
  const int64_t tok0 = (int64_t(blockIdx.x) * rounds + round) * 256 + wave * 64;
  const bool more = round < rounds && tok0 < n;   // wave-uniform; no barrier follows
  if (more) {
  // token fragments (B operand) and ||x||^2
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

  // Best and second-best score per token half.  A score is tracked as a key: its
  // low 4 bits replaced by 15 - v, where v (0..15) is its register within the
  // block, so that one maximum keeps both the best key and where it sits; the
  // second best is the median of (best, second, new).  A key is within 15 ulp of
  // its score (below 2^-19 of it), which the bound below takes into account.  The
  // block of the best is recorded whenever a block raises it.
  float b1[2] = {-INFINITY, -INFINITY}, b2[2] = {-INFINITY, -INFINITY};
  int blk1[2] = {0, 0};
  // Software pipeline over the 32-centre blocks: the products of block blk + 1
  // (into the other of two accumulator sets) are issued between the scan steps
  // of block blk, so that the matrix cores and the vector unit work at the same
  // time within a wavefront.
  uint4 af[KC];
  f32x16 nc;
  auto read_block = [&](int blk) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      af[kc] = *reinterpret_cast<const uint4*>(&sC[(blk * 32 + col) * ROWP + kc * 16 + half * 8]);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 t = *reinterpret_cast<const float4*>(&sN[blk * 32 + 8 * g4 + 4 * half]);
      nc[4 * g4 + 0] = t.x; nc[4 * g4 + 1] = t.y; nc[4 * g4 + 2] = t.z; nc[4 * g4 + 3] = t.w;
    }
  };
  auto scan_v = [&](const f32x16& c0, const f32x16& c1, int v) {
    const float k0 = __uint_as_float((__float_as_uint(c0[v]) & ~15u) | uint32_t(15 - v));
    const float k1 = __uint_as_float((__float_as_uint(c1[v]) & ~15u) | uint32_t(15 - v));
    b2[0] = __builtin_amdgcn_fmed3f(b1[0], b2[0], k0);
    b1[0] = key_max(b1[0], k0);
    b2[1] = __builtin_amdgcn_fmed3f(b1[1], b2[1], k1);
    b1[1] = key_max(b1[1], k1);
  };
  // scan block blk (accumulators cur) and, when there is one, multiply block
  // blk + 1 into nxt
  auto step = [&](int blk, const f32x16& cur0, const f32x16& cur1, f32x16& nxt0, f32x16& nxt1, bool has_next) {
    const float p0 = b1[0], p1 = b1[1];
    if (has_next) {                    // wave-uniform
      read_block(blk + 1);
      nxt0 = nc;
      nxt1 = nc;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        scan_v(cur0, cur1, (2 * kc) % 16);
        nxt0 = mfma32(as_bf16x8(af[kc]), xb[0][kc], nxt0);
        scan_v(cur0, cur1, (2 * kc + 1) % 16);
        nxt1 = mfma32(as_bf16x8(af[kc]), xb[1][kc], nxt1);
      }
      if constexpr (KC < 8) {
#pragma unroll
        for (int v = 2 * KC; v < 16; ++v) scan_v(cur0, cur1, v);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) scan_v(cur0, cur1, v);
    }
    blk1[0] = b1[0] != p0 ? blk : blk1[0];
    blk1[1] = b1[1] != p1 ? blk : blk1[1];
  };
  f32x16 cA0, cA1, cB0, cB1;
  read_block(0);
  cA0 = nc;
  cA1 = nc;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    cA0 = mfma32(as_bf16x8(af[kc]), xb[0][kc], cA0);
    cA1 = mfma32(as_bf16x8(af[kc]), xb[1][kc], cA1);
  }
  for (int blk = 0; blk < nblk; blk += 2) {
    step(blk, cA0, cA1, cB0, cB1, blk + 1 < nblk);
    if (blk + 1 >= nblk) break;
    step(blk + 1, cB0, cB1, cA0, cA1, blk + 2 < nblk);
  }
  int i1[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int v = 15 - int(__float_as_uint(b1[cb]) & 15u);
    i1[cb] = blk1[cb] * 32 + 8 * (v / 4) + 4 * half + (v % 4);
  }

  // Bound on the difference of the rounding errors of two scores.  A score sums
  // D exact products and -n_c/2 in fp32 (in any order: at most D roundings), and
  // n_c = ||c||^2 itself comes from at most D roundings, so
  // |err(t_c)| <= g (n_c + ||x|| sqrt(n_c)) with g = D 2^-24 (1 + 2^-16), using
  // |x.c| <= ||x|| ||c||; a gap of two scores is then off by at most
  // 2 g (cmax + ||x|| sqrt(cmax)), below (2D + 4) 2^-24 (cmax + ||x|| sqrt(cmax)).
  // A key differs from its score by less than 2^-19 |t_c| <= 2^-19 (cmax/2 +
  // ||x|| sqrt(cmax)), so a gap of two keys adds at most 2^-18 (cmax + ||x||
  // sqrt(cmax)) = 64 * 2^-24 (...): a token whose key gap exceeds the sum has its
  // best score more than the score bound above the second, and its best key is
  // its best score.  The candidate limit (best key - bound) stays below the best
  // score minus the score bound.
  const float err_scale = float(2 * D + 68) * 5.9604645e-08f;   // (2D + 68) * 2^-24
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
    if (valid && half == 0 && !flag) ids[int64_t(h) * n + tok] = static_cast<uint8_t>(id);
    const uint64_t mask = __ballot(flag);
    if (mask) {
      const int slot = nfl + int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u)));
      if (flag) {
        sFt[wave][slot] = int(tok);
        sFl[wave][slot] = nb1 - thr;
      }
      nfl += __popcll(mask);
    }
  }
  }
  // the list holds at most kFlagCap tokens and a round adds at most 64
  if (nfl > kFlagCap - 64 || (!more && nfl > 0)) {
    __builtin_amdgcn_wave_barrier();   // the list's LDS writes precede its reads (one wavefront: in order)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    flush(nfl);
    nfl = 0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  if (!more) break;
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

// Centre update from member lists sorted in LDS.  One workgroup of 8
// wavefronts per (head, group of CG consecutive centres); the head's ids (at
// most kSortedUpdateMaxTokens) are staged in LDS once.
//   1. count: wavefront w takes the w-th eighth of the tokens and counts, per
//      centre of the group, its members (the lanes of one 64-token step that hold
//      the same centre are found with one ballot per bit of the centre's index;
//      the last of them adds the count, so no atomics are needed);
//   2. prefix: start[u] = members of the group's centres before u; every
//      wavefront's write offset per centre follows in wavefront order;
//   3. scatter: the same walk writes each member's token index at its offset
//      plus its rank among the step's lanes of that centre -- a stable counting
//      sort, so every centre's members end up in token order;
//   4. sums: the sorted list is cut into eight equal runs, one per wavefront,
//      whose rows are loaded BATCH at a time and added in fp64 in list order;
//      a centre whose members all lie in the run gets its mean written at once,
//      a centre cut by a run boundary leaves a partial sum (at most two per
//      wavefront);
//   5. the partial sums are added in run order and those centres written.
// Every addition happens in a fixed order, so the result is deterministic; a
// centre's sum is its members' rows in token order, grouped by run.  The mean is
// one fp64 division rounded to nearest even in the storage type; a centre without
// members keeps its value.
//
// With GL (global lists), steps 1-3 are skipped: the member lists and the
// centres' list starts of the whole head come from member_lists_kernel (in the
// caller's workspace), so no workgroup scans the head's ids.
template <typename T, int D, bool GL>
__global__ __launch_bounds__(512) void kmeans_update_sorted_kernel(const T* __restrict__ x, T* __restrict__ cent,
                                                                   const uint8_t* __restrict__ ids, int C, int CG,
                                                                   int n, const uint32_t* __restrict__ glists,
                                                                   const uint32_t* __restrict__ gstarts) {
  constexpr int PER = D / 64;                 // channels per lane
  constexpr int WPR = PER * int(sizeof(T)) / 4 > 0 ? PER * int(sizeof(T)) / 4 : 1;   // 32-bit words per lane and row
  constexpr int BATCH = 32;                   // rows in flight per wavefront
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int c0 = blockIdx.x * CG;
  const int cg = min(CG, C - c0);
  const int npad = GL ? 0 : (n + 15) & ~15;                  // staged ids
  const int lpad = GL ? 0 : (2 * n + 15) & ~15;              // the group's list (uint16 token indices)
  uint8_t* sid = lds;
  uint16_t* list = reinterpret_cast<uint16_t*>(lds + npad);
  uint32_t* off = reinterpret_cast<uint32_t*>(lds + npad + lpad);                      // [8][CG]
  uint32_t* start = off + 8 * CG;                                                       // [CG + 1]
  int* pc = reinterpret_cast<int*>(start + CG + 1);                                     // [16] centre of a partial
  uint32_t* wsum = reinterpret_cast<uint32_t*>(pc + 16);                                // [8]
  double* part = reinterpret_cast<double*>(
      lds + ((npad + lpad + 4 * (8 * CG + CG + 1 + 16 + 8) + 15) & ~15));   // [16][D]
  // global lists: the group's segment of the head's list
  const uint32_t* glist = nullptr;
  if constexpr (GL) {
    const uint32_t* st = gstarts + int64_t(h) * (C + 1) + c0;
    const uint32_t base = st[0];
    glist = glists + int64_t(h) * n + base;
    for (int t = threadIdx.x; t <= cg; t += 512) start[t] = st[t] - base;
    if (threadIdx.x < 16) pc[threadIdx.x] = -1;
    __syncthreads();
  }
  auto list_at = [&](int i) -> int {
    if constexpr (GL) return int(glist[i]);
    else return int(list[i]);
  };

  const uint8_t* idh = ids + int64_t(h) * n;
  if constexpr (!GL) {
  if ((reinterpret_cast<uintptr_t>(idh) & 3) == 0) {
    const int n4 = n / 4;
    for (int i = threadIdx.x; i < n4; i += 512) reinterpret_cast<uint32_t*>(sid)[i] = reinterpret_cast<const uint32_t*>(idh)[i];
    for (int i = 4 * n4 + threadIdx.x; i < n; i += 512) sid[i] = idh[i];
  } else {
    for (int i = threadIdx.x; i < n; i += 512) sid[i] = idh[i];
  }
  for (int i = threadIdx.x; i < 8 * CG; i += 512) off[i] = 0u;
  if (threadIdx.x < 16) pc[threadIdx.x] = -1;
  __syncthreads();

  auto rank_of = [](uint64_t m) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
  };
  // lanes of this step holding the same centre as this lane (valid for matching lanes)
  auto same_centre = [&](bool m, int u) {
    uint64_t same = __ballot(m);
    for (int b = 0; (1 << b) < CG; ++b) {
      const bool bit = ((u >> b) & 1) != 0;
      const uint64_t bb = __ballot(m && bit);
      same &= bit ? bb : ~bb;
    }
    return same;
  };
  const int s0 = int(int64_t(n) * wave / 8), s1 = int(int64_t(n) * (wave + 1) / 8);
  // 1. counts per (wavefront, centre)
  for (int p0 = s0; p0 < s1; p0 += 64) {
    const int p = p0 + lane;
    const int u = p < s1 ? int(sid[p]) - c0 : -1;
    const bool m = u >= 0 && u < cg;
    const uint64_t same = same_centre(m, u);
    const int cnt = __popcll(same), rk = rank_of(same);
    if (m && rk == cnt - 1) off[wave * CG + u] += uint32_t(cnt);
  }
  __syncthreads();
  // 2. prefix over the group's centres (thread t for centre t < cg <= 256), then
  // the per-wavefront write offsets in wavefront order
  {
    const int t = threadIdx.x;
    uint32_t tot = 0u;
    if (t < cg)
      for (int w = 0; w < 8; ++w) tot += off[w * CG + t];
    uint32_t inc = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t base = 0u;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    const uint32_t excl = base + inc - tot;
    if (t < cg) {
      start[t] = excl;
      uint32_t run = excl;
      for (int w = 0; w < 8; ++w) {
        const uint32_t c = off[w * CG + t];
        off[w * CG + t] = run;
        run += c;
      }
    }
    if (t == cg - 1) start[cg] = excl + tot;
  }
  __syncthreads();
  // 3. stable scatter of the members' token indices
  for (int p0 = s0; p0 < s1; p0 += 64) {
    const int p = p0 + lane;
    const int u = p < s1 ? int(sid[p]) - c0 : -1;
    const bool m = u >= 0 && u < cg;
    const uint64_t same = same_centre(m, u);
    const int cnt = __popcll(same), below = rank_of(same);
    if (m) list[off[wave * CG + u] + below] = static_cast<uint16_t>(p);
    if (m && below == cnt - 1) off[wave * CG + u] += uint32_t(cnt);
  }
  __syncthreads();
  }   // !GL

  // 4. sums over this wavefront's run of the sorted list
  const T* xh = x + int64_t(h) * n * D + lane * PER;
  auto load_raw = [&](int j, uint32_t (&w)[WPR]) {
    const T* row = xh + int64_t(j) * D;
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
  auto write_mean = [&](int u, const double (&acc)[PER]) {
    const double cnt = double(start[u + 1] - start[u]);
    T* dst = cent + (int64_t(h) * C + c0 + u) * D + lane * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const double mean = __ddiv_rn(acc[i], cnt);
      if constexpr (sizeof(T) == 2)
        reinterpret_cast<uint16_t*>(dst)[i] = static_cast<uint16_t>(f64_to_bits_rne<8>(mean));
      else
        reinterpret_cast<uint32_t*>(dst)[i] = f64_to_bits_rne<24>(mean);
    }
  };
  const int M = int(start[cg]);
  const int r0 = int(int64_t(M) * wave / 8), r1 = int(int64_t(M) * (wave + 1) / 8);
  if (r0 < r1) {
    // the centre of list position r0: the largest u with start[u] <= r0
    int u = 0;
    {
      int lo = 0, hi = cg - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (int(start[mid]) <= r0) lo = mid; else hi = mid - 1;
      }
      u = lo;
    }
    int u_begin = int(start[u]), u_end = int(start[u + 1]);
    int seg = 0;
    double acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.0;
    for (int i0 = r0; i0 < r1; i0 += BATCH) {
      uint32_t w[BATCH][WPR];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int j = list_at(i0 + b < r1 ? i0 + b : r1 - 1);
        load_raw(j < n ? j : n - 1, w[b]);   // always in range (the list holds token indices < n)
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int i = i0 + b;
        if (i >= r1) break;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = __dadd_rn(acc[k], double(value(w[b], k)));
        if (i + 1 == u_end || i + 1 == r1) {
          if (u_begin >= r0 && u_end <= r1) {
            write_mean(u, acc);
          } else {
            const int slot = wave * 2 + (seg == 0 ? 0 : 1);
#pragma unroll
            for (int k = 0; k < PER; ++k) part[slot * D + lane * PER + k] = acc[k];
            if (lane == 0) pc[slot] = u;
          }
          ++seg;
#pragma unroll
          for (int k = 0; k < PER; ++k) acc[k] = 0.0;
          if (i + 1 < r1) {             // next centre with members
            ++u;
            while (u + 1 < cg && int(start[u + 1]) == int(start[u])) ++u;
            u_begin = int(start[u]);
            u_end = int(start[u + 1]);
          }
        }
      }
    }
  }
  __syncthreads();
  // 5. centres cut by a run boundary: partial sums added in run order
  if (wave == 0) {
    int cur = -1;
    double acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.0;
    for (int slot = 0; slot < 16; ++slot) {
      const int u = pc[slot];
      if (u < 0) continue;
      if (u != cur) {
        if (cur >= 0) write_mean(cur, acc);
        cur = u;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = part[slot * D + lane * PER + k];
      } else {
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = __dadd_rn(acc[k], part[slot * D + lane * PER + k]);
      }
    }
    if (cur >= 0) write_mean(cur, acc);
  }
}

// Member lists of a whole head for the centre update of long heads: a stable
// counting sort of the head's tokens by centre id, written to the caller's
// workspace as starts[u] (members of the centres before u; starts[C] = n) and
// lists[starts[u] ..] (the token indices of centre u's members).  The head is cut
// into P chunks (cut at multiples of 4) and each chunk into NW wavefront ranges
// (also at multiples of 4); wavefront w walks its range 1024 tokens at a time,
// lane l holding tokens p + 16l .. p + 16l + 15 (four 32-bit loads when the ids
// are 4-byte aligned) and the 16 steps of 64 taking token p + 16l + k in step k.
// Counting and scattering walk in the same order, so the order inside a centre's
// list is fixed (token order within a step, steps in walk order, ranges in
// wavefront order, chunks in token order) and the sums over it deterministic.
//   PHASE 0: P = 1, one workgroup per head counts, takes the prefix and scatters;
//   PHASE 1: workgroup (p, h) counts chunk p: wcnt[h][p][w][u] per wavefront and
//            ctot[h][p][u] over the chunk;
//   PHASE 2: workgroup (p, h) takes the prefix over the centres from ctot (chunk
//            0 writes starts), its wavefronts' offsets from wcnt, and scatters.
template <int NW, int PHASE>
__global__ __launch_bounds__(NW * 64) void member_lists_kernel(const uint8_t* __restrict__ ids, int C, int n, int P,
                                                               uint32_t* __restrict__ lists,
                                                               uint32_t* __restrict__ starts,
                                                               uint32_t* __restrict__ wcnt,
                                                               uint32_t* __restrict__ ctot) {
  static_assert(NW * 64 >= 256, "one thread per centre in the prefix");
  __shared__ uint32_t off[NW][256];
  __shared__ uint32_t wsum[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int p = blockIdx.x;
  const int h = blockIdx.y;
  const uint8_t* idh = ids + int64_t(h) * n;
  uint32_t* lh = lists + int64_t(h) * n;
  auto rank_of = [](uint64_t m) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
  };
  // lanes of this step holding the same centre as this lane (valid for matching lanes)
  auto same_centre = [&](bool m, int u) {
    uint64_t same = __ballot(m);
    for (int b = 0; (1 << b) < C; ++b) {
      const bool bit = ((u >> b) & 1) != 0;
      const uint64_t bb = __ballot(m && bit);
      same &= bit ? bb : ~bb;
    }
    return same;
  };
  const int cs0 = p == 0 ? 0 : int((int64_t(n) * p / P) & ~int64_t(3));
  const int cs1 = p == P - 1 ? n : int((int64_t(n) * (p + 1) / P) & ~int64_t(3));
  const int len = cs1 - cs0;
  const int s0 = cs0 + (wave == 0 ? 0 : int((int64_t(len) * wave / NW) & ~int64_t(3)));
  const int s1 = wave == NW - 1 ? cs1 : cs0 + int((int64_t(len) * (wave + 1) / NW) & ~int64_t(3));
  const bool words = ((reinterpret_cast<uintptr_t>(idh) | uintptr_t(n)) & 3) == 0;   // wave-uniform
  // calls fn(valid, centre, token) for the steps of the walk, in walk order
  auto walk = [&](auto&& fn) {
    for (int p0 = s0; p0 < s1; p0 += 1024) {
      const int q = p0 + 16 * lane;
      uint32_t w[4];
      if (words) {
        // the word holding the last token of the range bounds every read
        const int qmax = (s1 - 1) & ~3;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int a = q + 4 * j < qmax ? q + 4 * j : qmax;
          w[j] = *reinterpret_cast<const uint32_t*>(idh + a);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t v = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pe = q + 4 * j + e;
            v |= uint32_t(idh[pe < s1 ? pe : s1 - 1]) << (8 * e);
          }
          w[j] = v;
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int pk = q + k;
        const int u = int((w[k >> 2] >> (8 * (k & 3))) & 0xffu);
        fn(pk < s1 && u < C, u, pk);     // an id >= C belongs to no centre
      }
    }
  };
  const int t = threadIdx.x;
  const int64_t hp = int64_t(h) * P + p;
  if constexpr (PHASE != 2) {
    // 1. counts per (wavefront, centre)
    for (int i = t; i < NW * 256; i += NW * 64) (&off[0][0])[i] = 0u;
    __syncthreads();
    walk([&](bool m, int u, int) {
      const uint64_t same = same_centre(m, u);
      const int cnt = __popcll(same), rk = rank_of(same);
      if (m && rk == cnt - 1) off[wave][u] += uint32_t(cnt);
    });
    __syncthreads();
    if constexpr (PHASE == 1) {
      if (t < C) {
        uint32_t tot = 0u;
        for (int w = 0; w < NW; ++w) {
          wcnt[(hp * NW + w) * C + t] = off[w][t];
          tot += off[w][t];
        }
        ctot[hp * C + t] = tot;
      }
      return;
    }
  }
  // 2. starts over the centres (thread t for centre t < C <= 256), then every
  // wavefront's write offset per centre: chunks before this one, then
  // wavefronts before this one
  uint32_t tot = 0u, before = 0u;
  if (t < C) {
    if constexpr (PHASE == 0) {
      for (int w = 0; w < NW; ++w) tot += off[w][t];
    } else {
      for (int q = 0; q < P; ++q) {
        const uint32_t c = ctot[(int64_t(h) * P + q) * C + t];
        if (q < p) before += c;
        tot += c;
      }
    }
  }
  uint32_t inc = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  if (lane == 63 && wave < 4) wsum[wave] = inc;
  __syncthreads();
  uint32_t base = 0u;
  for (int w = 0; w < wave && w < 4; ++w) base += wsum[w];
  const uint32_t excl = base + inc - tot;
  if (t < C) {
    if (p == 0) starts[int64_t(h) * (C + 1) + t] = excl;
    uint32_t run = excl + before;
    for (int w = 0; w < NW; ++w) {
      const uint32_t c = PHASE == 0 ? off[w][t] : wcnt[(hp * NW + w) * C + t];
      off[w][t] = run;
      run += c;
    }
  }
  if (p == 0 && t == C - 1) starts[int64_t(h) * (C + 1) + C] = excl + tot;
  __syncthreads();
  // 3. scatter of the token indices, in the order of step 1
  walk([&](bool m, int u, int pk) {
    const uint64_t same = same_centre(m, u);
    const int cnt = __popcll(same), below = rank_of(same);
    const uint32_t o = m ? off[wave][u] : 0u;
    if (m) lh[o + uint32_t(below)] = uint32_t(pk);
    if (m && below == cnt - 1) off[wave][u] = o + uint32_t(cnt);
  });
}

}  // namespace

hipError_t launch_assign(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, const void* cent,
                         uint8_t* ids, hipStream_t st) {
  if (heads == 0 || n == 0) return hipSuccess;
  if (dim != 128 && dim != 64) return hipErrorInvalidValue;
  // the grid's second dimension takes the heads, at most 65535 per launch
  const size_t es = dt == KVC_BF16 ? 2 : 4;
  for (int h0 = 0; h0 < heads; h0 += 65535) {
    const int hc = heads - h0 < 65535 ? heads - h0 : 65535;
    const void* xh = static_cast<const char*>(x) + size_t(h0) * size_t(n) * size_t(dim) * es;
    const void* ch = static_cast<const char*>(cent) + size_t(h0) * size_t(C) * size_t(dim) * es;
    uint8_t* ih = ids + size_t(h0) * size_t(n);
    if (dt == KVC_BF16) {
      // blocks of 256 tokens per head, shared out over enough workgroups per head
      // for about kAssignMinGroups workgroups in all (two fit a compute unit), each
      // taking the same number of consecutive blocks
      const int64_t blocks = (n + 255) / 256;
      const int64_t want = (kAssignMinGroups + hc - 1) / hc;
      const int64_t groups0 = blocks < want ? blocks : want;
      const int rounds = int((blocks + groups0 - 1) / groups0);
      const dim3 grid(unsigned((blocks + rounds - 1) / rounds), unsigned(hc));
      if (dim == 128)
        hipLaunchKernelGGL((assign_mfma_kernel<128>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(xh),
                           static_cast<const bf16_t*>(ch), C, n, rounds, ih);
      else
        hipLaunchKernelGGL((assign_mfma_kernel<64>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(xh),
                           static_cast<const bf16_t*>(ch), C, n, rounds, ih);
    } else {
      const dim3 grid(unsigned((n + 3) / 4), unsigned(hc));
      if (dim == 128)
        hipLaunchKernelGGL((assign_exact_kernel<float, 128>), grid, dim3(256), 0, st, static_cast<const float*>(xh),
                           static_cast<const float*>(ch), C, n, ih);
      else
        hipLaunchKernelGGL((assign_exact_kernel<float, 64>), grid, dim3(256), 0, st, static_cast<const float*>(xh),
                           static_cast<const float*>(ch), C, n, ih);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Heads longer than kSortedUpdateMaxTokens (whose ids do not fit in LDS), and
// heads longer than kGlobalListTokens when there are at most
// kGlobalListMaxHeads of them, have their member lists sorted once per head into
// the workspace (member_lists_kernel) rather than by every workgroup of the head
// in LDS: with few heads the update splits a head over many workgroups, each of
// which would sort the whole head again (12 heads x 32760 tokens: 95 -> 50 us;
// 40 x 32760: 312 -> 138 us; 720 x 4680 stays in LDS, 314 us against 356 us).
// The sort is cut into chunks of at least kListChunkTokens tokens so that about
// kListMinGroups workgroups share it when the heads are few.
bool update_global_lists(int heads, int64_t n) {
  return n > kSortedUpdateMaxTokens || (n > kGlobalListTokens && heads <= kGlobalListMaxHeads);
}

int member_list_chunks(int heads, int64_t n) {
  const int64_t want = (kListMinGroups + heads - 1) / heads;
  const int64_t most = (n + kListChunkTokens - 1) / kListChunkTokens;
  const int64_t P = want < most ? want : most;
  return P < 1 ? 1 : int(P);
}

size_t kmeans_update_workspace(int heads, int64_t n, int C) {
  if (!update_global_lists(heads, n)) return 256;     // reserved; the lists live in LDS
  const int P = member_list_chunks(heads, n);
  const size_t counts = P > 1 ? size_t(heads) * size_t(P) * size_t(kListChunkWaves + 1) * size_t(C) * 4 : 0;
  return size_t(heads) * size_t(n) * 4 + size_t(heads) * size_t(C + 1) * 4 + counts + 256;
}

size_t sorted_update_lds(int64_t n, int CG, int dim, bool gl) {
  const size_t npad = gl ? 0 : (size_t(n) + 15) & ~size_t(15);
  const size_t lpad = gl ? 0 : (2 * size_t(n) + 15) & ~size_t(15);
  return ((npad + lpad + 4 * (8 * size_t(CG) + CG + 1 + 16 + 8) + 15) & ~size_t(15)) + 16 * size_t(dim) * 8;
}

template <typename T, int D>
hipError_t run_kmeans_update_sorted(int heads, int64_t n, const void* x, int C, void* cent, const uint8_t* ids,
                                    void* ws, hipStream_t st) {
  // workgroups per head: enough for about kUpdateMinGroups in all, at most 16
  // (groups of at least 16 centres)
  // (groups of at least 16 centres; with global lists, of at least
  // 256 / kGlobalListMaxSplit, as no workgroup scans the ids)
  const bool gl = update_global_lists(heads, n);
  const int smax = gl ? kGlobalListMaxSplit : 16;
  int S = int((kUpdateMinGroups + heads - 1) / heads);
  S = S < 1 ? 1 : (S > smax ? smax : S);
  const int CG = (C + S - 1) / S;
  uint32_t* glists = nullptr;
  uint32_t* gstarts = nullptr;
  if (gl) {
    glists = static_cast<uint32_t*>(ws);
    gstarts = glists + int64_t(heads) * n;
    const int P = member_list_chunks(heads, n);
    if (P == 1) {     // heads enough to fill the chip: one workgroup of 16 wavefronts per head
      hipLaunchKernelGGL((member_lists_kernel<16, 0>), dim3(1u, unsigned(heads)), dim3(1024), 0, st, ids, C, int(n),
                         1, glists, gstarts, nullptr, nullptr);
    } else {
      uint32_t* wcnt = gstarts + int64_t(heads) * (C + 1);
      uint32_t* ctot = wcnt + int64_t(heads) * P * kListChunkWaves * C;
      const dim3 grid(static_cast<unsigned>(P), static_cast<unsigned>(heads));
      hipLaunchKernelGGL((member_lists_kernel<kListChunkWaves, 1>), grid, dim3(kListChunkWaves * 64), 0, st, ids, C,
                         int(n), P, glists, gstarts, wcnt, ctot);
      hipLaunchKernelGGL((member_lists_kernel<kListChunkWaves, 2>), grid, dim3(kListChunkWaves * 64), 0, st, ids, C,
                         int(n), P, glists, gstarts, wcnt, ctot);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t lds = sorted_update_lds(n, CG, D, gl);
  const void* fn = gl ? reinterpret_cast<const void*>(&kmeans_update_sorted_kernel<T, D, true>)
                      : reinterpret_cast<const void*>(&kmeans_update_sorted_kernel<T, D, false>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  const dim3 grid(unsigned((C + CG - 1) / CG), unsigned(heads));
  if (gl)
    hipLaunchKernelGGL((kmeans_update_sorted_kernel<T, D, true>), grid, dim3(512), lds, st, static_cast<const T*>(x),
                       static_cast<T*>(cent), ids, C, CG, int(n), glists, gstarts);
  else
    hipLaunchKernelGGL((kmeans_update_sorted_kernel<T, D, false>), grid, dim3(512), lds, st, static_cast<const T*>(x),
                       static_cast<T*>(cent), ids, C, CG, int(n), nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_kmeans_update(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, void* cent,
                                const uint8_t* ids, void* ws, hipStream_t st) {
  if (heads == 0 || n == 0) return hipSuccess;
  if (n >= (int64_t(1) << 31)) return hipErrorInvalidValue;   // token indices are 32-bit in the lists
  if (update_global_lists(heads, n) && ws == nullptr) return hipErrorInvalidValue;
  if (dt == KVC_BF16 && dim == 128) return run_kmeans_update_sorted<bf16_t, 128>(heads, n, x, C, cent, ids, ws, st);
  if (dt == KVC_BF16 && dim == 64) return run_kmeans_update_sorted<bf16_t, 64>(heads, n, x, C, cent, ids, ws, st);
  if (dt == KVC_F32 && dim == 128) return run_kmeans_update_sorted<float, 128>(heads, n, x, C, cent, ids, ws, st);
  if (dt == KVC_F32 && dim == 64) return run_kmeans_update_sorted<float, 64>(heads, n, x, C, cent, ids, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
