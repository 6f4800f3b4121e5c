// Query-aware centre assignment of key tokens (QSAC) and the query statistics it
// weighs with (QuantWM, section 4.1, Eqs. 6-12; the cold start of the appendix).
//
// For a key token x, centres mu_j and channel weights w (w_c = E[q_c^2] over the
// queries seen so far; all ones at the cold start):
//   1. d_w(x, mu_j) = sum_c w_c (x_c - mu_jc)^2 picks the M nearest centres (Eq. 9,
//      diagonal form; ties to the lower index);
//   2. each candidate is scored by S_j = sum_g W_g R_g^2 with R_g the range of
//      x - mu_j over group g and W_g = sum_{c in g} w_c (Eqs. 10-12: the Widrow
//      error model of uniform b-bit quantization, common factor dropped);
//   3. the token takes the candidate with the smallest score (ties to the lower
//      index).
//
// bf16 tokens.  d_w(x, mu_j) - ||x||_w^2 = ||mu_j||_w^2 - 2 (w*x).mu_j is formed on
// v_mfma_f32_32x32x16_bf16: -2 w*x (fp32; the -2 is folded into the staged
// weights, an exact scaling) is split into bf16 hi + lo parts, so that two
// products against the bf16 centre give
// the dot product to about 2^-18 relative; the accumulator starts at ||mu_j||_w^2.
// Each lane keeps its M+1 smallest scores as packed keys (the score with its 8
// low mantissa bits replaced by the centre index, so within 2^-15 of the score,
// relative), in a sorted list that takes a new key with one min and M med3
// operations.  When the gap between the M-th and (M+1)-th key is not larger than
// twice a bound on the score error plus the packing error, the candidate set is
// recomputed exactly: fp64 distances of the centres whose computed score lies
// within that margin.  The candidates' QSAC scores are
// computed in fp32.  fp32 tokens take the exact path
// throughout, with fp64 scores.
#include "kvc_internal.h"
#include "dev_common.h"
#include "mfma.h"

namespace kvc {
namespace {

// The L smallest (score, index) pairs seen, ascending, ties by index.
template <typename S, int L>
struct TopList {
  S s[L];
  int i[L];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int k = 0; k < L; ++k) { s[k] = S(INFINITY); i[k] = 0x7fffffff; }
  }
  // branch-free insertion: the larger of each comparison moves down the list
  __device__ __forceinline__ void insert(S v, int vi) {
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const bool lt = v < s[k] || (v == s[k] && vi < i[k]);
      const S ts = lt ? v : s[k];
      const int ti = lt ? vi : i[k];
      v = lt ? s[k] : v;
      vi = lt ? i[k] : vi;
      s[k] = ts;
      i[k] = ti;
    }
  }
};

template <typename T>
__device__ __forceinline__ double elem64(const T* p, int c);
template <>
__device__ __forceinline__ double elem64<bf16_t>(const bf16_t* p, int c) {
  return double(__uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(p)[c]) << 16));
}
template <>
__device__ __forceinline__ double elem64<float>(const float* p, int c) {
  return double(p[c]);
}

// Exact candidates of one token, by one wavefront: the fp64 weighted distance of
// every centre (lane k takes centres k, k+64, ...; channels in ascending order)
// goes to the wave's LDS slot, then every lane scans them in index order and
// keeps the M nearest.  All lanes return the same list.
template <typename T, int D, int M>
__device__ void exact_candidates(const T* __restrict__ xr, const T* __restrict__ centh, const float* __restrict__ sW,
                                 int C, int lane, double* __restrict__ sD, TopList<double, M>& out) {
  for (int c = lane; c < C; c += 64) {
    const T* cr = centh + int64_t(c) * D;
    double d = 0.0;
    for (int k = 0; k < D; ++k) {
      const double t = elem64<T>(xr, k) - elem64<T>(cr, k);
      d = __dadd_rn(d, __dmul_rn(double(sW[k]), __dmul_rn(t, t)));
    }
    sD[c] = d;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  out.init();
  for (int c = 0; c < C; ++c) out.insert(sD[c], c);
  __builtin_amdgcn_wave_barrier();
}

// fp64 QSAC score of centre row cr for token row xr (groups of G channels).
template <typename T, int D>
__device__ double qsac_score64(const T* __restrict__ xr, const T* __restrict__ cr, const float* __restrict__ sWg,
                               int G) {
  double s = 0.0;
  for (int g0 = 0; g0 < D; g0 += G) {
    double mn = INFINITY, mx = -INFINITY;
    for (int k = g0; k < g0 + G; ++k) {
      const double r = elem64<T>(xr, k) - elem64<T>(cr, k);
      mn = fmin(mn, r);
      mx = fmax(mx, r);
    }
    const double R = mx - mn;
    s = __dadd_rn(s, __dmul_rn(double(sWg[g0 / G]), __dmul_rn(R, R)));
  }
  return s;
}

// Weights (all ones without w) and their group sums into LDS.
template <int D>
__device__ __forceinline__ void load_weights(const float* __restrict__ w, int h, int G, float* sW, float* sWg) {
  const int tid = threadIdx.x;
  if (tid < D) sW[tid] = w ? w[int64_t(h) * D + tid] : 1.f;
  __syncthreads();
  if (tid < D / G) {
    float s = 0.f;
    for (int k = 0; k < G; ++k) s += sW[tid * G + k];
    sWg[tid] = s;
  }
  __syncthreads();
}

// fp32 tokens: one wavefront per token, exact candidates and fp64 scores.
template <int D, int M>
__global__ __launch_bounds__(256) void qsac_exact_kernel(const float* __restrict__ x, const float* __restrict__ cent,
                                                         const float* __restrict__ w, int C, int64_t n, int G,
                                                         uint8_t* __restrict__ ids) {
  __shared__ float sW[D];
  __shared__ float sWg[D / 16];
  __shared__ double sD[4][256];
  const int h = blockIdx.y;
  load_weights<D>(w, h, G, sW, sWg);
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int64_t j = int64_t(blockIdx.x) * 4 + wave;
  if (j >= n) return;               // wave-uniform, after the block's last barrier
  const float* xr = x + (int64_t(h) * n + j) * D;
  const float* centh = cent + int64_t(h) * C * D;
  TopList<double, M> cand;
  exact_candidates<float, D, M>(xr, centh, sW, C, lane, sD[wave], cand);
  double best = INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < M; ++k) {
    if (cand.i[k] >= C) continue;
    const double s = qsac_score64<float, D>(xr, centh + int64_t(cand.i[k]) * D, sWg, G);
    if (s < best || (s == best && cand.i[k] < bi)) { best = s; bi = cand.i[k]; }
  }
  if (bi >= C) bi = cand.i[0] < C ? cand.i[0] : 0;   // non-finite scores: the nearest candidate
  if (lane == 0) ids[int64_t(h) * n + j] = static_cast<uint8_t>(bi);
}

template <int D, int M>
__global__ __launch_bounds__(256) void qsac_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ cent,
                                                        const float* __restrict__ w, int C, int64_t n, int G,
                                                        uint8_t* __restrict__ ids) {
  constexpr int ROWP = D + 8;          // padded LDS row (bf16 elements): conflict-free fragment reads
  constexpr int KC = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sC[256 * ROWP];
  __shared__ float sN[256];
  __shared__ float sW[D];
  __shared__ float sWm2[D];            // -2 w: the token operand's factor (exact scaling)
  __shared__ float sWg[D / 16];
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

  // centre table into LDS (all loads of a thread issued before its stores)
  {
    constexpr int PER_T = 256 * (D / 8) / 256;
    uint4 v[PER_T];
#pragma unroll
    for (int it = 0; it < PER_T; ++it) {
      const int e = tid + it * 256;
      const int row = e / (D / 8), c8 = e % (D / 8);
      v[it] = make_uint4(0, 0, 0, 0);
      if (row < C) v[it] = *reinterpret_cast<const uint4*>(centh + int64_t(row) * D + c8 * 8);
    }
#pragma unroll
    for (int it = 0; it < PER_T; ++it) {
      const int e = tid + it * 256;
      const int row = e / (D / 8), c8 = e % (D / 8);
      if (row < rows) *reinterpret_cast<uint4*>(&sC[row * ROWP + c8 * 8]) = v[it];
    }
  }
  load_weights<D>(w, h, G, sW, sWg);   // ends with a barrier
  // ||mu||_w^2 in fp32, channels in order; padding rows score the largest finite
  // value (their packed keys stay finite and sort last)
  {
    float sn = 3.40282347e+38f;
    if (tid < C) {
      sn = 0.f;
      for (int c = 0; c < D; ++c) {
        const float m = __uint_as_float(uint32_t(sC[tid * ROWP + c]) << 16);
        sn = fmaf(sW[c] * m, m, sn);
      }
    }
    if (tid < rows) sN[tid] = sn;
    if (tid < D) sWm2[tid] = -2.f * sW[tid];
  }
  __syncthreads();
  float cmax = 0.f;
  for (int c = lane; c < C; c += 64) cmax = fmaxf(cmax, sN[c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, 64));
  // Bound on |computed - exact| of one score, u = 2^-24: the weighted norm takes
  // 2D roundings (n_c (1 + 2D u)); b = fl(w*x) (u) and its hi + lo split (2^-18)
  // perturb the cross term by (u + 2^-18) S; the 2D + 1 terms of the matrix
  // accumulation add 2D u (n_c + 2 S); S = sum |w x mu| <= sqrt(||x||_w^2 n_c)
  // (weights >= 0).  So |err| <= (4D + 4) u cmax + (2^-17 + (4D + 4) u)
  // sqrt(||x||_w^2 cmax) with cmax = max_c n_c.
  const float err_a = float(4 * D + 4) * 5.9604645e-08f;
  const float err_b = 7.6293945e-06f + err_a;

  const int64_t wave_tok0 = int64_t(blockIdx.x) * 256 + wave * 64;
  for (int cb = 0; cb < 2; ++cb) {
    const int64_t tok0 = wave_tok0 + cb * 32;
    if (tok0 >= n) break;              // wave-uniform; no barrier follows
    const int64_t tok = tok0 + col;
    const bool valid = tok < n;
    const bf16_t* xr = x + (int64_t(h) * n + (valid ? tok : tok0)) * D;

    // token fragment: channels kc*16 + half*8 + e; raw values kept for the scores
    uint4 xraw[KC];
    bf16x8 bhi[KC], blo[KC];
    float xxw = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      xraw[kc] = valid ? *reinterpret_cast<const uint4*>(xr + kc * 16 + half * 8) : make_uint4(0, 0, 0, 0);
      const uint32_t ww[4] = {xraw[kc].x, xraw[kc].y, xraw[kc].z, xraw[kc].w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = kc * 16 + half * 8 + 2 * i;
        // b = -2 w x: the factor -2 scales fl(w x), its bf16 parts and the norm
        // terms exactly, so these are -2 times the parts of w x
        const float x0 = bf16_lo(ww[i]), x1 = bf16_hi(ww[i]);
        const float b0 = sWm2[c] * x0, b1 = sWm2[c + 1] * x1;
        xxw = fmaf(b0, x0, xxw);
        xxw = fmaf(b1, x1, xxw);
        const uint32_t hp = pack_bf16x2(b0, b1);
        hw[i] = hp;
        lw[i] = pack_bf16x2(b0 - bf16_lo(hp), b1 - bf16_hi(hp));
      }
      bhi[kc] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
      blo[kc] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
    xxw = -0.5f * (xxw + __shfl_xor(xxw, 32, 64));   // ||x||_w^2

    // approximate weighted scores: the M+1 smallest packed keys of this lane's
    // rows (this half's 16 rows of each block), ascending
    float key[M + 1];
#pragma unroll
    for (int k = 0; k <= M; ++k) key[k] = INFINITY;
    // insertion into the sorted list from its old entries: entry k becomes the
    // median of old entries k-1, k and the new key, entry 0 the smaller of old
    // entry 0 and the new key
    auto put = [&](float v) {
      float nk[M + 1];
      // written out: the compiler's min would first canonicalize the packed keys
      asm("v_min_f32 %0, %1, %2" : "=v"(nk[0]) : "v"(key[0]), "v"(v));
#pragma unroll
      for (int k = 1; k <= M; ++k) nk[k] = __builtin_amdgcn_fmed3f(key[k - 1], key[k], v);
#pragma unroll
      for (int k = 0; k <= M; ++k) key[k] = nk[k];
    };
    for (int blk = 0; blk < nblk; ++blk) {
      f32x16 acc;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 t = *reinterpret_cast<const float4*>(&sN[blk * 32 + 8 * g4 + 4 * half]);
        acc[4 * g4 + 0] = t.x; acc[4 * g4 + 1] = t.y; acc[4 * g4 + 2] = t.z; acc[4 * g4 + 3] = t.w;
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&sC[(blk * 32 + col) * ROWP + kc * 16 + half * 8]));
        acc = mfma32(a, bhi[kc], acc);
        acc = mfma32(a, blo[kc], acc);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t row = uint32_t(blk * 32 + 8 * (v / 4) + 4 * half + (v % 4));
        put(__uint_as_float((__float_as_uint(acc[v]) & ~0xFFu) | row));
      }
    }
    // merge with the other half of the rows (lane ^ 32): copy its list first
    {
      float ok[M + 1];
#pragma unroll
      for (int k = 0; k <= M; ++k) ok[k] = __shfl_xor(key[k], 32, 64);
#pragma unroll
      for (int k = 0; k <= M; ++k) put(ok[k]);
    }
    int cand[M];
#pragma unroll
    for (int k = 0; k < M; ++k) cand[k] = key[k] < INFINITY ? int(__float_as_uint(key[k]) & 0xFFu) : 0x7fffffff;
    // the set of the M nearest is certain when the (M+1)-th key is more than
    // twice the score error bound, plus the packing error of the two keys (2^-15
    // relative each, taken as 2^-14), above the M-th one (or there are at most M
    // centres)
    const float thr = err_a * cmax + err_b * sqrtf(xxw * cmax);
    const float pack_err = 6.1035156e-05f * (fabsf(key[M]) + fabsf(key[M - 1]));
    const bool flag = valid && C > M && !(key[M] - key[M - 1] > 2.f * thr + pack_err);   // also catches NaN
    uint64_t mask = __ballot(flag && half == 0);
    if (mask) {
      // Each computed score is within thr of its exact value, so every centre of
      // the exact M nearest scores at most 2*thr above the M-th computed score
      // (itself within the packing error of the M-th key):
      // this pass's scores are formed once more to mark the centres under that
      // limit, and only those are re-scored exactly (fp64, dimensions spread over
      // the lanes, a fixed reduction order).
      const float lim = key[M - 1] + 6.1035156e-05f * fabsf(key[M - 1]) + 2.f * thr;
      uint32_t cm[8];                 // marked rows of block blk: 16 bits per lane
#pragma unroll
      for (int q = 0; q < 8; ++q) cm[q] = 0;
      for (int blk = 0; blk < nblk; ++blk) {
        f32x16 acc;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 t = *reinterpret_cast<const float4*>(&sN[blk * 32 + 8 * g4 + 4 * half]);
          acc[4 * g4 + 0] = t.x; acc[4 * g4 + 1] = t.y; acc[4 * g4 + 2] = t.z; acc[4 * g4 + 3] = t.w;
        }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&sC[(blk * 32 + col) * ROWP + kc * 16 + half * 8]));
          acc = mfma32(a, bhi[kc], acc);
          acc = mfma32(a, blo[kc], acc);
        }
        uint32_t bits = 0;
#pragma unroll
        for (int v = 0; v < 16; ++v) bits |= (acc[v] <= lim ? 1u : 0u) << v;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q == blk) cm[q] = bits;
      }
      constexpr int PERL = D / 64;    // dimensions per lane in the exact re-scoring
      while (mask) {
        const int b = __builtin_ctzll(mask);
        mask &= mask - 1;
        // the token's row from the two lanes that hold it, through this
        // wavefront's LDS row (LDS operations of one wavefront complete in order)
        if (col == b) {
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) *reinterpret_cast<uint4*>(&sX[wave][kc * 16 + half * 8]) = xraw[kc];
        }
        double xd[PERL], wd[PERL];
#pragma unroll
        for (int i = 0; i < PERL; ++i) {
          xd[i] = double(__uint_as_float(uint32_t(sX[wave][lane * PERL + i]) << 16));
          wd[i] = double(sW[lane * PERL + i]);
        }
        auto exact = [&](int ci) -> double {
          double part = 0.0;
#pragma unroll
          for (int i = 0; i < PERL; ++i) {
            const double t = xd[i] - double(__uint_as_float(uint32_t(sC[ci * ROWP + lane * PERL + i]) << 16));
            part = __dadd_rn(part, __dmul_rn(wd[i], __dmul_rn(t, t)));
          }
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) part = __dadd_rn(part, __shfl_xor(part, o, 64));
          return part;
        };
        TopList<double, M> ex;
        ex.init();
        int seen = 0;
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
            if (ci >= C) continue;     // a padding row (only under a non-finite limit)
            ex.insert(exact(ci), ci);
            ++seen;
          }
        }
        if (seen < M) {               // non-finite scores: every centre, exactly
          ex.init();
          for (int ci = 0; ci < C; ++ci) ex.insert(exact(ci), ci);
        }
        if (col == b) {
#pragma unroll
          for (int k = 0; k < M; ++k) cand[k] = ex.i[k];
        }
      }
    }

    // QSAC scores of the candidates in fp32: each half of a token's lanes holds 8
    // channels of every 16; group ranges are combined across the pair
    float best = INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < M; ++k) {
      const int cj = cand[k];
      const bool ok = cj < C;
      const int row = ok ? cj : 0;
      float score = 0.f, mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 cm = *reinterpret_cast<const uint4*>(&sC[row * ROWP + kc * 16 + half * 8]);
        const uint32_t xw[4] = {xraw[kc].x, xraw[kc].y, xraw[kc].z, xraw[kc].w};
        const uint32_t mw[4] = {cm.x, cm.y, cm.z, cm.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float r0 = bf16_lo(xw[i]) - bf16_lo(mw[i]);
          const float r1 = bf16_hi(xw[i]) - bf16_hi(mw[i]);
          mn = fminf(mn, fminf(r0, r1));
          mx = fmaxf(mx, fmaxf(r0, r1));
        }
        if ((kc * 16 + 16) % G == 0) {   // last chunk of a group
          mn = fminf(mn, __shfl_xor(mn, 32, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const float R = mx - mn;
          score = __fadd_rn(score, __fmul_rn(sWg[(kc * 16) / G], __fmul_rn(R, R)));
          mn = INFINITY;
          mx = -INFINITY;
        }
      }
      if (ok && (score < best || (score == best && cj < bi))) { best = score; bi = cj; }
    }
    if (bi >= C) bi = cand[0] < C ? cand[0] : 0;        // non-finite scores: the nearest candidate
    if (valid && half == 0) ids[int64_t(h) * n + tok] = static_cast<uint8_t>(bi);
  }
}

// Second moments of the queries per head and channel (QuantWM, section 4.1,
// Eqs. 6-8, diagonal): w <- (n_prev * w + sum_i q_ic^2) / (n_prev + n_q), sums in
// fp64, in two launches with a fixed reduction order:
//   1. grid (row blocks, heads): a workgroup reads its block of rows whole (each
//      row by consecutive threads, 16 bytes each), every thread summing its
//      channels over the rows i = lane row + k * RL in increasing order; the RL
//      row lanes are then added in order, giving the block's partial sums;
//   2. one thread per (head, channel) adds the blocks' partial sums in block
//      order and folds in the previous statistics.
template <typename T, int D>
__global__ __launch_bounds__(256) void query_stats_partial_kernel(const T* __restrict__ q, int64_t n_q, int64_t rows,
                                                                  double* __restrict__ part) {
  constexpr int CPT = 16 / int(sizeof(T));     // channels per thread (one 16-byte load)
  constexpr int NG = D / CPT;                  // channel groups of a row
  constexpr int RL = 256 / NG;                 // row lanes
  __shared__ double sp[RL][D];
  const int h = blockIdx.y, b = blockIdx.x;
  const int g = threadIdx.x % NG, rl = threadIdx.x / NG;
  const int64_t r0 = int64_t(b) * rows;
  const int64_t r1 = r0 + rows < n_q ? r0 + rows : n_q;
  const T* qh = q + int64_t(h) * n_q * D + g * CPT;
  double s[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) s[k] = 0.0;
  for (int64_t i = r0 + rl; i < r1; i += RL) {
    float v[CPT];
    load_row<CPT>(qh + i * D, v);
#pragma unroll
    for (int k = 0; k < CPT; ++k) s[k] = __dadd_rn(s[k], __dmul_rn(double(v[k]), double(v[k])));
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k) sp[rl][g * CPT + k] = s[k];
  __syncthreads();
  if (threadIdx.x < D) {
    double tot = sp[0][threadIdx.x];
    for (int k = 1; k < RL; ++k) tot = __dadd_rn(tot, sp[k][threadIdx.x]);
    part[(int64_t(h) * gridDim.x + b) * D + threadIdx.x] = tot;
  }
}

template <int D>
__global__ __launch_bounds__(D) void query_stats_finish_kernel(const double* __restrict__ part, int nb, int64_t n_q,
                                                               int64_t n_prev, float* __restrict__ w) {
  const int h = blockIdx.x, c = threadIdx.x;
  const double* ph = part + int64_t(h) * nb * D + c;
  double tot = 0.0;
  for (int b = 0; b < nb; ++b) tot = __dadd_rn(tot, ph[int64_t(b) * D]);
  float* wc = w + int64_t(h) * D + c;
  if (n_prev > 0) tot = __dadd_rn(tot, __dmul_rn(double(*wc), double(n_prev)));
  *wc = float(tot / double(n_prev + n_q));
}

template <int D, int M>
hipError_t run_qsac(int heads, int64_t n, kvc_dtype dt, const void* x, int C, const void* cent, const float* w,
                    int G, uint8_t* ids, hipStream_t st) {
  if (dt == KVC_BF16) {
    const dim3 grid(unsigned((n + 255) / 256), unsigned(heads));
    hipLaunchKernelGGL((qsac_mfma_kernel<D, M>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(x),
                       static_cast<const bf16_t*>(cent), w, C, n, G, ids);
  } else {
    const dim3 grid(unsigned((n + 3) / 4), unsigned(heads));
    hipLaunchKernelGGL((qsac_exact_kernel<D, M>), grid, dim3(256), 0, st, static_cast<const float*>(x),
                       static_cast<const float*>(cent), w, C, n, G, ids);
  }
  return hipGetLastError();
}

template <int D>
hipError_t pick_m(int heads, int64_t n, kvc_dtype dt, const void* x, int C, const void* cent, const float* w,
                  int n_cand, int G, uint8_t* ids, hipStream_t st) {
  switch (n_cand) {
    case 1: return run_qsac<D, 1>(heads, n, dt, x, C, cent, w, G, ids, st);
    case 2: return run_qsac<D, 2>(heads, n, dt, x, C, cent, w, G, ids, st);
    case 4: return run_qsac<D, 4>(heads, n, dt, x, C, cent, w, G, ids, st);
    case 8: return run_qsac<D, 8>(heads, n, dt, x, C, cent, w, G, ids, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_assign_qsac(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, const void* cent,
                              const float* w, int n_cand, int group, uint8_t* ids, hipStream_t st) {
  if (heads == 0 || n == 0) return hipSuccess;
  if (dim == 128) return pick_m<128>(heads, n, dt, x, C, cent, w, n_cand, group, ids, st);
  if (dim == 64) return pick_m<64>(heads, n, dt, x, C, cent, w, n_cand, group, ids, st);
  return hipErrorInvalidValue;
}

int query_stats_blocks(int heads, int64_t n_q) {
  // about 1024 workgroups in all, at most one per 256 rows
  const int64_t want = (1024 + heads - 1) / heads;
  const int64_t most = (n_q + 255) / 256;
  const int64_t nb = want < most ? want : most;
  return int(nb > 0 ? nb : 1);
}

size_t query_stats_workspace(int heads, int64_t n_q, int dim) {
  return size_t(heads) * size_t(query_stats_blocks(heads, n_q)) * size_t(dim) * sizeof(double);
}

template <typename T, int D>
hipError_t run_query_stats(int heads, int64_t n_q, const void* q, int64_t n_prev, float* w, double* part,
                           hipStream_t st) {
  const int nb = query_stats_blocks(heads, n_q);
  const int64_t rows = (n_q + nb - 1) / nb;
  hipLaunchKernelGGL((query_stats_partial_kernel<T, D>), dim3(unsigned(nb), unsigned(heads)), dim3(256), 0, st,
                     static_cast<const T*>(q), n_q, rows, part);
  hipLaunchKernelGGL((query_stats_finish_kernel<D>), dim3(unsigned(heads)), dim3(D), 0, st, part, nb, n_q, n_prev, w);
  return hipGetLastError();
}

hipError_t launch_query_stats(int heads, int64_t n_q, int dim, kvc_dtype dt, const void* q, int64_t n_prev,
                              float* w, void* ws, hipStream_t st) {
  if (heads == 0 || n_q == 0) return hipSuccess;
  double* part = static_cast<double*>(ws);
  if (dt == KVC_BF16) {
    if (dim == 128) return run_query_stats<bf16_t, 128>(heads, n_q, q, n_prev, w, part, st);
    return run_query_stats<bf16_t, 64>(heads, n_q, q, n_prev, w, part, st);
  }
  if (dim == 128) return run_query_stats<float, 128>(heads, n_q, q, n_prev, w, part, st);
  return run_query_stats<float, 64>(heads, n_q, q, n_prev, w, part, st);
}

}  // namespace kvc
