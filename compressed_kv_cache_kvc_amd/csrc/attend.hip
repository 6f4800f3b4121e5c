// Attention of the current chunk's queries over compressed history.
//
// The history is read as centre + dequantized residual (TempoKV, section 3.3,
// Eq. 2), decoded during attention rather than reconstructed up front (TempoKV,
// section 4.2 on the latency of decoding the cache during attention).  The
// softmax runs online over 64-token tiles and each row's log-sum-exp is returned
// for merging (NanoKV, Figure 4d).  The low-dimensional variant reads far history
// as coefficients in a reduced basis, with reduced queries and a restored output
// dimension (NanoKV, Figure 4a and 4d).
//
// Work decomposition (matrix-core path): a workgroup of 8 wavefronts owns 256
// queries of one head (32 per wavefront) and one share of the history tiles.
// Per tile:
//   1. every thread dequantizes one (token, channel group) of K and of V from the
//      packed codes, the fp16 (scale, zero) pair and the centre row into fp16
//      tiles in LDS (K row-major, V transposed with a key permutation that lets
//      the probabilities feed the second product straight from registers);
//   2. each wavefront computes S^T = K_hat Q^T on v_mfma_f32_32x32x16_f16, so a
//      lane holds 32 scores of one query; the online softmax uses exp2 with the
//      1/sqrt(d) log2(e) factor applied in fp32;
//   3. O^T += V_hat^T P^T on the same instruction.
// The tiles are fp16 rather than bf16: same matrix-core rate, three more mantissa
// bits, which keeps the logit error of keys with large outlier channels inside
// the accuracy target.  Reconstructed keys, values and the queries must lie in the
// fp16 range, the same range the codec's fp16 scale and zero-point already impose.
//
// Latency hiding: the centre ids of tile t+2 and the codes, metadata and centre
// rows of tile t+1 are loaded (unconditionally, with clamped indices, so no load
// result is needed before its use) while tile t is multiplied; tile t+1 is then
// dequantized into the other LDS buffer.  The running maximum of a row is only
// raised when a tile's maximum exceeds it by more than 8 (log2 units), so the
// output accumulator is rarely rescaled; probabilities then stay below 2^8.
#include "kvc_internal.h"
#include "dev_common.h"
#include "mfma.h"

#include <type_traits>

namespace kvc {
namespace {

struct AttendParams {
  const uint16_t* q;      // queries [H][n_q][DQ]: bf16 (full dim) or fp16 (reduced queries, low-dim path)
  int64_t n_q;
  int heads;
  int n_split;
  float scale_log2;       // log2(e) / sqrt(head dim)
  float* out;             // [n_split][H][n_q][DOUT]
  float* lse;             // [n_split][H][n_q]
  const float* basis_v;   // low-dim: [H][DOUT][DQ]
};

template <int NB>
using code_t = typename std::conditional<(NB > 4), uint64_t, uint32_t>::type;

template <int NB>
__device__ __forceinline__ code_t<NB> load_code_bits(const uint8_t* p) {
  if constexpr (NB == 1) return *p;
  else if constexpr (NB == 2) return *reinterpret_cast<const uint16_t*>(p);
  else if constexpr (NB == 4) return *reinterpret_cast<const uint32_t*>(p);
  else {
    static_assert(NB == 8, "code chunk");
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return uint64_t(w.x) | (uint64_t(w.y) << 32);
  }
}

// Position of key offset o (0..15) inside a 16-key chunk of the transposed V
// tile: bits 2 and 3 swapped, matching the row order of the S^T accumulator.
__device__ __forceinline__ int vperm(int k) {
  const int o = k & 15;
  return (k & ~15) | (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1);
}

template <int DQ, int KB, int VB, int G, typename CT, bool LOWDIM, int DOUT>
__global__ __launch_bounds__(512, 1) void attend_kernel(AttendParams p, SegList segs) {
  constexpr int KC = DQ / 16;     // k-chunks of the QK^T product
  constexpr int NDB = DQ / 32;    // 32-row blocks of O^T
  constexpr int ROWK = DQ + 8;    // padded LDS rows (fp16 elements)
  constexpr int ROWV = 64 + 8;
  constexpr int CH = DQ / 8;      // channels per dequantizing thread
  constexpr int KNB = CH * KB / 8, VNB = CH * VB / 8;
  static_assert(G % CH == 0, "a thread's channels must sit in one group");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][64 * ROWK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][DQ * ROWV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int h = blockIdx.y;
  const int split = blockIdx.z;
  const int64_t qi = int64_t(blockIdx.x) * 256 + wave * 32 + col;
  const bool q_ok = qi < p.n_q;

  // B operand Q^T in fp16: bf16 queries convert exactly inside the fp16 range
  f16x8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (q_ok) w = *reinterpret_cast<const uint4*>(p.q + (int64_t(h) * p.n_q + qi) * DQ + kc * 16 + half * 8);
    if constexpr (!LOWDIM) {
      w = make_uint4(pack_f16x2(bf16_lo(w.x), bf16_hi(w.x)), pack_f16x2(bf16_lo(w.y), bf16_hi(w.y)),
                     pack_f16x2(bf16_lo(w.z), bf16_hi(w.z)), pack_f16x2(bf16_lo(w.w), bf16_hi(w.w)));
    }
    qf[kc] = as_f16x8(w);
  }

  const int64_t T = segs.total_tiles;
  const int64_t t_begin = T * split / p.n_split;
  const int64_t t_end = T * (split + 1) / p.n_split;

  const int dk = lane;            // dequant role: token within the tile
  const int dg = wave;            // channel group [dg*CH, dg*CH + CH)

  using cent_t = typename std::conditional<LOWDIM, float, CT>::type;
  constexpr int CW = CH * int(sizeof(cent_t)) / 16;   // 16-byte words of one centre chunk
  static_assert(CW >= 1, "centre chunk");

  // A cursor holds the segment of the tiles it walks over, with its arrays
  // already offset to this workgroup's head; being wave-uniform its fields live
  // in scalar registers, and are reloaded only when the cursor crosses into the
  // next segment, so no scalar memory load sits in the tile loop otherwise.
  struct Cursor {
    int si;
    int64_t tile_begin, tile_end;
    int n_tokens;
    const uint8_t *k_codes, *v_codes, *k_ids, *v_ids;
    const uint32_t *k_meta, *v_meta;
    const cent_t *k_cent, *v_cent;
  };
  auto cursor_load = [&](Cursor& c, int si) {
    const SegDev& s = segs.s[si];
    c.si = si;
    c.tile_begin = s.tile_begin;
    c.tile_end = si + 1 < segs.n ? segs.s[si + 1].tile_begin : segs.total_tiles;
    c.n_tokens = int(s.n_tokens);
    const int64_t hn = int64_t(h) * s.n_tokens;
    c.k_codes = s.k_codes + hn * (DQ * KB / 8);
    c.v_codes = s.v_codes + hn * (DQ * VB / 8);
    c.k_ids = s.k_ids + hn;
    c.v_ids = s.v_ids + hn;
    c.k_meta = s.k_meta + hn * (DQ / G);
    c.v_meta = s.v_meta + hn * (DQ / G);
    const int64_t hc = int64_t(h) * s.n_centroids * DQ;
    if constexpr (LOWDIM) {
      c.k_cent = reinterpret_cast<const cent_t*>(s.k_cent_proj) + hc;
      c.v_cent = reinterpret_cast<const cent_t*>(s.v_cent_proj) + hc;
    } else {
      c.k_cent = static_cast<const cent_t*>(s.k_cent) + hc;
      c.v_cent = static_cast<const cent_t*>(s.v_cent) + hc;
    }
  };
  auto cursor_seek = [&](Cursor& c, int64_t t) {
    while (t >= c.tile_end) cursor_load(c, c.si + 1);
  };
  // token (within the head) of this thread's row in tile t, clamped into the
  // segment so that every load is in bounds; rows past the end read real
  // (finite) data and are masked out of the softmax
  auto row_of = [&](const Cursor& c, int64_t t) -> uint32_t {
    const int j0 = int(t - c.tile_begin) * 64;
    const int last = c.n_tokens - 1;
    return uint32_t(j0 + dk < last ? j0 + dk : last);
  };

  // ---- register pipeline (raw loaded words; converted only at dequantization)
  int kid_n = 0, vid_n = 0;       // ids of the tile to load next (t+1)
  code_t<KNB> kc_r = 0;
  code_t<VNB> vc_r = 0;
  uint32_t km_r = 0, vm_r = 0;
  uint4 kcw[CW], vcw[CW];

  auto load_ids = [&](const Cursor& c, int64_t t, int& ki, int& vi) {
    const uint32_t j = row_of(c, t);
    ki = c.k_ids[j];
    vi = c.v_ids[j];
  };
  auto load_data = [&](const Cursor& c, int64_t t, int ki, int vi) {
    const uint32_t j = row_of(c, t);
    kc_r = load_code_bits<KNB>(c.k_codes + (j * uint32_t(DQ * KB / 8) + uint32_t(dg * KNB)));
    vc_r = load_code_bits<VNB>(c.v_codes + (j * uint32_t(DQ * VB / 8) + uint32_t(dg * VNB)));
    km_r = c.k_meta[j * uint32_t(DQ / G) + uint32_t((dg * CH) / G)];
    vm_r = c.v_meta[j * uint32_t(DQ / G) + uint32_t((dg * CH) / G)];
    const uint4* kp = reinterpret_cast<const uint4*>(c.k_cent + (uint32_t(ki) * DQ + dg * CH));
    const uint4* vp = reinterpret_cast<const uint4*>(c.v_cent + (uint32_t(vi) * DQ + dg * CH));
#pragma unroll
    for (int i = 0; i < CW; ++i) { kcw[i] = kp[i]; vcw[i] = vp[i]; }
  };

  // element e of a raw centre chunk as fp32
  auto cent_at = [&](const uint4 (&w)[CW], int e) -> float {
    if constexpr (sizeof(cent_t) == 2) {
      const uint4 q = w[e / 8];
      const int k = (e % 8) / 2;
      const uint32_t x = k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
      return (e & 1) ? bf16_hi(x) : bf16_lo(x);
    } else {
      const uint4 q = w[e / 4];
      const int k = e % 4;
      return __uint_as_float(k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w);
    }
  };

  auto store_tile = [&](int buf) {
    const float ks = f16_bits_to_f32(km_r & 0xffffu), kz = f16_bits_to_f32(km_r >> 16);
    const float vs = f16_bits_to_f32(vm_r & 0xffffu), vz = f16_bits_to_f32(vm_r >> 16);
    uint32_t kw[CH / 2];
#pragma unroll
    for (int e = 0; e < CH; e += 2) {
      const float q0 = float(uint32_t(kc_r >> (KB * e)) & ((1u << KB) - 1));
      const float q1 = float(uint32_t(kc_r >> (KB * (e + 1))) & ((1u << KB) - 1));
      const float k0 = cent_at(kcw, e) + fmaf(q0, ks, kz);
      const float k1 = cent_at(kcw, e + 1) + fmaf(q1, ks, kz);
      kw[e / 2] = pack_f16x2(k0, k1);
    }
    uint16_t* kdst = &sK[buf][dk * ROWK + dg * CH];
    if constexpr (CH == 16) {
      reinterpret_cast<uint4*>(kdst)[0] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
      reinterpret_cast<uint4*>(kdst)[1] = make_uint4(kw[4], kw[5], kw[6], kw[7]);
    } else if constexpr (CH == 8) {
      reinterpret_cast<uint4*>(kdst)[0] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
    } else {
      static_assert(CH == 4, "channels per thread");
      reinterpret_cast<uint2*>(kdst)[0] = make_uint2(kw[0], kw[1]);
    }
    const int vp = vperm(dk);
#pragma unroll
    for (int e = 0; e < CH; e += 2) {
      const float q0 = float(uint32_t(vc_r >> (VB * e)) & ((1u << VB) - 1));
      const float q1 = float(uint32_t(vc_r >> (VB * (e + 1))) & ((1u << VB) - 1));
      const float v0 = cent_at(vcw, e) + fmaf(q0, vs, vz);
      const float v1 = cent_at(vcw, e + 1) + fmaf(q1, vs, vz);
      const uint32_t w = pack_f16x2(v0, v1);
      sV[buf][(dg * CH + e) * ROWV + vp] = static_cast<uint16_t>(w & 0xffffu);
      sV[buf][(dg * CH + e + 1) * ROWV + vp] = static_cast<uint16_t>(w >> 16);
    }
  };

  float m_run = -INFINITY;        // reference maximum of the row, log2 units
  float l_run = 0.f;              // this lane's share of the running sum
  f32x16 o[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[b][v] = 0.f;

  auto clamp_t = [&](int64_t t) { return t < t_end ? t : t_end - 1; };
  Cursor cur_ids, cur_data, cur_comp;
  if (t_begin < t_end) {
    cursor_load(cur_data, 0);
    cursor_seek(cur_data, t_begin);
    cur_ids = cur_data;
    cur_comp = cur_data;
    int k0, v0;
    load_ids(cur_data, t_begin, k0, v0);
    load_data(cur_data, t_begin, k0, v0);
    cursor_seek(cur_ids, clamp_t(t_begin + 1));
    load_ids(cur_ids, clamp_t(t_begin + 1), kid_n, vid_n);
    store_tile(0);
  }
  __syncthreads();

  for (int64_t t = t_begin; t < t_end; ++t) {
    const int buf = int((t - t_begin) & 1);
    // issue the loads of tile t+1 (data) and t+2 (ids), clamped to the last tile so
    // that they are unconditional; they are consumed after the compute
    {
      const int64_t t1 = clamp_t(t + 1), t2 = clamp_t(t + 2);
      cursor_seek(cur_data, t1);
      load_data(cur_data, t1, kid_n, vid_n);
      cursor_seek(cur_ids, t2);
      load_ids(cur_ids, t2, kid_n, vid_n);
    }
    cursor_seek(cur_comp, t);
    const int nvalid_left = cur_comp.n_tokens - int(t - cur_comp.tile_begin) * 64;
    const int nvalid = nvalid_left >= 64 ? 64 : nvalid_left;

    // S^T = K_hat Q^T for keys [0, 32) and [32, 64)
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const f16x8 a = as_f16x8(*reinterpret_cast<const uint4*>(&sK[buf][(kb * 32 + col) * ROWK + kc * 16 + half * 8]));
        sacc[kb] = mfma32h(a, qf[kc], sacc[kb]);
      }
    }
    if (nvalid < 64) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
          if (key >= nvalid) sacc[kb][v] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * p.scale_log2;
    // raise the reference maximum only when the tile exceeds it by more than 2^8
    const bool raise = mx > m_run + 8.f;
    if (__any(raise)) {
      const float m_new = raise ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[b][v] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v], p.scale_log2, -m_run));
        sacc[kb][v] = e;
        psum += e;
      }
    l_run += psum;

    f16x8 pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int kb = c / 2, base = 8 * (c % 2);
      pf[c] = as_f16x8(make_uint4(pack_f16x2(sacc[kb][base + 0], sacc[kb][base + 1]),
                                  pack_f16x2(sacc[kb][base + 2], sacc[kb][base + 3]),
                                  pack_f16x2(sacc[kb][base + 4], sacc[kb][base + 5]),
                                  pack_f16x2(sacc[kb][base + 6], sacc[kb][base + 7])));
    }
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f16x8 a = as_f16x8(*reinterpret_cast<const uint4*>(&sV[buf][(b * 32 + col) * ROWV + c * 16 + half * 8]));
        o[b] = mfma32h(a, pf[c], o[b]);
      }

    store_tile(buf ^ 1);           // the last iteration writes a spare copy nobody reads
    __syncthreads();
  }

  // epilogue: normalise, write this split's (out, lse)
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t row = (int64_t(split) * p.heads + h) * p.n_q + qi;
  if constexpr (!LOWDIM) {
    if (q_ok) {
      float* dst = p.out + row * DOUT;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dim = b * 32 + 8 * g4 + 4 * half;
          *reinterpret_cast<float4*>(dst + dim) =
              make_float4(o[b][4 * g4] * inv, o[b][4 * g4 + 1] * inv, o[b][4 * g4 + 2] * inv, o[b][4 * g4 + 3] * inv);
        }
    }
  } else {
    // restore the output dimension: out = U_V O' (fp32).  Each lane first gathers
    // all DQ coefficients of its query, then computes half of the DOUT outputs.
    float coef[DQ];
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float mine = o[b][v] * inv;
        const float other = __shfl_xor(mine, 32, 64);
        // row 8*(v/4) + 4*half + v%4 is held by this lane, the other half's by the partner
        coef[b * 32 + 8 * (v / 4) + (v % 4)] = half == 0 ? mine : other;
        coef[b * 32 + 8 * (v / 4) + 4 + (v % 4)] = half == 0 ? other : mine;
      }
    if (q_ok) {
      const float* U = p.basis_v + int64_t(h) * DOUT * DQ;
      float* dst = p.out + row * DOUT;
      for (int i0 = half * (DOUT / 2); i0 < (half + 1) * (DOUT / 2); i0 += 4) {
        float acc4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float a = 0.f;
#pragma unroll
          for (int k = 0; k < DQ; ++k) a = fmaf(U[(i0 + u) * DQ + k], coef[k], a);
          acc4[u] = a;
        }
        *reinterpret_cast<float4*>(dst + i0) = make_float4(acc4[0], acc4[1], acc4[2], acc4[3]);
      }
    }
  }
  if (q_ok && half == 0) p.lse[row] = l > 0.f ? (m_run + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// fp32 queries: one thread per query, fp32 dequantization and softmax throughout.
template <int D, int KB, int VB, int G>
__global__ __launch_bounds__(64) void attend_f32_kernel(const float* __restrict__ q, int64_t n_q, int heads,
                                                        SegList segs, float scale, float* __restrict__ out,
                                                        float* __restrict__ lse) {
  const int64_t qi = int64_t(blockIdx.x) * 64 + threadIdx.x;
  const int h = blockIdx.y;
  if (qi >= n_q) return;
  float qv[D];
  load_row<D>(q + (int64_t(h) * n_q + qi) * D, qv);
  float m = -INFINITY, l = 0.f;
  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.f;
  for (int si = 0; si < segs.n; ++si) {
    const SegDev& s = segs.s[si];
    const float* kcent = static_cast<const float*>(s.k_cent) + int64_t(h) * s.n_centroids * D;
    const float* vcent = static_cast<const float*>(s.v_cent) + int64_t(h) * s.n_centroids * D;
    for (int64_t j = 0; j < s.n_tokens; ++j) {
      const int64_t tok = int64_t(h) * s.n_tokens + j;
      const float* kc = kcent + int64_t(s.k_ids[tok]) * D;
      const uint8_t* kcode = s.k_codes + tok * (D * KB / 8);
      float dot = 0.f;
      for (int i = 0; i < D; ++i) {
        const uint32_t w = s.k_meta[tok * (D / G) + i / G];
        const float code = float((kcode[i / (8 / KB)] >> (KB * (i % (8 / KB)))) & ((1 << KB) - 1));
        const float kh = kc[i] + fmaf(code, f16_bits_to_f32(w & 0xffffu), f16_bits_to_f32(w >> 16));
        dot = fmaf(qv[i], kh, dot);
      }
      const float sc = dot * scale;
      const float m_new = fmaxf(m, sc);
      const float alpha = expf(m - m_new);
      const float pw = expf(sc - m_new);
      l = l * alpha + pw;
      m = m_new;
      const float* vc = vcent + int64_t(s.v_ids[tok]) * D;
      const uint8_t* vcode = s.v_codes + tok * (D * VB / 8);
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const uint32_t w = s.v_meta[tok * (D / G) + i / G];
        const float code = float((vcode[i / (8 / VB)] >> (VB * (i % (8 / VB)))) & ((1 << VB) - 1));
        const float vh = vc[i] + fmaf(code, f16_bits_to_f32(w & 0xffffu), f16_bits_to_f32(w >> 16));
        acc[i] = fmaf(acc[i], alpha, pw * vh);
      }
    }
  }
  float* dst = out + (int64_t(h) * n_q + qi) * D;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) dst[i] = acc[i] * inv;
  lse[int64_t(h) * n_q + qi] = l > 0.f ? m + logf(l) : -INFINITY;
}

// Reduced queries q' = U^T q (fp32 accumulation, bf16 result).
__global__ __launch_bounds__(256) void project_queries_kernel(const uint16_t* __restrict__ q, const float* __restrict__ basis,
                                                              int64_t n_q, int D, int R, uint16_t* __restrict__ qp) {
  const int64_t item = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  if (item >= n_q * R) return;
  const int64_t qi = item / R;
  const int k = int(item % R);
  const uint16_t* qr = q + (int64_t(h) * n_q + qi) * D;
  const float* U = basis + int64_t(h) * D * R;
  float a = 0.f;
  for (int i = 0; i < D; ++i) a = fmaf(__uint_as_float(uint32_t(qr[i]) << 16), U[i * R + k], a);
  qp[(int64_t(h) * n_q + qi) * R + k] = static_cast<uint16_t>(pack_f16x2(a, 0.f) & 0xffffu);
}

// Projected centres c' = U^T c (fp32).
template <typename CT>
__global__ __launch_bounds__(256) void project_centres_kernel(const CT* __restrict__ cent, const float* __restrict__ basis,
                                                              int C, int D, int R, float* __restrict__ proj) {
  const int item = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  if (item >= C * R) return;
  const int c = item / R;
  const int k = item % R;
  const float* U = basis + int64_t(h) * D * R;
  float a = 0.f;
  for (int i = 0; i < D; ++i) {
    float cv;
    if constexpr (sizeof(CT) == 2)
      cv = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(cent)[(int64_t(h) * C + c) * D + i]) << 16);
    else
      cv = reinterpret_cast<const float*>(cent)[(int64_t(h) * C + c) * D + i];
    a = fmaf(cv, U[i * R + k], a);
  }
  proj[(int64_t(h) * C + c) * R + k] = a;
}

template <int DQ, typename CT, bool LOWDIM, int DOUT>
hipError_t pick_bits(const AttendParams& p, const SegList& segs, int kb, int vb, int g, hipStream_t st) {
  const dim3 grid(unsigned((p.n_q + 255) / 256), unsigned(p.heads), unsigned(p.n_split));
#define KVC_CASE(KB_, VB_, G_)                                                                               \
  if (kb == KB_ && vb == VB_ && g == G_) {                                                                   \
    hipLaunchKernelGGL((attend_kernel<DQ, KB_, VB_, G_, CT, LOWDIM, DOUT>), grid, dim3(512), 0, st, p, segs); \
    return hipGetLastError();                                                                                \
  }
  KVC_CASE(2, 2, 16) KVC_CASE(2, 4, 16) KVC_CASE(4, 2, 16) KVC_CASE(4, 4, 16)
  KVC_CASE(2, 2, 32) KVC_CASE(2, 4, 32) KVC_CASE(4, 2, 32) KVC_CASE(4, 4, 32)
#undef KVC_CASE
  return hipErrorInvalidValue;
}

template <int D>
hipError_t pick_f32(const float* q, int64_t n_q, int heads, const SegList& segs, int kb, int vb, int g, float* out,
                    float* lse, hipStream_t st) {
  const dim3 grid(unsigned((n_q + 63) / 64), unsigned(heads));
  const float scale = 1.0f / sqrtf(float(D));
#define KVC_CASE(KB_, VB_, G_)                                                                                 \
  if (kb == KB_ && vb == VB_ && g == G_) {                                                                     \
    hipLaunchKernelGGL((attend_f32_kernel<D, KB_, VB_, G_>), grid, dim3(64), 0, st, q, n_q, heads, segs, scale, out, \
                       lse);                                                                                   \
    return hipGetLastError();                                                                                  \
  }
  KVC_CASE(2, 2, 16) KVC_CASE(2, 4, 16) KVC_CASE(4, 2, 16) KVC_CASE(4, 4, 16)
  KVC_CASE(2, 2, 32) KVC_CASE(2, 4, 32) KVC_CASE(4, 2, 32) KVC_CASE(4, 4, 32)
#undef KVC_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attend(int heads, int64_t n_q, int dim, kvc_dtype q_dtype, const void* q, const SegList& segs,
                         int k_bits, int v_bits, int group, kvc_dtype cdt, int n_split, float* out, float* lse,
                         hipStream_t st) {
  if (heads == 0 || n_q == 0) return hipSuccess;
  if (segs.total_tiles == 0) {
    // empty history: out = 0, lse = -inf, through the merge kernel with one -inf part
    k_bits = v_bits = 2;
    group = 16;
  }
  if (q_dtype == KVC_F32) {
    if (dim == 128) return pick_f32<128>(static_cast<const float*>(q), n_q, heads, segs, k_bits, v_bits, group, out, lse, st);
    if (dim == 64) return pick_f32<64>(static_cast<const float*>(q), n_q, heads, segs, k_bits, v_bits, group, out, lse, st);
    return hipErrorInvalidValue;
  }
  AttendParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.n_q = n_q;
  p.heads = heads;
  p.n_split = n_split;
  p.scale_log2 = 1.4426950408889634f / sqrtf(float(dim));
  p.out = out;
  p.lse = lse;
  p.basis_v = nullptr;
  if (cdt != KVC_BF16 && segs.total_tiles > 0) return hipErrorInvalidValue;
  if (dim == 128) return pick_bits<128, bf16_t, false, 128>(p, segs, k_bits, v_bits, group, st);
  if (dim == 64) return pick_bits<64, bf16_t, false, 64>(p, segs, k_bits, v_bits, group, st);
  return hipErrorInvalidValue;
}

hipError_t launch_project_queries(int heads, int64_t n_q, int dim, int rank, const void* q, const float* basis,
                                  uint16_t* q_proj, hipStream_t st) {
  if (heads == 0 || n_q == 0) return hipSuccess;
  const dim3 grid(unsigned((n_q * rank + 255) / 256), unsigned(heads));
  hipLaunchKernelGGL(project_queries_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t*>(q), basis, n_q, dim,
                     rank, q_proj);
  return hipGetLastError();
}

hipError_t launch_project_centres(int heads, int C, int dim, int rank, kvc_dtype cdt, const void* cent,
                                  const float* basis, float* proj, hipStream_t st) {
  if (heads == 0 || C == 0) return hipSuccess;
  const dim3 grid(unsigned((C * rank + 255) / 256), unsigned(heads));
  if (cdt == KVC_BF16)
    hipLaunchKernelGGL((project_centres_kernel<bf16_t>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(cent),
                       basis, C, dim, rank, proj);
  else
    hipLaunchKernelGGL((project_centres_kernel<float>), grid, dim3(256), 0, st, static_cast<const float*>(cent), basis,
                       C, dim, rank, proj);
  return hipGetLastError();
}

hipError_t launch_attend_lowdim(int heads, int64_t n_q, int dim, int rank, const uint16_t* q_proj,
                                const float* basis_v, const SegList& segs, int k_bits, int v_bits, int group,
                                int n_split, float* out, float* lse, hipStream_t st) {
  if (heads == 0 || n_q == 0) return hipSuccess;
  if (segs.total_tiles == 0) { k_bits = v_bits = 2; group = 16; }
  AttendParams p;
  p.q = q_proj;
  p.n_q = n_q;
  p.heads = heads;
  p.n_split = n_split;
  p.scale_log2 = 1.4426950408889634f / sqrtf(float(dim));
  p.out = out;
  p.lse = lse;
  p.basis_v = basis_v;
  if (dim != 128) return hipErrorInvalidValue;
  if (rank == 32) return pick_bits<32, float, true, 128>(p, segs, k_bits, v_bits, group, st);
  if (rank == 64) return pick_bits<64, float, true, 128>(p, segs, k_bits, v_bits, group, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
