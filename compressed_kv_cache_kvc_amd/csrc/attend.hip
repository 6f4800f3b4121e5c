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
//      the probabilities feed the second product straight from registers).
//      Dequantization runs two channels at a time in packed fp16: the hardware's
//      fp4/fp8 conversions turn a pair of codes into exact small integers, one
//      fused multiply-add applies (scale, zero) and one add the centre, read from
//      an fp16 copy of the centre table.  The pairs are channels (c, c+2) of each
//      block of four, so the tiles, the table and the queries all hold the
//      channels of a block in the order 0, 2, 1, 3 (the contraction does not care;
//      the output rows are put back in order when written);
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
  const uint16_t* q_lo;   // low-dim path: fp16 remainders of the reduced queries [H][n_q][DQ]
  int64_t n_q;
  int heads;
  int n_split;
  float scale_log2;       // log2(e) / sqrt(head dim)
  float* out;             // [n_split][H][n_q][DOUT]
  float* lse;             // [n_split][H][n_q]
  const float* basis_v;   // low-dim: [H][DOUT][DQ]
  const float* u_psac;    // logit compensation: [H][DQ][8] principal query directions
};

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Channel held at position p of a tile row, centre-table row or query fragment:
// the middle two channels of every block of four are swapped (an involution).
__host__ __device__ constexpr int tile_channel(int p) { return (p & ~3) | ((p & 1) << 1) | ((p >> 1) & 1); }

// Codes of the channel pairs of one thread's chunk, spread so that each pair
// converts with one instruction.  Pair j (tile positions 2j, 2j+1) holds channels
// 4*(j/2) + j%2 and that + 2.  2-bit codes go to nibbles and convert as fp4 e2m1,
// whose codes 0..3 are 0, 0.5, 1, 1.5 (times the power-of-two scale 2); 4-bit
// codes go to bytes and convert as fp8 e4m3, whose codes 0..15 are q * 2^-9 (times
// the scale 2^9).  Either way the result is the integer code, exactly, in fp16.
template <int NB, int CH>
struct CodePairs;

template <int CH>
struct CodePairs<2, CH> {
  static_assert(CH <= 16, "2-bit chunk fits one word");
  uint32_t a, b;   // a: nibble n holds code 2n; b: code 2n+1
  __device__ __forceinline__ explicit CodePairs(uint32_t w) : a(w & 0x33333333u), b((w >> 2) & 0x33333333u) {}
  __device__ __forceinline__ h2 pair(int j) const {
    const uint32_t src = (j & 1) ? b : a;
    switch (j >> 1) {       // byte m = codes (4m, 4m+2) of a, (4m+1, 4m+3) of b
      case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, 2.0f, 0);
      case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, 2.0f, 1);
      case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, 2.0f, 2);
      default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, 2.0f, 3);
    }
  }
};

template <int CH>
struct CodePairs<4, CH> {
  static constexpr int NW = (CH * 4 + 31) / 32;
  uint32_t a[NW], b[NW];   // byte k of a[i]: code 8i + 2k; of b[i]: code 8i + 2k + 1
  template <typename W>
  __device__ __forceinline__ explicit CodePairs(W w) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t x = uint32_t(w >> (32 * i));
      a[i] = x & 0x0F0F0F0Fu;
      b[i] = (x >> 4) & 0x0F0F0F0Fu;
    }
  }
  __device__ __forceinline__ h2 pair(int j) const {
    const int m = j >> 1;   // word m/2 of the spread codes, 16-bit half m%2
    const uint32_t src = (j & 1) ? b[m >> 1] : a[m >> 1];
    if (m & 1) return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 512.0f, true);
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 512.0f, false);
  }
};

// 16-bit residuals (fp16, stored in channel order): word k of the chunk holds
// channels 2k, 2k+1; pair j is gathered from the two words of its block of four.
struct Code32 {
  uint4 lo, hi;
};
template <int CH>
struct CodePairs<16, CH> {
  uint32_t w[CH / 2];
  __device__ __forceinline__ explicit CodePairs(uint4 v) {
    static_assert(CH == 8, "16-byte chunk");
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  __device__ __forceinline__ explicit CodePairs(const Code32& v) {
    static_assert(CH == 16, "32-byte chunk");
    w[0] = v.lo.x; w[1] = v.lo.y; w[2] = v.lo.z; w[3] = v.lo.w;
    w[4] = v.hi.x; w[5] = v.hi.y; w[6] = v.hi.z; w[7] = v.hi.w;
  }
  __device__ __forceinline__ h2 pair(int j) const {
    const int m = j >> 1;     // block of four channels: words 2m (4m, 4m+1) and 2m+1 (4m+2, 4m+3)
    return as_h2(__builtin_amdgcn_perm(w[2 * m + 1], w[2 * m], (j & 1) ? 0x07060302u : 0x05040100u));
  }
};

// (fp16(c.lo * sc + t0), fp16(c.hi * sc + t1)) for fp32 t and sc and a packed fp16
// pair c, each with a single rounding: v_fma_mix{lo,hi}_f16 with the fp16 source c
// and the fp32 sources sc and t, computed in fp32 and rounded once to the
// destination half.
__device__ __forceinline__ uint32_t round_add_f16x2(float t0, float t1, uint32_t c, float sc) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %2, %3, %1 op_sel_hi:[1,0,0]" : "=&v"(r) : "v"(t0), "v"(c), "v"(sc));
  asm("v_fma_mixhi_f16 %0, %2, %3, %1 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(t1), "v"(c), "v"(sc));
  return r;
}

template <int NB>
using code_t = typename std::conditional<
    (NB > 16), Code32,
    typename std::conditional<(NB > 8), uint4, typename std::conditional<(NB > 4), uint64_t, uint32_t>::type>::type>::type;

template <int NB>
__device__ __forceinline__ code_t<NB> load_code_bits(const uint8_t* p) {
  if constexpr (NB == 1) return *p;
  else if constexpr (NB == 2) return *reinterpret_cast<const uint16_t*>(p);
  else if constexpr (NB == 4) return *reinterpret_cast<const uint32_t*>(p);
  else if constexpr (NB == 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return uint64_t(w.x) | (uint64_t(w.y) << 32);
  } else if constexpr (NB == 16) {
    return *reinterpret_cast<const uint4*>(p);
  } else {
    static_assert(NB == 32, "code chunk");
    return Code32{reinterpret_cast<const uint4*>(p)[0], reinterpret_cast<const uint4*>(p)[1]};
  }
}

// Transposing LDS read (ds_read_b64_tr_b16).  In each group of 16 lanes, lane
// 4a + b receives element b of the 8 bytes addressed by lanes a, a+4, a+8, a+12
// (as its elements 0..3): a 4x4 transpose of 16-bit values across lanes.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, v);
}

// SEQ (the rank-32 coefficient path): a tile's scores, softmax and values in one
// step, four wavefronts per SIMD (two workgroups per compute unit) instead of the
// two-tile overlap inside a wavefront.
template <int DQ, bool LOWDIM>
constexpr bool kSeqSchedule = LOWDIM && DQ == 32;

template <int DQ, int KB, int VB, int G, bool LOWDIM, int DOUT, bool PSAC = false>
__global__ __launch_bounds__(512, (kSeqSchedule<DQ, LOWDIM> ? 4 : 1)) void attend_kernel(AttendParams p, SegList segs) {
  constexpr bool SEQ = kSeqSchedule<DQ, LOWDIM>;
  static_assert(!PSAC || (!LOWDIM && !SEQ), "logit compensation: full-dimensional path only");
  constexpr int NK = SEQ ? 5 : 4;  // K tile buffers
  constexpr int KC = DQ / 16;     // k-chunks of the QK^T product
  constexpr int NDB = DQ / 32;    // 32-row blocks of O^T
  constexpr int ROWK = DQ + 8;    // padded LDS rows (fp16 elements)
  // V tile rows (keys) padded against bank conflicts of the transposing reads
  // (a row stride of 8, 16 or 48 dwords modulo 64; at DQ = 128 the LDS budget of
  // four K and five V buffers leaves room for 8)
  constexpr int ROWV = DQ == 128 ? 144 : DQ == 64 ? 96 : 32;
  constexpr int CH = DQ / 8;      // channels per dequantizing thread
  constexpr int KNB = CH * KB / 8, VNB = CH * VB / 8;
  static_assert(G % CH == 0, "a thread's channels must sit in one group");
  __shared__ __attribute__((aligned(16))) uint16_t sK[NK][64 * ROWK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[5][64 * ROWV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  // Workgroups go to the 8 XCDs in turn (workgroup i to XCD i mod 8). Renumber
  // them so that each XCD receives a contiguous range of (query block, split,
  // head) triples, query block fastest: the workgroups that read the same
  // history tiles then share one XCD's L2.
  int qb, split, h;
  {
    const unsigned nb = gridDim.x, q8 = nb >> 3, r8 = nb & 7;
    const unsigned xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const unsigned logical = xcd < r8 ? xcd * (q8 + 1) + slot : r8 * (q8 + 1) + (xcd - r8) * q8 + slot;
    const unsigned nqb = unsigned((p.n_q + 255) >> 8);
    qb = int(logical % nqb);
    const unsigned rest = logical / nqb;
    split = int(rest % unsigned(p.n_split));
    h = int(rest / unsigned(p.n_split));
  }
  const int64_t qi = int64_t(qb) * 256 + wave * 32 + col;
  const bool q_ok = qi < p.n_q;

  // B operand Q^T in fp16, channels in tile order: bf16 queries convert exactly
  // inside the fp16 range; reduced queries arrive in fp16 and tile order already.
  // The factor c = log2(e)/sqrt(d) goes into the key tile (inside its one fp16
  // rounding), so that the score products are base-2 exponents already.
  const float c_sc = p.scale_log2;
  f16x8 qf[KC];
  // reduced queries are a sum hi + lo of two fp16 values: one fp16 rounding of
  // q' alone would put about 2^-12 of a logit into its error, which a logit
  // concentrated on few coefficients does not average out; the lo part costs one
  // more score product per k-chunk
  f16x8 ql[LOWDIM ? KC : 1];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (q_ok) w = *reinterpret_cast<const uint4*>(p.q + (int64_t(h) * p.n_q + qi) * DQ + kc * 16 + half * 8);
    if constexpr (!LOWDIM) {
      w = make_uint4(pack_f16x2(bf16_lo(w.x), bf16_lo(w.y)), pack_f16x2(bf16_hi(w.x), bf16_hi(w.y)),
                     pack_f16x2(bf16_lo(w.z), bf16_lo(w.w)), pack_f16x2(bf16_hi(w.z), bf16_hi(w.w)));
    } else {
      uint4 wl = make_uint4(0, 0, 0, 0);
      if (q_ok) wl = *reinterpret_cast<const uint4*>(p.q_lo + (int64_t(h) * p.n_q + qi) * DQ + kc * 16 + half * 8);
      ql[kc] = as_f16x8(wl);
    }
    qf[kc] = as_f16x8(w);
  }

  const int T = int(segs.total_tiles);           // at most 24 * 2^19 tiles
  const int t_begin = int(int64_t(T) * split / p.n_split);
  const int t_end = int(int64_t(T) * (split + 1) / p.n_split);

  // dequantization role: eight lanes per token, so that the code, metadata and
  // centre-row loads of a wavefront cover whole rows (coalesced)
  const int dk = (wave << 3) | (lane >> 3);   // token within the tile
  const int dg = lane & 7;                    // channel group [dg*CH, dg*CH + CH)

  // a thread's centre chunk: CH fp16 values from the table, as CH/2 channel pairs
  constexpr int CWD = CH / 2;
  static_assert(CWD == 2 || CWD % 4 == 0, "centre chunk");

  // A cursor holds the segment of the tiles it walks over, with its arrays
  // already offset to this workgroup's head; being wave-uniform its fields live
  // in scalar registers, and are reloaded only when the cursor crosses into the
  // next segment, so no scalar memory load sits in the tile loop otherwise.
  // Three cursors walk the tiles (ids two tiles ahead, data one ahead of the
  // dequantization, and the tile being scored); each holds the segment it is in
  // and only the arrays it reads, already offset to this workgroup's head.  Being
  // wave-uniform their fields live in scalar registers and are reloaded only when
  // a cursor crosses into the next segment.
  struct Span {
    int si, tile_begin, tile_end, n_tokens;
  };
  struct IdCur {
    Span s;
    const uint8_t *k_ids, *v_ids;
  };
  struct DataCur {
    Span s;
    const uint8_t *k_codes, *v_codes;
    const uint32_t *k_meta, *v_meta;
    const uint16_t *k_tab, *v_tab;
    const uint16_t* psac;
  };
  auto span_load = [&](Span& c, int si) {
    c.si = si;
    c.tile_begin = int(segs.s[si].tile_begin);
    c.tile_end = int(si + 1 < segs.n ? segs.s[si + 1].tile_begin : segs.total_tiles);
    c.n_tokens = int(segs.s[si].n_tokens);
  };
  auto ids_load = [&](IdCur& c, int si) {
    span_load(c.s, si);
    const SegDev& s = segs.s[si];
    const int64_t hn = int64_t(h) * s.n_tokens;
    c.k_ids = s.k_ids + hn;
    c.v_ids = s.v_ids + hn;
  };
  auto data_load = [&](DataCur& c, int si) {
    span_load(c.s, si);
    const SegDev& s = segs.s[si];
    const int64_t hn = int64_t(h) * s.n_tokens;
    c.k_codes = s.k_codes + hn * (DQ * KB / 8);
    c.v_codes = s.v_codes + hn * (DQ * VB / 8);
    c.k_meta = s.k_meta + hn * (DQ / G);
    c.v_meta = s.v_meta + hn * (DQ / G);
    const int64_t hc = int64_t(h) * s.n_centroids * DQ;
    c.k_tab = s.k_tab + hc;
    c.v_tab = s.v_tab + hc;
    if constexpr (PSAC) c.psac = s.psac + hn * 8;
  };
  auto ids_seek = [&](IdCur& c, int t) {
    while (t >= c.s.tile_end) ids_load(c, c.s.si + 1);
  };
  auto data_seek = [&](DataCur& c, int t) {
    while (t >= c.s.tile_end) data_load(c, c.s.si + 1);
  };
  auto span_seek = [&](Span& c, int t) {
    while (t >= c.tile_end) span_load(c, c.si + 1);
  };
  // token (within the head) of this thread's row in tile t, clamped into the
  // segment so that every load is in bounds; rows past the end read real
  // (finite) data and are masked out of the softmax
  auto row_of = [&](const Span& c, int t) -> uint32_t {
    const int j0 = (t - c.tile_begin) * 64;
    const int last = c.n_tokens - 1;
    return uint32_t(j0 + dk < last ? j0 + dk : last);
  };

  // ---- register pipeline (raw loaded words; converted only at dequantization)
  int kid_n = 0, vid_n = 0;       // ids of the tile to load next (t+1)
  code_t<KNB> kc_r{};
  code_t<VNB> vc_r{};
  // metadata words (scale | zero << 16); 16-bit residuals keep (1, 0)
  uint32_t km_r = KB == 16 ? 0x3c00u : 0u, vm_r = VB == 16 ? 0x3c00u : 0u;
  uint4 pc_r = make_uint4(0, 0, 0, 0);   // kept key-error coefficients of the token (dg == 7 lanes)
  uint32_t kcw[CWD], vcw[CWD];

  auto load_ids = [&](const IdCur& c, int t, int& ki, int& vi) {
    const uint32_t j = row_of(c.s, t);
    ki = c.k_ids[j];
    vi = c.v_ids[j];
  };
  auto load_data = [&](const DataCur& c, int t, int ki, int vi) {
    const uint32_t j = row_of(c.s, t);
    kc_r = load_code_bits<KNB>(c.k_codes + (j * uint32_t(DQ * KB / 8) + uint32_t(dg * KNB)));
    vc_r = load_code_bits<VNB>(c.v_codes + (j * uint32_t(DQ * VB / 8) + uint32_t(dg * VNB)));
    if constexpr (PSAC)
      if (dg == 7) pc_r = *reinterpret_cast<const uint4*>(c.psac + j * 8u);
    if constexpr (KB != 16) km_r = c.k_meta[j * uint32_t(DQ / G) + uint32_t((dg * CH) / G)];
    if constexpr (VB != 16) vm_r = c.v_meta[j * uint32_t(DQ / G) + uint32_t((dg * CH) / G)];
    const uint16_t* kp = c.k_tab + (uint32_t(ki) * DQ + dg * CH);
    const uint16_t* vp = c.v_tab + (uint32_t(vi) * DQ + dg * CH);
    if constexpr (CWD == 2) {
      const uint2 a = *reinterpret_cast<const uint2*>(kp), b = *reinterpret_cast<const uint2*>(vp);
      kcw[0] = a.x; kcw[1] = a.y; vcw[0] = b.x; vcw[1] = b.y;
    } else {
#pragma unroll
      for (int i = 0; i < CWD / 4; ++i) {
        const uint4 a = reinterpret_cast<const uint4*>(kp)[i], b = reinterpret_cast<const uint4*>(vp)[i];
        kcw[4 * i] = a.x; kcw[4 * i + 1] = a.y; kcw[4 * i + 2] = a.z; kcw[4 * i + 3] = a.w;
        vcw[4 * i] = b.x; vcw[4 * i + 1] = b.y; vcw[4 * i + 2] = b.z; vcw[4 * i + 3] = b.w;
      }
    }
  };

  // (scale, scale) and (zero, zero) of a metadata word (scale | zero << 16)
  auto scale2 = [](uint32_t m) { return as_h2(__builtin_amdgcn_perm(m, m, 0x01000100u)); };
  auto zero2 = [](uint32_t m) { return as_h2(__builtin_amdgcn_perm(m, m, 0x03020302u)); };

  auto store_tile = [&](int kbuf, int vbuf) {
    // keys, scaled by c: c*(q*s + z) in fp32 (q*(c*s) + c*z), then one rounding of
    // the sum with c times the centre to fp16; the key tile's rounding error moves
    // every logit, so keys get the single-rounding form
    const CodePairs<KB, CH> kq(kc_r);
    const h2 km = as_h2(km_r);
    const float ks = float(km[0]) * c_sc, kz = float(km[1]) * c_sc;
    uint32_t kw[CH / 2];
#pragma unroll
    for (int j = 0; j < CH / 2; ++j) {
      const h2 c = kq.pair(j);
      kw[j] = round_add_f16x2(fmaf(float(c[0]), ks, kz), fmaf(float(c[1]), ks, kz), kcw[j], c_sc);
    }
    uint16_t* kdst = &sK[kbuf][dk * ROWK + dg * CH];
    if constexpr (CH == 16) {
      reinterpret_cast<uint4*>(kdst)[0] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
      reinterpret_cast<uint4*>(kdst)[1] = make_uint4(kw[4], kw[5], kw[6], kw[7]);
    } else if constexpr (CH == 8) {
      reinterpret_cast<uint4*>(kdst)[0] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
    } else {
      static_assert(CH == 4, "channels per thread");
      reinterpret_cast<uint2*>(kdst)[0] = make_uint2(kw[0], kw[1]);
    }
    // the token's compensation coefficients go to the row's 8 padding columns
    if constexpr (PSAC)
      if (dg == 7) *reinterpret_cast<uint4*>(&sK[kbuf][dk * ROWK + DQ]) = pc_r;
    // values: (q*s + z) and the centre add in packed fp16 (two roundings; an
    // error in a value moves only its own share of the output)
    const CodePairs<VB, CH> vq(vc_r);
    const h2 vs = scale2(vm_r), vz = zero2(vm_r);
    uint32_t vw[CH / 2];
#pragma unroll
    for (int j = 0; j < CH / 2; ++j) vw[j] = as_u32(__builtin_elementwise_fma(vq.pair(j), vs, vz) + as_h2(vcw[j]));
    uint16_t* vdst = &sV[vbuf][dk * ROWV + dg * CH];
    if constexpr (CH == 16) {
      reinterpret_cast<uint4*>(vdst)[0] = make_uint4(vw[0], vw[1], vw[2], vw[3]);
      reinterpret_cast<uint4*>(vdst)[1] = make_uint4(vw[4], vw[5], vw[6], vw[7]);
    } else if constexpr (CH == 8) {
      reinterpret_cast<uint4*>(vdst)[0] = make_uint4(vw[0], vw[1], vw[2], vw[3]);
    } else {
      reinterpret_cast<uint2*>(vdst)[0] = make_uint2(vw[0], vw[1]);
    }
  };

  // reference maximum of the row (log2 units), a sum of two fp16 values hi + lo
  // that enters the scores through the bias product below; set from the first tile
  float m_run = 0.f;
  float l_run = 0.f;              // this lane's share of the running sum
  f32x16 o[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[b][v] = 0.f;

  auto clamp_t = [&](int t) { return t < t_end ? t : t_end - 1; };

  // Bias product: one more v_mfma_f32_32x32x16_f16 per 32 keys subtracts the
  // reference maximum from the scores.  Upper-half lanes (k = 8..15) hold 1, 1 in the
  // A operand and -m_hi, -m_lo of the lane's query in the B operand.  With logit
  // compensation (kept key error along the principal query directions) the
  // lower-half lanes (k = 0..7) hold the key rows' 8 coefficients (A, from the K
  // row's padding columns) and c * U^T q (B, fp32 then fp16); otherwise their B
  // entries are zero.
  __shared__ __attribute__((aligned(16))) uint32_t sOne[4];
  if (PSAC && tid == 0) {
    sOne[0] = 0x3c003c00u; sOne[1] = 0u; sOne[2] = 0u; sOne[3] = 0u;
  }
  f16x8 qpf = as_f16x8(make_uint4(0, 0, 0, 0));
  if constexpr (PSAC) {
    if (q_ok && half == 0) {
      const uint16_t* qrow = p.q + (int64_t(h) * p.n_q + qi) * DQ;
      const float* U = p.u_psac + int64_t(h) * DQ * 8;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < DQ; ++c) {
        const float qc = __uint_as_float(uint32_t(qrow[c]) << 16);
        const float4 u0 = *reinterpret_cast<const float4*>(U + c * 8);
        const float4 u1 = *reinterpret_cast<const float4*>(U + c * 8 + 4);
        acc[0] = fmaf(u0.x, qc, acc[0]); acc[1] = fmaf(u0.y, qc, acc[1]);
        acc[2] = fmaf(u0.z, qc, acc[2]); acc[3] = fmaf(u0.w, qc, acc[3]);
        acc[4] = fmaf(u1.x, qc, acc[4]); acc[5] = fmaf(u1.y, qc, acc[5]);
        acc[6] = fmaf(u1.z, qc, acc[6]); acc[7] = fmaf(u1.w, qc, acc[7]);
      }
      qpf = as_f16x8(make_uint4(pack_f16x2(c_sc * acc[0], c_sc * acc[1]), pack_f16x2(c_sc * acc[2], c_sc * acc[3]),
                                pack_f16x2(c_sc * acc[4], c_sc * acc[5]), pack_f16x2(c_sc * acc[6], c_sc * acc[7])));
    }
  }
  f16x8 qbias = qpf;                                         // B operand of the bias product
  const f16x8 a_one = as_f16x8(make_uint4(0x3c003c00u, 0u, 0u, 0u));
  auto bias_qk = [&](int kbuf_, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f16x8 a = a_one;
      if constexpr (PSAC) {
        const uint32_t* src = half ? sOne : reinterpret_cast<const uint32_t*>(&sK[kbuf_][(kb * 32 + col) * ROWK + DQ]);
        a = as_f16x8(*reinterpret_cast<const uint4*>(src));
      }
      sacc[kb] = mfma32h(a, qbias, sacc[kb]);
    }
  };

  // S^T = c K_hat Q^T - m of the K tile in buffer kb_, keys [0, 32) and [32, 64)
  auto qk = [&](int kb_, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f16x8 a = as_f16x8(*reinterpret_cast<const uint4*>(&sK[kb_][(kb * 32 + col) * ROWK + kc * 16 + half * 8]));
        sacc[kb] = mfma32h(a, qf[kc], sacc[kb]);
        if constexpr (LOWDIM) sacc[kb] = mfma32h(a, ql[kc], sacc[kb]);
      }
    bias_qk(kb_, sacc);
  };

  // mask the keys past the end of the segment: this lane's rows are 4*half +
  // (its register rows), tested against a wave-uniform mask of the valid keys
  auto mask_tail = [&](f32x16 (&sacc)[2], int nvalid) {
    if (nvalid < 64) {
      const uint64_t mine = ((uint64_t(1) << nvalid) - 1) >> (4 * half);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (!((mine >> (kb * 32 + 8 * (v / 4) + (v % 4))) & 1)) sacc[kb][v] = -INFINITY;
    }
  };

  // Software pipeline over tiles: while tile t's exponentials are computed the
  // matrix cores already form tile t+1's scores, and while tile t's values are
  // multiplied tile t+3 is dequantized.  K tiles live in four buffers and V tiles
  // in five, so that one barrier per two tiles suffices: a tile is written at
  // least two steps before it is read, and a buffer is rewritten at least two
  // steps after its last read (the barriers follow every second step).
  IdCur cur_ids;
  DataCur cur_data;
  Span cur_comp;
  f32x16 sa[2], sb[2];
  if (t_begin < t_end) {
    data_load(cur_data, 0);
    data_seek(cur_data, t_begin);
    ids_load(cur_ids, 0);
    ids_seek(cur_ids, t_begin);
    span_load(cur_comp, 0);
    span_seek(cur_comp, t_begin);
    int k0, v0;
    load_ids(cur_ids, t_begin, k0, v0);
    load_data(cur_data, t_begin, k0, v0);
    ids_seek(cur_ids, clamp_t(t_begin + 1));
    load_ids(cur_ids, clamp_t(t_begin + 1), kid_n, vid_n);
    store_tile(0, 0);
    data_seek(cur_data, clamp_t(t_begin + 1));
    load_data(cur_data, clamp_t(t_begin + 1), kid_n, vid_n);
    ids_seek(cur_ids, clamp_t(t_begin + 2));
    load_ids(cur_ids, clamp_t(t_begin + 2), kid_n, vid_n);
    store_tile(1, 1);
    data_seek(cur_data, clamp_t(t_begin + 2));
    load_data(cur_data, clamp_t(t_begin + 2), kid_n, vid_n);
    ids_seek(cur_ids, clamp_t(t_begin + 3));
    load_ids(cur_ids, clamp_t(t_begin + 3), kid_n, vid_n);
    store_tile(2, 2);
  }
  __syncthreads();
  if constexpr (!SEQ)
    if (t_begin < t_end) qk(0, sa);

  int vbuf = 0;                     // V buffer of tile t; tile t+3 goes to (vbuf + 3) % 5
  int kbuf = 0;                     // K buffer of tile t; tile t+3 goes to (kbuf + 3) % NK
  constexpr int NQK = 2 * KC;       // score products per tile
  constexpr int NPV = 4 * NDB;      // value products per tile
  constexpr int PPM = 16 / NQK;     // exponential pairs between two score products
  static_assert(16 % NQK == 0 && CH % NPV == 0, "work per product");
  constexpr int IPM = CH / NPV;     // dequantization pairs between two value products

  // One tile step.  The matrix products of the step (tile t+1's scores, then tile
  // t's values) are issued one at a time, each followed by its share of the vector
  // work (tile t's exponentials, then tile t+3's dequantization) and preceded
  // three products earlier by the LDS read of its operand; scheduling fences keep this
  // order, so the matrix cores and the vector unit work side by side.
  auto step = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    // the K tile scored in this step: t+1, or t itself in the SEQ schedule
    const int kread = SEQ ? kbuf : (kbuf == NK - 1 ? 0 : kbuf + 1);
    auto frag = [&](int f) -> f16x8 {
      if (f < NQK) {          // K fragment: keys (f & 1)*32 + col, channels (f >> 1)*16 + half*8
        return as_f16x8(*reinterpret_cast<const uint4*>(
            &sK[kread][((f & 1) * 32 + col) * ROWK + (f >> 1) * 16 + half * 8]));
      }
      // V^T fragment for product i = f - NQK: dims (i % NDB)*32 + [0, 32), keys of
      // chunk i / NDB in the order of the probabilities (bits 2 and 3 of the key
      // offset swapped), read from the row-major V tile with two transposing
      // loads: lane s supplies key row 8*half_call + 4*(s >> 5) + ((s >> 2) & 3) of
      // the chunk and four dims from 16*((s >> 4) & 1) + 4*(s & 3); the hardware
      // hands lane l the four keys of its dim l % 32
      const int i = f - NQK;
      const uint16_t* base = &sV[vbuf][((i / NDB) * 16 + 4 * (lane >> 5) + ((lane >> 2) & 3)) * ROWV +
                                       (i % NDB) * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)];
      const uint2 lo = lds_read_tr16(base), hi = lds_read_tr16(base + 8 * ROWV);
      return as_f16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    // operand reads run FA products ahead of their use (a ring of FA + 1
    // fragments): four with 2-bit values in the overlapped schedule, three with
    // wider values (whose code registers leave no room for a fifth fragment) and
    // in the sequential schedule, two with logit compensation (the token's kept
    // coefficients take the registers)
    constexpr int FA = PSAC ? 2 : ((VB == 2 && !SEQ) ? 4 : 3), FR = FA + 1;
    f16x8 fr[FR];
#pragma unroll
    for (int f = 0; f < FA; ++f) fr[f] = frag(f);
    {
      const int t3 = clamp_t(t + 3), t4 = clamp_t(t + 4);
      data_seek(cur_data, t3);
      load_data(cur_data, t3, kid_n, vid_n);
      ids_seek(cur_ids, t4);
      load_ids(cur_ids, t4, kid_n, vid_n);
    }
    span_seek(cur_comp, t);
    const int nvalid_left = cur_comp.n_tokens - (t - cur_comp.tile_begin) * 64;
    if constexpr (!SEQ) mask_tail(cur, nvalid_left >= 64 ? 64 : nvalid_left);

    // tile t's exponentials (the scores are c*q.k - m already), one pair at a time,
    // as fp16 probabilities; the row sum is taken over the same rounded values
    uint32_t pw[16];
    float psum = 0.f;
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    auto exp_pair = [&](int k) {
      const int kb = k >> 3, v = 2 * (k & 7);
      const float e0 = __builtin_amdgcn_exp2f(cur[kb][v]);
      const float e1 = __builtin_amdgcn_exp2f(cur[kb][v + 1]);
      pw[k] = pack_f16x2(e0, e1);
      psum = __builtin_amdgcn_fdot2(as_h2(pw[k]), ones, psum, false);
    };
    // The reference maximum is raised lazily: a tile whose probabilities (against
    // the current m) sum to more than 2^8 in some row, and the first tile, take this
    // branch, which moves m of every row to the tile's maximum where that lies above
    // m (the first tile: always), shifts the scores of this tile and of the next
    // (already formed with the old m), rescales the output accumulator and the sum,
    // and recomputes the exponentials.  A row's probabilities are thus at most 2^8
    // each, so fp16 holds them.
    auto rescale = [&](bool first) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, cur[kb][v]);
      // the other half of the row sits in lane l ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float target = m_run + (first ? (mx > -INFINITY ? mx : 0.f) : (mx > 0.f ? mx : 0.f));
      const _Float16 m_hi = (_Float16)target;
      const _Float16 m_lo = (_Float16)(target - (float)m_hi);
      const float m_new = (float)m_hi + (float)m_lo;
      const float delta = m_new - m_run;
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < NDB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[b][v] *= alpha;
      }
      m_run = m_new;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) cur[kb][v] -= delta;
      if constexpr (!SEQ) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) nxt[kb][v] -= delta;
      }
      if (half) {
        const h2 nm = {(_Float16)(-m_hi), (_Float16)(-m_lo)};
        qbias = as_f16x8(make_uint4(as_u32(nm), 0u, 0u, 0u));
      }
      psum = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) exp_pair(k);
    };
    f16x8 pf[4];

    // tile t+3's dequantization, one channel pair at a time: item j < CH/2 is key
    // pair j (keys: one rounding of fp32 q*s + z plus the centre), item CH/2 + j
    // value pair j (packed fp16)
    const int vstore = vbuf >= 2 ? vbuf - 2 : vbuf + 3;
    const int kstore = kbuf + 3 < NK ? kbuf + 3 : kbuf + 3 - NK;
    uint32_t kw[CH / 2], vw[CH / 2];
    auto dq_item = [&](int j, const CodePairs<KB, CH>& kq, float ks, float kz, const CodePairs<VB, CH>& vq, h2 vs,
                       h2 vz) {
      if (j < CH / 2) {
        const h2 c = kq.pair(j);
        kw[j] = round_add_f16x2(fmaf(float(c[0]), ks, kz), fmaf(float(c[1]), ks, kz), kcw[j], c_sc);
        uint16_t* kdst = &sK[kstore][dk * ROWK + dg * CH];
        if constexpr (CH == 4) {
          if (j == 1) reinterpret_cast<uint2*>(kdst)[0] = make_uint2(kw[0], kw[1]);
        } else if ((j & 3) == 3) {
          reinterpret_cast<uint4*>(kdst)[j >> 2] = make_uint4(kw[j - 3], kw[j - 2], kw[j - 1], kw[j]);
        }
        if constexpr (PSAC)
          if (j == CH / 2 - 1 && dg == 7) *reinterpret_cast<uint4*>(&sK[kstore][dk * ROWK + DQ]) = pc_r;
      } else {
        const int jj = j - CH / 2;
        vw[jj] = as_u32(__builtin_elementwise_fma(vq.pair(jj), vs, vz) + as_h2(vcw[jj]));
        uint16_t* vdst = &sV[vstore][dk * ROWV + dg * CH];
        if constexpr (CH == 4) {
          if (jj == 1) reinterpret_cast<uint2*>(vdst)[0] = make_uint2(vw[0], vw[1]);
        } else if ((jj & 3) == 3) {
          reinterpret_cast<uint4*>(vdst)[jj >> 2] = make_uint4(vw[jj - 3], vw[jj - 2], vw[jj - 1], vw[jj]);
        }
      }
    };

    if constexpr (SEQ) {
      // tile t's scores, then its softmax and exponentials
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        fr[(i + FA) % FR] = frag(i + FA);
        if (i < 2)
          cur[i] = mfma32h(fr[i % FR], qf[0], f32x16{});
        else
          cur[i & 1] = mfma32h(fr[i % FR], qf[i >> 1], cur[i & 1]);
        cur[i & 1] = mfma32h(fr[i % FR], ql[i >> 1], cur[i & 1]);   // SEQ is a low-dim schedule
      }
      bias_qk(kbuf, cur);
      mask_tail(cur, nvalid_left >= 64 ? 64 : nvalid_left);
#pragma unroll
      for (int k = 0; k < 16; ++k) exp_pair(k);
    } else {
      // the score products and exponentials run at raised wave priority: the SIMD
      // then favours the wavefront whose matrix products feed the next tile
      // (measured +2% over equal priorities)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        fr[(i + FA) % FR] = frag(i + FA);
        if (i < 2)
          nxt[i] = mfma32h(fr[i % FR], qf[0], f32x16{});
        else
          nxt[i & 1] = mfma32h(fr[i % FR], qf[i >> 1], nxt[i & 1]);
        if constexpr (LOWDIM) nxt[i & 1] = mfma32h(fr[i % FR], ql[i >> 1], nxt[i & 1]);
#pragma unroll
        for (int u = 0; u < PPM; ++u) exp_pair(i * PPM + u);
        __builtin_amdgcn_sched_barrier(0);
      }
      bias_qk(kread, nxt);
      __builtin_amdgcn_s_setprio(0);
    }
    if (__any(!(psum <= 256.f)) || t == t_begin) rescale(t == t_begin);
    l_run += psum;
#pragma unroll
    for (int c = 0; c < 4; ++c) pf[c] = as_f16x8(make_uint4(pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]));

    const CodePairs<KB, CH> kq(kc_r);
    const h2 kmh = as_h2(km_r);
    const float ks = float(kmh[0]) * c_sc, kz = float(kmh[1]) * c_sc;
    const CodePairs<VB, CH> vq(vc_r);
    const h2 vs = scale2(vm_r), vz = zero2(vm_r);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (NQK + i + FA < NQK + NPV) fr[(NQK + i + FA) % FR] = frag(NQK + i + FA);
      o[i % NDB] = mfma32h(fr[(NQK + i) % FR], pf[i / NDB], o[i % NDB]);
#pragma unroll
      for (int u = 0; u < IPM; ++u) dq_item(i * IPM + u, kq, ks, kz, vq, vs, vz);
      __builtin_amdgcn_sched_barrier(0);
    }
    vbuf = vbuf == 4 ? 0 : vbuf + 1;
    kbuf = kbuf == NK - 1 ? 0 : kbuf + 1;
  };
  for (int t = t_begin; t < t_end; t += 2) {
    if constexpr (SEQ) {
      step(t, sa, sa);
      if (t + 1 < t_end) step(t + 1, sa, sa);
    } else {
      step(t, sa, sb);
      if (t + 1 < t_end) step(t + 1, sb, sa);
    }
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
              make_float4(o[b][4 * g4] * inv, o[b][4 * g4 + 2] * inv, o[b][4 * g4 + 1] * inv, o[b][4 * g4 + 3] * inv);
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
        // row 8*(v/4) + 4*half + v%4 is held by this lane, the other half's by the
        // partner; rows are tile positions, coefficients are stored by channel
        coef[tile_channel(b * 32 + 8 * (v / 4) + (v % 4))] = half == 0 ? mine : other;
        coef[tile_channel(b * 32 + 8 * (v / 4) + 4 + (v % 4))] = half == 0 ? other : mine;
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

// fp32 queries: one wavefront per (query, head), fp32 dequantization and softmax
// throughout.  The lanes take the keys of the history in turn (key j of a segment
// on lane j mod 64), so that a wavefront's loads of codes, metadata and ids cover
// consecutive tokens; each lane keeps its own running maximum, sum and output
// row, and the 64 partial results are combined at the end (rescaled to the
// common maximum and added across the lanes).  The query row is read from LDS
// at one address per instruction (a broadcast).
template <int D, int KB, int VB, int G>
__global__ __launch_bounds__(256) void attend_f32_kernel(const float* __restrict__ q, int64_t n_q,
                                                         SegList segs, float scale, float* __restrict__ out,
                                                         float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) float sq[4][D];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t qi = int64_t(blockIdx.x) * 4 + wave;
  const int h = blockIdx.y;
  if (qi >= n_q) return;                       // wave-uniform; no barrier follows
  const float* qr = q + (int64_t(h) * n_q + qi) * D;
  for (int c = lane; c < D; c += 64) sq[wave][c] = qr[c];
  __builtin_amdgcn_wave_barrier();             // LDS writes of a wavefront complete in order
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  float m = -INFINITY, l = 0.f;
  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.f;
  for (int si = 0; si < segs.n; ++si) {
    const SegDev& s = segs.s[si];
    const float* kcent = static_cast<const float*>(s.k_cent) + int64_t(h) * s.n_centroids * D;
    const float* vcent = static_cast<const float*>(s.v_cent) + int64_t(h) * s.n_centroids * D;
    for (int64_t j = lane; j < s.n_tokens; j += 64) {
      const int64_t tok = int64_t(h) * s.n_tokens + j;
      const float* kc = kcent + int64_t(s.k_ids[tok]) * D;
      const uint8_t* kcode = s.k_codes + tok * (D * KB / 8);
      float dot = 0.f;
#pragma unroll 4
      for (int i = 0; i < D; ++i) {
        const uint32_t w = s.k_meta[tok * (D / G) + i / G];
        const float code = float((kcode[i / (8 / KB)] >> (KB * (i % (8 / KB)))) & ((1 << KB) - 1));
        const float kh = kc[i] + fmaf(code, f16_bits_to_f32(w & 0xffffu), f16_bits_to_f32(w >> 16));
        dot = fmaf(sq[wave][i], kh, dot);
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
  // combine the lanes: common maximum, then sums of the rescaled partials
  float mw = m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mw = fmaxf(mw, __shfl_xor(mw, off, 64));
  const float f = (m == -INFINITY) ? 0.f : expf(m - mw);   // a lane without keys adds nothing
  l *= f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* dst = out + (int64_t(h) * n_q + qi) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    float a = acc[i] * f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off, 64);
    if (lane == (i & 63)) dst[i] = a * inv;
  }
  if (lane == 0) lse[int64_t(h) * n_q + qi] = l > 0.f ? mw + logf(l) : -INFINITY;
}

// Reduced queries q' = U^T q (fp32 accumulation, fp16 result in tile channel order).
// One thread per query, R accumulators; the head's basis is staged in LDS and
// read by all lanes at the same address (broadcast).
template <int D, int R>
__global__ __launch_bounds__(256) void project_queries_kernel(const uint16_t* __restrict__ q,
                                                              const float* __restrict__ basis, int64_t n_q,
                                                              uint16_t* __restrict__ qp) {
  __shared__ __attribute__((aligned(16))) float sU[D * R];
  const int h = blockIdx.y;
  const float* Uh = basis + int64_t(h) * D * R;
  for (int i = threadIdx.x; i < D * R / 4; i += 256)
    reinterpret_cast<float4*>(sU)[i] = reinterpret_cast<const float4*>(Uh)[i];
  __syncthreads();
  const int64_t qi = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (qi >= n_q) return;
  const uint16_t* qr = q + (int64_t(h) * n_q + qi) * D;
  float acc[R];
#pragma unroll
  for (int k = 0; k < R; ++k) acc[k] = 0.f;
  for (int c8 = 0; c8 < D / 8; ++c8) {
    const uint4 w = reinterpret_cast<const uint4*>(qr)[c8];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xv = (e & 1) ? bf16_hi(ww[e / 2]) : bf16_lo(ww[e / 2]);
      const float4* Urow = reinterpret_cast<const float4*>(&sU[(c8 * 8 + e) * R]);
#pragma unroll
      for (int k4 = 0; k4 < R / 4; ++k4) {
        const float4 u = Urow[k4];
        acc[4 * k4 + 0] = fmaf(xv, u.x, acc[4 * k4 + 0]);
        acc[4 * k4 + 1] = fmaf(xv, u.y, acc[4 * k4 + 1]);
        acc[4 * k4 + 2] = fmaf(xv, u.z, acc[4 * k4 + 2]);
        acc[4 * k4 + 3] = fmaf(xv, u.w, acc[4 * k4 + 3]);
      }
    }
  }
  // position p holds coefficient tile_channel(p); pairs of positions per word.
  // hi = fp16(q'), lo = fp16(q' - hi) (the difference is exact in fp32)
  uint32_t* dst = reinterpret_cast<uint32_t*>(qp + (int64_t(h) * n_q + qi) * R);
  uint32_t* dlo = reinterpret_cast<uint32_t*>(qp + (int64_t(gridDim.y) * n_q + int64_t(h) * n_q + qi) * R);
#pragma unroll
  for (int p2 = 0; p2 < R / 2; ++p2) {
    const float a0 = acc[tile_channel(2 * p2)], a1 = acc[tile_channel(2 * p2 + 1)];
    const uint32_t hw = pack_f16x2(a0, a1);
    const h2 hv = as_h2(hw);
    dst[p2] = hw;
    dlo[p2] = pack_f16x2(a0 - float(hv[0]), a1 - float(hv[1]));
  }
}

// Projected centres c' = U^T c (fp32 accumulation), as an fp16 table in tile
// channel order.
template <typename CT>
__global__ __launch_bounds__(256) void project_centres_kernel(const CT* __restrict__ cent, const float* __restrict__ basis,
                                                              int C, int D, int R, uint16_t* __restrict__ tab) {
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
  tab[(int64_t(h) * C + c) * R + tile_channel(k)] = static_cast<uint16_t>(pack_f16x2(a, 0.f) & 0xffffu);
}

// fp16 copies of the bf16 centre tables of all segments (K and V), in tile
// channel order (exact for bf16 values inside the fp16 normal range): one thread
// per eight channels, table j covering threads [start[j], start[j+1]).
struct TableJobs {
  const uint4* src[2 * kMaxSegs];
  uint4* dst[2 * kMaxSegs];
  int64_t start[2 * kMaxSegs + 1];
  int n;
};

__global__ __launch_bounds__(256) void centre_tables_kernel(TableJobs jobs) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= jobs.start[jobs.n]) return;
  int j = 0;
  while (i >= jobs.start[j + 1]) ++j;
  const int64_t e = i - jobs.start[j];
  const uint4 w = jobs.src[j][e];   // channels (0, 1), (2, 3), (4, 5), (6, 7)
  jobs.dst[j][e] = make_uint4(pack_f16x2(bf16_lo(w.x), bf16_lo(w.y)), pack_f16x2(bf16_hi(w.x), bf16_hi(w.y)),
                              pack_f16x2(bf16_lo(w.z), bf16_lo(w.w)), pack_f16x2(bf16_hi(w.z), bf16_hi(w.w)));
}

template <int DQ, bool LOWDIM, int DOUT, bool PSAC = false>
hipError_t pick_bits(const AttendParams& p, const SegList& segs, int kb, int vb, int g, hipStream_t st) {
  const dim3 grid(unsigned((p.n_q + 255) / 256) * unsigned(p.heads) * unsigned(p.n_split));
#define KVC_CASE(KB_, VB_, G_)                                                                                     \
  if (kb == KB_ && vb == VB_ && g == G_) {                                                                         \
    hipLaunchKernelGGL((attend_kernel<DQ, KB_, VB_, G_, LOWDIM, DOUT, PSAC>), grid, dim3(512), 0, st, p, segs); \
    return hipGetLastError();                                                                                      \
  }
  KVC_CASE(2, 2, 16) KVC_CASE(2, 4, 16) KVC_CASE(4, 2, 16) KVC_CASE(4, 4, 16)
  KVC_CASE(2, 2, 32) KVC_CASE(2, 4, 32) KVC_CASE(4, 2, 32) KVC_CASE(4, 4, 32)
  if constexpr (!LOWDIM && !PSAC) {
    KVC_CASE(16, 16, 16)     // 16-bit residual segments (no groups; G is nominal)
  }
#undef KVC_CASE
  return hipErrorInvalidValue;
}

template <int D>
hipError_t pick_f32(const float* q, int64_t n_q, int heads, const SegList& segs, int kb, int vb, int g, float* out,
                    float* lse, hipStream_t st) {
  const dim3 grid(unsigned((n_q + 3) / 4), unsigned(heads));
  const float scale = 1.0f / sqrtf(float(D));
#define KVC_CASE(KB_, VB_, G_)                                                                                  \
  if (kb == KB_ && vb == VB_ && g == G_) {                                                                      \
    hipLaunchKernelGGL((attend_f32_kernel<D, KB_, VB_, G_>), grid, dim3(256), 0, st, q, n_q, segs, scale, out, \
                       lse);                                                                                    \
    return hipGetLastError();                                                                                   \
  }
  KVC_CASE(2, 2, 16) KVC_CASE(2, 4, 16) KVC_CASE(4, 2, 16) KVC_CASE(4, 4, 16)
  KVC_CASE(2, 2, 32) KVC_CASE(2, 4, 32) KVC_CASE(4, 2, 32) KVC_CASE(4, 4, 32)
#undef KVC_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attend(int heads, int64_t n_q, int dim, kvc_dtype q_dtype, const void* q, const SegList& segs,
                         int k_bits, int v_bits, int group, kvc_dtype cdt, int n_split, float* out, float* lse,
                         hipStream_t st, const float* u_psac) {
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
  p.q_lo = nullptr;
  p.n_q = n_q;
  p.heads = heads;
  p.n_split = n_split;
  p.scale_log2 = 1.4426950408889634f / sqrtf(float(dim));
  p.out = out;
  p.lse = lse;
  p.basis_v = nullptr;
  p.u_psac = u_psac;
  if (cdt != KVC_BF16 && segs.total_tiles > 0) return hipErrorInvalidValue;
  if (u_psac != nullptr && segs.total_tiles > 0) {
    if (dim != 128) return hipErrorInvalidValue;
    return pick_bits<128, false, 128, true>(p, segs, k_bits, v_bits, group, st);
  }
  if (dim == 128) return pick_bits<128, false, 128>(p, segs, k_bits, v_bits, group, st);
  if (dim == 64) return pick_bits<64, false, 64>(p, segs, k_bits, v_bits, group, st);
  return hipErrorInvalidValue;
}

hipError_t launch_project_queries(int heads, int64_t n_q, int dim, int rank, const void* q, const float* basis,
                                  uint16_t* q_proj, hipStream_t st) {
  if (heads == 0 || n_q == 0) return hipSuccess;
  const dim3 grid(unsigned((n_q + 255) / 256), unsigned(heads));
  const auto* qb = static_cast<const uint16_t*>(q);
  if (dim == 128 && rank == 32)
    hipLaunchKernelGGL((project_queries_kernel<128, 32>), grid, dim3(256), 0, st, qb, basis, n_q, q_proj);
  else if (dim == 128 && rank == 64)
    hipLaunchKernelGGL((project_queries_kernel<128, 64>), grid, dim3(256), 0, st, qb, basis, n_q, q_proj);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_project_centres(int heads, int C, int dim, int rank, kvc_dtype cdt, const void* cent,
                                  const float* basis, uint16_t* tab, hipStream_t st) {
  if (heads == 0 || C == 0) return hipSuccess;
  const dim3 grid(unsigned((C * rank + 255) / 256), unsigned(heads));
  if (cdt == KVC_BF16)
    hipLaunchKernelGGL((project_centres_kernel<bf16_t>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(cent),
                       basis, C, dim, rank, tab);
  else
    hipLaunchKernelGGL((project_centres_kernel<float>), grid, dim3(256), 0, st, static_cast<const float*>(cent), basis,
                       C, dim, rank, tab);
  return hipGetLastError();
}

hipError_t launch_centre_tables(int heads, int dim, const SegList& segs, hipStream_t st) {
  if (heads == 0 || segs.n == 0) return hipSuccess;
  if (dim % 8 != 0) return hipErrorInvalidValue;
  TableJobs jobs;
  jobs.n = 0;
  jobs.start[0] = 0;
  for (int i = 0; i < segs.n; ++i) {
    const int64_t n8 = int64_t(heads) * segs.s[i].n_centroids * dim / 8;
    for (int t = 0; t < 2; ++t) {
      jobs.src[jobs.n] = static_cast<const uint4*>(t == 0 ? segs.s[i].k_cent : segs.s[i].v_cent);
      jobs.dst[jobs.n] = reinterpret_cast<uint4*>(const_cast<uint16_t*>(t == 0 ? segs.s[i].k_tab : segs.s[i].v_tab));
      jobs.start[jobs.n + 1] = jobs.start[jobs.n] + n8;
      ++jobs.n;
    }
  }
  const int64_t total = jobs.start[jobs.n];
  hipLaunchKernelGGL(centre_tables_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st, jobs);
  return hipGetLastError();
}

hipError_t launch_attend_lowdim(int heads, int64_t n_q, int dim, int rank, const uint16_t* q_proj,
                                const float* basis_v, const SegList& segs, int k_bits, int v_bits, int group,
                                int n_split, float* out, float* lse, hipStream_t st) {
  if (heads == 0 || n_q == 0) return hipSuccess;
  if (segs.total_tiles == 0) { k_bits = v_bits = 2; group = 16; }
  AttendParams p;
  p.q = q_proj;
  p.q_lo = q_proj + int64_t(heads) * n_q * rank;
  p.n_q = n_q;
  p.heads = heads;
  p.n_split = n_split;
  p.scale_log2 = 1.4426950408889634f / sqrtf(float(dim));
  p.out = out;
  p.lse = lse;
  p.basis_v = basis_v;
  p.u_psac = nullptr;
  if (dim != 128) return hipErrorInvalidValue;
  if (rank == 32) return pick_bits<32, true, 128>(p, segs, k_bits, v_bits, group, st);
  if (rank == 64) return pick_bits<64, true, 128>(p, segs, k_bits, v_bits, group, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
