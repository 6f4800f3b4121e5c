// C ABI: argument validation, workspace planning and kernel dispatch.
// Every check runs before any launch; no C++ exception leaves this file.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kvc_internal.h"

namespace {

thread_local std::string g_last_error;

kvc_status fail(kvc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvc_status ok() {
  g_last_error.clear();
  return KVC_OK;
}

kvc_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define KVC_REQUIRE(cond, st, ...) \
  do {                             \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define KVC_PTR(p, needed, name)                                                        \
  do {                                                                                  \
    if (needed) {                                                                       \
      if ((p) == nullptr) return fail(KVC_ERR_INVALID_ARG, "%s is NULL", name);         \
      if (!aligned16(p)) return fail(KVC_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
    }                                                                                   \
  } while (0)

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

bool valid_dtype(kvc_dtype d) { return d == KVC_F32 || d == KVC_BF16; }
size_t dtype_size(kvc_dtype d) { return d == KVC_F32 ? 4 : 2; }

int64_t tiles_of(int64_t n) { return (n + kvc::kAttendTile - 1) / kvc::kAttendTile; }

// Codec of a segment: what one attention kernel instantiation handles.
struct CodecKey {
  int kb, vb, g;
  kvc_dtype cdt;
  bool operator==(const CodecKey& o) const { return kb == o.kb && vb == o.vb && g == o.g && cdt == o.cdt; }
};

CodecKey codec_of(const kvc_segment& s) {
  // 16-bit residual segments have no groups: one nominal group value
  return CodecKey{s.k_bits, s.v_bits, s.k_bits == 16 ? 16 : s.group, s.cent_dtype};
}

// Validate a segment list for attention; fills the device list with every
// non-empty segment (tiles numbered across the whole list) and, per device
// segment, the index of its codec among the distinct codecs of the call (in order
// of first appearance).  Without allow_mixed every segment must share one codec.
kvc_status check_segments(int32_t heads, int32_t dim, const kvc_segment* segs, int32_t n_segs,
                          int32_t want_rank, bool allow_mixed, kvc::SegList* out, CodecKey* codecs,
                          int* n_codecs, int* codec_of_seg, const uint16_t* const* psac_coefs = nullptr) {
  KVC_REQUIRE(n_segs >= 0, KVC_ERR_INVALID_ARG, "n_segs < 0");
  KVC_REQUIRE(n_segs == 0 || segs != nullptr, KVC_ERR_INVALID_ARG, "segs is NULL");
  KVC_REQUIRE(n_segs <= kvc::kMaxSegs, KVC_ERR_UNSUPPORTED, "at most %d segments per call", kvc::kMaxSegs);
  out->n = 0;
  out->total_tiles = 0;
  *n_codecs = 0;
  for (int i = 0; i < n_segs; ++i) {
    const kvc_segment& s = segs[i];
    KVC_REQUIRE(s.n_tokens >= 0, KVC_ERR_INVALID_ARG, "segment %d: n_tokens < 0", i);
    // the attention kernel addresses a head's rows with 32-bit offsets
    KVC_REQUIRE(s.n_tokens <= (int64_t(1) << 25), KVC_ERR_UNSUPPORTED,
                "segment %d: at most 2^25 tokens per head and segment", i);
    KVC_REQUIRE(s.rank == want_rank, KVC_ERR_INVALID_ARG, "segment %d: rank %d, expected %d", i, s.rank,
                want_rank);
    const int code_dim = want_rank ? want_rank : dim;
    const bool raw = s.k_bits == 16 || s.v_bits == 16;
    KVC_REQUIRE(s.k_bits == 2 || s.k_bits == 4 || s.k_bits == 16, KVC_ERR_INVALID_ARG,
                "segment %d: k_bits must be 2, 4 or 16", i);
    KVC_REQUIRE(s.v_bits == 2 || s.v_bits == 4 || s.v_bits == 16, KVC_ERR_INVALID_ARG,
                "segment %d: v_bits must be 2, 4 or 16", i);
    KVC_REQUIRE(!raw || (s.k_bits == 16 && s.v_bits == 16 && want_rank == 0), KVC_ERR_UNSUPPORTED,
                "segment %d: 16-bit residuals need k_bits = v_bits = 16 and full dimension", i);
    // a 16-bit residual row is 2*dim <= 256 bytes: 2^24 rows keep its 32-bit offsets in range
    KVC_REQUIRE(!raw || s.n_tokens <= (int64_t(1) << 24), KVC_ERR_UNSUPPORTED,
                "segment %d: at most 2^24 tokens per head in a 16-bit residual segment", i);
    KVC_REQUIRE(raw || (s.group > 0 && code_dim % s.group == 0), KVC_ERR_INVALID_ARG,
                "segment %d: group %d does not divide %d", i, s.group, code_dim);
    KVC_REQUIRE(s.n_centroids >= 1 && s.n_centroids <= 256, KVC_ERR_INVALID_ARG,
                "segment %d: n_centroids must be in [1, 256]", i);
    KVC_REQUIRE(valid_dtype(s.cent_dtype), KVC_ERR_INVALID_ARG, "segment %d: bad centre dtype", i);
    if (s.n_tokens == 0) continue;
    const CodecKey key = codec_of(s);
    int ci = 0;
    while (ci < *n_codecs && !(codecs[ci] == key)) ++ci;
    if (ci == *n_codecs) {
      KVC_REQUIRE(allow_mixed || *n_codecs == 0, KVC_ERR_UNSUPPORTED,
                  "segment %d: all segments of a call must share bits, group and centre dtype", i);
      codecs[(*n_codecs)++] = key;
    }
    KVC_PTR(s.k_codes, true, "segment k_codes");
    KVC_PTR(s.v_codes, true, "segment v_codes");
    KVC_PTR(s.k_meta, !raw, "segment k_meta");
    KVC_PTR(s.v_meta, !raw, "segment v_meta");
    KVC_PTR(s.k_ids, true, "segment k_ids");
    KVC_PTR(s.v_ids, true, "segment v_ids");
    KVC_PTR(s.k_cent, true, "segment k_cent");
    KVC_PTR(s.v_cent, true, "segment v_cent");
    codec_of_seg[out->n] = ci;
    kvc::SegDev& d = out->s[out->n++];
    d.n_tokens = s.n_tokens;
    d.tile_begin = out->total_tiles;
    d.n_centroids = s.n_centroids;
    d.k_codes = s.k_codes;
    d.v_codes = s.v_codes;
    d.k_meta = reinterpret_cast<const uint32_t*>(s.k_meta);
    d.v_meta = reinterpret_cast<const uint32_t*>(s.v_meta);
    d.k_ids = s.k_ids;
    d.v_ids = s.v_ids;
    d.k_cent = s.k_cent;
    d.v_cent = s.v_cent;
    d.k_tab = nullptr;
    d.v_tab = nullptr;
    d.psac = nullptr;
    if (psac_coefs != nullptr) {
      KVC_REQUIRE(!raw, KVC_ERR_UNSUPPORTED, "segment %d: the logit compensation reads 2/4-bit keys only", i);
      KVC_PTR(psac_coefs[i], true, "segment compensation coefficients");
      d.psac = psac_coefs[i];
    }
    out->total_tiles += tiles_of(s.n_tokens);
  }
  (void)heads;
  return ok();
}

// The segments of one codec, tiles renumbered from 0.
kvc::SegList codec_subset(const kvc::SegList& all, const int* codec_of_seg, int ci) {
  kvc::SegList sl;
  sl.n = 0;
  sl.total_tiles = 0;
  for (int i = 0; i < all.n; ++i) {
    if (codec_of_seg[i] != ci) continue;
    sl.s[sl.n] = all.s[i];
    sl.s[sl.n].tile_begin = sl.total_tiles;
    sl.total_tiles += tiles_of(all.s[i].n_tokens);
    ++sl.n;
  }
  return sl;
}

// Partial results of a full-dim bf16 attention call: the splits of every codec's
// launch (one launch per distinct codec), merged by LSE at the end.
int attend_parts(int32_t heads, int64_t n_q, const kvc_segment* segs, int32_t n_segs) {
  CodecKey keys[kvc::kMaxSegs];
  int64_t tiles[kvc::kMaxSegs];
  int n = 0;
  for (int i = 0; segs != nullptr && i < n_segs && i < kvc::kMaxSegs; ++i) {
    if (segs[i].n_tokens <= 0) continue;
    const CodecKey key = codec_of(segs[i]);
    int ci = 0;
    while (ci < n && !(keys[ci] == key)) ++ci;
    if (ci == n) { keys[n] = key; tiles[n] = 0; ++n; }
    tiles[ci] += tiles_of(segs[i].n_tokens);
  }
  int parts = 0;
  for (int ci = 0; ci < n; ++ci) parts += kvc::attend_split_plan(heads, n_q, tiles[ci], kvc::kAttendRows);
  return parts > 0 ? parts : 1;
}

int64_t total_tokens(const kvc_segment* segs, int32_t n_segs) {
  int64_t t = 0;
  if (segs == nullptr) return 0;
  for (int i = 0; i < n_segs; ++i) t += segs[i].n_tokens > 0 ? segs[i].n_tokens : 0;
  return t;
}

int64_t total_tiles_of(const kvc_segment* segs, int32_t n_segs) {
  int64_t t = 0;
  if (segs == nullptr) return 0;
  for (int i = 0; i < n_segs; ++i) t += segs[i].n_tokens > 0 ? tiles_of(segs[i].n_tokens) : 0;
  return t;
}

// fp16 centre tables (K and V) of every non-empty segment, code_dim channels a row
size_t table_bytes(int32_t heads, int32_t code_dim, const kvc_segment* segs, int32_t n_segs) {
  size_t b = 0;
  for (int i = 0; segs != nullptr && i < n_segs; ++i)
    if (segs[i].n_tokens > 0 && segs[i].n_centroids > 0)
      b += 2 * align_up(size_t(heads) * size_t(segs[i].n_centroids) * code_dim * 2);
  return b;
}

size_t split_bytes(int32_t heads, int64_t n_q, int32_t dim, int n_split) {
  if (n_split <= 1) return 0;
  const size_t rows = size_t(heads) * size_t(n_q);
  return align_up(size_t(n_split) * rows * dim * 4) + align_up(size_t(n_split) * rows * 4);
}

}  // namespace

namespace kvc {

// Split of the history across workgroups.  One workgroup occupies one compute
// unit (256 on the chip).  When the query blocks alone cover at least 192 of
// them, splitting cannot raise the fraction of busy units by much and only adds
// a merge pass, so the history stays whole; otherwise it is split (up to 8 ways,
// at least 16 tiles per split) until about two workgroups per unit exist.
int attend_split_plan(int heads, int64_t n_q, int64_t total_tiles, int rows_per_block) {
  if (total_tiles <= 0 || n_q <= 0 || heads <= 0) return 1;
  const int64_t blocks = int64_t(heads) * ((n_q + rows_per_block - 1) / rows_per_block);
  if (blocks >= 192) return 1;
  int s = 1;
  while (s < 8 && blocks * (s + 1) <= 512 && total_tiles / (s + 1) >= 16) ++s;
  return s;
}

}  // namespace kvc

extern "C" {

const char* kvc_status_string(kvc_status status) {
  switch (status) {
    case KVC_OK: return "KVC_OK";
    case KVC_ERR_INVALID_ARG: return "KVC_ERR_INVALID_ARG";
    case KVC_ERR_UNSUPPORTED: return "KVC_ERR_UNSUPPORTED";
    case KVC_ERR_WORKSPACE: return "KVC_ERR_WORKSPACE";
    case KVC_ERR_HIP: return "KVC_ERR_HIP";
  }
  return "unknown kvc_status";
}

const char* kvc_last_error(void) { return g_last_error.c_str(); }

const char* kvc_version(void) { return "kvc 0.1.0 (gfx950)"; }

// ------------------------------------------------------------------------------ fit / assign
size_t kvc_fit_assign_workspace_bytes(int32_t heads, int64_t n_tokens, int32_t dim, int32_t n_centroids) {
  (void)dim;
  if (heads <= 0 || n_centroids <= 0) return 0;
  // member lists of long heads, or reserved (the centre update keeps its lists in LDS)
  return align_up(kvc::kmeans_update_workspace(heads, n_tokens > 0 ? n_tokens : 0, n_centroids));
}

kvc_status kvc_fit_assign(int32_t heads, int64_t n_tokens, int32_t dim, kvc_dtype dt, const void* x,
                          int32_t n_centroids, void* centroids, int32_t n_iters, uint8_t* ids_out,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_tokens >= 0, KVC_ERR_INVALID_ARG, "heads and n_tokens must be >= 0");
    KVC_REQUIRE(n_tokens < (int64_t(1) << 31), KVC_ERR_INVALID_ARG, "n_tokens must be < 2^31 (32-bit token indices)");
    KVC_REQUIRE(heads <= 65535, KVC_ERR_UNSUPPORTED, "at most 65535 heads per call");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(valid_dtype(dt), KVC_ERR_INVALID_ARG, "bad dtype");
    KVC_REQUIRE(n_centroids >= 1 && n_centroids <= 256, KVC_ERR_INVALID_ARG, "n_centroids must be in [1, 256]");
    KVC_REQUIRE(n_iters >= 0, KVC_ERR_INVALID_ARG, "n_iters must be >= 0");
    const bool work = heads > 0 && n_tokens > 0;
    KVC_PTR(x, work, "x");
    KVC_PTR(centroids, heads > 0, "centroids");
    KVC_PTR(ids_out, work, "ids_out");
    if (!work) return ok();
    const size_t need = kvc_fit_assign_workspace_bytes(heads, n_tokens, dim, n_centroids);
    KVC_REQUIRE(ws_bytes >= need, KVC_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    KVC_PTR(ws, true, "ws");
    for (int it = 0; it <= n_iters; ++it) {
      hipError_t e = kvc::launch_assign(heads, n_tokens, dim, dt, x, n_centroids, centroids, ids_out, stream);
      if (e != hipSuccess) return hip_status(e, "assign");
      if (it == n_iters) break;
      e = kvc::launch_kmeans_update(heads, n_tokens, dim, dt, x, n_centroids, centroids, ids_out,
                                    ws, stream);
      if (e != hipSuccess) return hip_status(e, "k-means update");
    }
    return ok();
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_fit_assign");
  }
}

// ------------------------------------------------------------------------------ query-aware assignment
kvc_status kvc_assign_qsac(int32_t heads, int64_t n_tokens, int32_t dim, kvc_dtype dt, const void* x,
                           int32_t n_centroids, const void* centroids, const float* w, int32_t n_cand,
                           int32_t group, uint8_t* ids_out, hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_tokens >= 0, KVC_ERR_INVALID_ARG, "heads and n_tokens must be >= 0");
    KVC_REQUIRE(heads <= 65535, KVC_ERR_UNSUPPORTED, "at most 65535 heads per call");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(valid_dtype(dt), KVC_ERR_INVALID_ARG, "bad dtype");
    KVC_REQUIRE(n_centroids >= 1 && n_centroids <= 256, KVC_ERR_INVALID_ARG, "n_centroids must be in [1, 256]");
    KVC_REQUIRE(n_cand >= 1, KVC_ERR_INVALID_ARG, "n_cand must be >= 1");
    KVC_REQUIRE(n_cand == 1 || n_cand == 2 || n_cand == 4 || n_cand == 8, KVC_ERR_UNSUPPORTED,
                "n_cand must be 1, 2, 4 or 8");
    KVC_REQUIRE(group > 0 && dim % group == 0, KVC_ERR_INVALID_ARG, "group must divide dim");
    KVC_REQUIRE(group == 16 || group == 32, KVC_ERR_UNSUPPORTED, "group must be 16 or 32");
    const bool work = heads > 0 && n_tokens > 0;
    KVC_PTR(x, work, "x");
    KVC_PTR(centroids, work, "centroids");
    KVC_PTR(ids_out, work, "ids_out");
    if (w) KVC_PTR(w, work, "w");
    if (!work) return ok();
    return hip_status(kvc::launch_assign_qsac(heads, n_tokens, dim, dt, x, n_centroids, centroids, w, n_cand,
                                              group, ids_out, stream),
                      "qsac assign");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_assign_qsac");
  }
}

size_t kvc_query_stats_workspace_bytes(int32_t heads, int64_t n_q, int32_t dim) {
  if (heads <= 0 || n_q <= 0 || (dim != 64 && dim != 128)) return 0;
  return align_up(kvc::query_stats_workspace(heads, n_q, dim));
}

kvc_status kvc_query_stats(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                           int64_t n_prev, float* w, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_q >= 0 && n_prev >= 0, KVC_ERR_INVALID_ARG, "heads, n_q and n_prev must be >= 0");
    KVC_REQUIRE(heads <= 65535, KVC_ERR_UNSUPPORTED, "at most 65535 heads per call");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(valid_dtype(q_dtype), KVC_ERR_INVALID_ARG, "bad dtype");
    const bool work = heads > 0 && n_q > 0;
    KVC_PTR(q, work, "q");
    KVC_PTR(w, work, "w");
    if (!work) return ok();
    const size_t need = kvc_query_stats_workspace_bytes(heads, n_q, dim);
    KVC_REQUIRE(ws_bytes >= need, KVC_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    KVC_PTR(ws, true, "ws");
    return hip_status(kvc::launch_query_stats(heads, n_q, dim, q_dtype, q, n_prev, w, ws, stream), "query stats");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_query_stats");
  }
}

// ------------------------------------------------------------------------------ routing
kvc_status kvc_route_frames(int32_t n_frames, int32_t n_recent, int32_t period, int32_t n_sink,
                            int32_t all_full_until, uint8_t* full_dim) {
  KVC_REQUIRE(n_frames >= 0 && n_recent >= 0 && period >= 0 && n_sink >= 0 && all_full_until >= 0,
              KVC_ERR_INVALID_ARG, "frame counts must be >= 0");
  KVC_REQUIRE(n_frames == 0 || full_dim != nullptr, KVC_ERR_INVALID_ARG, "full_dim is NULL");
  for (int32_t f = 0; f < n_frames; ++f) {
    const bool full = n_frames <= all_full_until || f >= n_frames - n_recent || f < n_sink ||
                      (period > 0 && f % period == 0);
    full_dim[f] = full ? 1 : 0;
  }
  return ok();
}

int32_t kvc_anchor_bits(int32_t k_bits, int32_t v_bits) {
  int32_t b = k_bits > v_bits ? k_bits : v_bits;
  return b > 4 ? b : 4;
}

// ------------------------------------------------------------------------------ encode
size_t kvc_encode_workspace_bytes(int32_t heads, int64_t n_tokens, int32_t dim, int32_t n_centroids,
                                  int32_t ids_given) {
  (void)heads; (void)n_tokens; (void)dim; (void)n_centroids; (void)ids_given;
  return 0;   // the assignment (ids_in NULL) needs no workspace
}

kvc_status kvc_encode(int32_t heads, int64_t n_tokens, int32_t dim, kvc_dtype dt, const void* x,
                      int32_t n_centroids, const void* centroids, const uint8_t* ids_in, uint8_t* ids_out,
                      const float* basis, int32_t rank, int32_t bits, int32_t group, uint8_t* codes,
                      uint16_t* meta, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_tokens >= 0, KVC_ERR_INVALID_ARG, "heads and n_tokens must be >= 0");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(valid_dtype(dt), KVC_ERR_INVALID_ARG, "bad dtype");
    KVC_REQUIRE(n_centroids >= 1 && n_centroids <= 256, KVC_ERR_INVALID_ARG, "n_centroids must be in [1, 256]");
    KVC_REQUIRE(bits == 2 || bits == 4 || bits == 16, KVC_ERR_INVALID_ARG, "bits must be 2, 4 or 16");
    KVC_REQUIRE((basis == nullptr) == (rank == 0), KVC_ERR_INVALID_ARG, "rank must be 0 exactly when basis is NULL");
    const int code_dim = rank ? rank : dim;
    const bool raw = bits == 16;      // fp16 residuals: no groups, no metadata
    KVC_REQUIRE(!raw || rank == 0, KVC_ERR_UNSUPPORTED, "16-bit residuals are full-dimensional only");
    KVC_REQUIRE(raw || rank == 0 || (rank >= group && rank <= dim), KVC_ERR_INVALID_ARG,
                "rank must be 0 or in [group, dim]");
    KVC_REQUIRE(raw || (group > 0 && code_dim % group == 0), KVC_ERR_INVALID_ARG,
                "group must divide the coded dimension");
    KVC_REQUIRE(raw || group == 16 || group == 32, KVC_ERR_UNSUPPORTED, "group must be 16 or 32");
    KVC_REQUIRE(rank == 0 || ((rank == 32 || rank == 64) && dim == 128), KVC_ERR_UNSUPPORTED,
                "coefficient codes need dim 128 and rank 32 or 64");
    KVC_REQUIRE(ids_out == nullptr || ids_out != ids_in, KVC_ERR_INVALID_ARG, "ids_out must not alias ids_in");
    const bool work = heads > 0 && n_tokens > 0;
    KVC_PTR(x, work, "x");
    KVC_PTR(centroids, work, "centroids");
    KVC_PTR(codes, work, "codes");
    KVC_PTR(meta, work && !raw, "meta");
    KVC_PTR(basis, work && rank > 0, "basis");
    if (ids_in) KVC_PTR(ids_in, work, "ids_in");
    if (ids_out) KVC_PTR(ids_out, work, "ids_out");
    if (!work) return ok();
    const uint8_t* ids = ids_in;
    if (ids == nullptr) {
      KVC_REQUIRE(ids_out != nullptr, KVC_ERR_INVALID_ARG, "ids_out is needed when ids_in is NULL");
      (void)ws; (void)ws_bytes;
      hipError_t e = kvc::launch_assign(heads, n_tokens, dim, dt, x, n_centroids, centroids, ids_out, stream);
      if (e != hipSuccess) return hip_status(e, "assign");
      ids = ids_out;
    } else if (ids_out != nullptr) {
      hipError_t e = hipMemcpyAsync(ids_out, ids_in, size_t(heads) * size_t(n_tokens), hipMemcpyDeviceToDevice,
                                    stream);
      if (e != hipSuccess) return hip_status(e, "copy ids");
    }
    hipError_t e = kvc::launch_encode(heads, n_tokens, dim, dt, x, n_centroids, centroids, ids, basis, rank, bits,
                                      group, codes, meta, stream);
    return hip_status(e, "encode");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_encode");
  }
}

// ------------------------------------------------------------------------------ predictive residual codec
int32_t kvc_tempo_param_count(int32_t dim) { return dim > 0 ? 7 * dim + dim * dim : 0; }

namespace {
kvc_status tempo_check(int32_t heads, int32_t frame_tokens, int32_t first_frame, int32_t n_frames, int32_t dim,
                       int32_t k_bits, int32_t v_bits, int32_t group, const float* params, const void* k_codes,
                       const void* k_meta, const void* v_codes, const void* v_meta, const float* state) {
  KVC_REQUIRE(heads >= 0 && frame_tokens >= 0 && n_frames >= 0 && first_frame >= 0, KVC_ERR_INVALID_ARG,
              "heads, frame_tokens, n_frames and first_frame must be >= 0");
  KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
  KVC_REQUIRE((k_bits == 2 || k_bits == 4) && (v_bits == 2 || v_bits == 4), KVC_ERR_INVALID_ARG,
              "k_bits and v_bits must be 2 or 4");
  KVC_REQUIRE(group > 0 && dim % group == 0, KVC_ERR_INVALID_ARG, "group must divide dim");
  KVC_REQUIRE(group == 16 || group == 32, KVC_ERR_UNSUPPORTED, "group must be 16 or 32");
  KVC_REQUIRE(first_frame > 0 || n_frames <= 1, KVC_ERR_INVALID_ARG,
              "the anchor frame (first_frame = 0) is coded alone: n_frames must be 1");
  KVC_REQUIRE(first_frame > 0 || (k_bits == 4 && v_bits == 4), KVC_ERR_INVALID_ARG,
              "the anchor frame is coded at max(4, b_K, b_V) = 4 bits");
  KVC_REQUIRE(heads <= 65535, KVC_ERR_UNSUPPORTED, "at most 65535 heads per call");
  KVC_REQUIRE(int64_t(n_frames) * frame_tokens <= (int64_t(1) << 26), KVC_ERR_UNSUPPORTED,
              "at most 2^26 tokens per head and call");
  const bool work = heads > 0 && frame_tokens > 0 && n_frames > 0;
  KVC_PTR(params, work, "params");
  KVC_PTR(k_codes, work, "k_codes");
  KVC_PTR(k_meta, work, "k_meta");
  KVC_PTR(v_codes, work, "v_codes");
  KVC_PTR(v_meta, work, "v_meta");
  KVC_PTR(state, work, "state");
  return ok();
}
}  // namespace

kvc_status kvc_tempo_encode(int32_t heads, int32_t frame_tokens, int32_t first_frame, int32_t n_frames, int32_t dim,
                            kvc_dtype dt, const void* k, const void* v, const float* params, int32_t k_bits,
                            int32_t v_bits, int32_t group, uint8_t* k_codes, uint16_t* k_meta, uint8_t* v_codes,
                            uint16_t* v_meta, float* state, hipStream_t stream) {
  try {
    kvc_status st = tempo_check(heads, frame_tokens, first_frame, n_frames, dim, k_bits, v_bits, group, params,
                                k_codes, k_meta, v_codes, v_meta, state);
    if (st != KVC_OK) return st;
    KVC_REQUIRE(valid_dtype(dt), KVC_ERR_INVALID_ARG, "bad dtype");
    const bool work = heads > 0 && frame_tokens > 0 && n_frames > 0;
    KVC_PTR(k, work, "k");
    KVC_PTR(v, work, "v");
    if (!work) return ok();
    return hip_status(kvc::launch_tempo(false, heads, frame_tokens, first_frame, n_frames, dim, dt, k, v, params,
                                        k_bits, v_bits, group, k_codes, k_meta, v_codes, v_meta, state, nullptr,
                                        nullptr, stream),
                      "tempo encode");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_tempo_encode");
  }
}

kvc_status kvc_tempo_decode(int32_t heads, int32_t frame_tokens, int32_t first_frame, int32_t n_frames, int32_t dim,
                            const float* params, int32_t k_bits, int32_t v_bits, int32_t group,
                            const uint8_t* k_codes, const uint16_t* k_meta, const uint8_t* v_codes,
                            const uint16_t* v_meta, float* state, uint16_t* k_hat, uint16_t* v_hat,
                            hipStream_t stream) {
  try {
    kvc_status st = tempo_check(heads, frame_tokens, first_frame, n_frames, dim, k_bits, v_bits, group, params,
                                k_codes, k_meta, v_codes, v_meta, state);
    if (st != KVC_OK) return st;
    const bool work = heads > 0 && frame_tokens > 0 && n_frames > 0;
    KVC_PTR(k_hat, work, "k_hat");
    KVC_PTR(v_hat, work, "v_hat");
    if (!work) return ok();
    return hip_status(kvc::launch_tempo(true, heads, frame_tokens, first_frame, n_frames, dim, KVC_BF16, nullptr,
                                        nullptr, params, k_bits, v_bits, group, const_cast<uint8_t*>(k_codes),
                                        const_cast<uint16_t*>(k_meta), const_cast<uint8_t*>(v_codes),
                                        const_cast<uint16_t*>(v_meta), state, k_hat, v_hat, stream),
                      "tempo decode");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_tempo_decode");
  }
}

// ------------------------------------------------------------------------------ attention
size_t kvc_attend_workspace_bytes(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype,
                                  const kvc_segment* segs, int32_t n_segs) {
  if (heads <= 0 || n_q <= 0 || (dim != 64 && dim != 128)) return 0;
  if (q_dtype == KVC_F32) return 0;  // the fp32 path reads the fp32 centres and does not split
  const int parts = attend_parts(heads, n_q, segs, n_segs);
  return split_bytes(heads, n_q, dim, parts) + table_bytes(heads, dim, segs, n_segs);
}

namespace {
kvc_status attend_impl(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                       const kvc_segment* segs, int32_t n_segs, float* out, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t stream, const float* u_psac, const uint16_t* const* psac_coefs) {
  try {
    KVC_REQUIRE(heads >= 0 && n_q >= 0, KVC_ERR_INVALID_ARG, "heads and n_q must be >= 0");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(valid_dtype(q_dtype), KVC_ERR_INVALID_ARG, "bad q dtype");
    kvc::SegList sl;
    CodecKey codecs[kvc::kMaxSegs];
    int n_codecs = 0;
    int codec_of_seg[kvc::kMaxSegs];
    kvc_status st = check_segments(heads, dim, segs, n_segs, 0, /*allow_mixed=*/true, &sl, codecs, &n_codecs,
                                   codec_of_seg, psac_coefs);
    if (st != KVC_OK) return st;
    const bool work = heads > 0 && n_q > 0;
    KVC_PTR(q, work, "q");
    KVC_PTR(out, work, "out");
    KVC_PTR(lse, work, "lse");
    if (u_psac != nullptr) {
      KVC_PTR(u_psac, work, "u");
      KVC_REQUIRE(dim == 128 && q_dtype == KVC_BF16, KVC_ERR_UNSUPPORTED,
                  "the logit compensation needs dim 128 and bf16 queries");
    }
    if (!work) return ok();
    // one workgroup of 512 work-items per (256-query block, head, history split of at
    // most 8): the dispatch's work-item count must fit 32 bits
    KVC_REQUIRE(heads <= 65535 && (n_q + 255) / 256 * heads <= (int64_t(1) << 20), KVC_ERR_UNSUPPORTED,
                "at most 65535 heads and 2^20 blocks of 256 queries per call");
    for (int ci = 0; ci < n_codecs; ++ci) {
      KVC_REQUIRE(codecs[ci].g == 16 || codecs[ci].g == 32, KVC_ERR_UNSUPPORTED, "group must be 16 or 32");
      KVC_REQUIRE(q_dtype == codecs[ci].cdt, KVC_ERR_UNSUPPORTED, "queries and centres must share a dtype");
    }
    if (q_dtype == KVC_F32) {
      // fp32 queries: one launch over the fp32 centres (a single 2/4-bit codec)
      KVC_REQUIRE(n_codecs <= 1, KVC_ERR_UNSUPPORTED, "fp32 queries need one codec for all segments");
      KVC_REQUIRE(n_codecs == 0 || codecs[0].kb != 16, KVC_ERR_UNSUPPORTED,
                  "fp32 queries do not read 16-bit residual segments");
      KVC_REQUIRE(n_q <= (int64_t(1) << 26), KVC_ERR_UNSUPPORTED, "fp32 queries: at most 2^26 per head");
      const CodecKey c = n_codecs ? codecs[0] : CodecKey{2, 2, 16, KVC_F32};
      return hip_status(kvc::launch_attend(heads, n_q, dim, q_dtype, q, sl, c.kb, c.vb, c.g, c.cdt, 1, out, lse,
                                           stream),
                        "attend");
    }
    // bf16 queries: one launch per codec of the segment list, each split over the
    // history as planned; all partial results are merged by LSE at the end
    int split_of[kvc::kMaxSegs];
    int parts = 0;
    kvc::SegList sub[kvc::kMaxSegs];
    for (int ci = 0; ci < n_codecs; ++ci) {
      sub[ci] = codec_subset(sl, codec_of_seg, ci);
      split_of[ci] = kvc::attend_split_plan(heads, n_q, sub[ci].total_tiles, kvc::kAttendRows);
      parts += split_of[ci];
    }
    if (parts == 0) parts = 1;
    const size_t need = split_bytes(heads, n_q, dim, parts) + table_bytes(heads, dim, segs, n_segs);
    KVC_REQUIRE(ws_bytes >= need, KVC_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    if (need) KVC_PTR(ws, true, "ws");
    char* w = static_cast<char*>(ws);
    float* part_out = out;
    float* part_lse = lse;
    if (parts > 1) {
      part_out = reinterpret_cast<float*>(w);
      w += align_up(size_t(parts) * heads * n_q * dim * 4);
      part_lse = reinterpret_cast<float*>(w);
      w += align_up(size_t(parts) * heads * n_q * 4);
    }
    // fp16 centre tables in the attention tiles' channel order, every segment in one launch
    for (int i = 0; i < sl.n; ++i) {
      const size_t tb = align_up(size_t(heads) * size_t(sl.s[i].n_centroids) * dim * 2);
      sl.s[i].k_tab = reinterpret_cast<uint16_t*>(w);
      sl.s[i].v_tab = reinterpret_cast<uint16_t*>(w + tb);
      w += 2 * tb;
    }
    hipError_t e = kvc::launch_centre_tables(heads, dim, sl, stream);
    if (e != hipSuccess) return hip_status(e, "centre tables");
    if (n_codecs == 0) {
      // empty history: out = 0, lse = -inf
      e = kvc::launch_attend(heads, n_q, dim, q_dtype, q, sl, 2, 2, 16, KVC_BF16, 1, out, lse, stream);
      return hip_status(e, "attend");
    }
    const int64_t rows = int64_t(heads) * n_q;
    int slot = 0;
    for (int ci = 0; ci < n_codecs; ++ci) {
      kvc::SegList& g = sub[ci];
      for (int i = 0, j = 0; i < sl.n; ++i)
        if (codec_of_seg[i] == ci) { g.s[j].k_tab = sl.s[i].k_tab; g.s[j].v_tab = sl.s[i].v_tab; ++j; }
      float* po = parts > 1 ? part_out + slot * rows * dim : out;
      float* pl = parts > 1 ? part_lse + slot * rows : lse;
      e = kvc::launch_attend(heads, n_q, dim, q_dtype, q, g, codecs[ci].kb, codecs[ci].vb, codecs[ci].g,
                             codecs[ci].cdt, split_of[ci], po, pl, stream, u_psac);
      if (e != hipSuccess) return hip_status(e, "attend");
      slot += split_of[ci];
    }
    if (parts > 1) {
      e = kvc::launch_lse_merge_strided(heads, n_q, dim, parts, part_out, part_lse, out, lse, stream);
      if (e != hipSuccess) return hip_status(e, "partial merge");
    }
    return ok();
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_attend");
  }
}
}  // namespace

kvc_status kvc_attend(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                      const kvc_segment* segs, int32_t n_segs, float* out, float* lse, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  return attend_impl(heads, n_q, dim, q_dtype, q, segs, n_segs, out, lse, ws, ws_bytes, stream, nullptr, nullptr);
}

}  // extern "C"

// ------------------------------------------------------------------------------ attention without allocation
// Workspace of kvc_attend_noalloc: one array per GPU, resident from the load of
// the library's code object until the process ends.  Host code never passes the
// array's own name to a kernel or a copy (on the host it names a host-side
// stand-in); it uses the device address that hipGetSymbolAddress returns for the
// current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[KVC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call
// on that device); nullptr with the message set on failure.
void* scratch_on_current_device(kvc_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_status(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = fail(KVC_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *st = hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *st = KVC_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

kvc_status kvc_attend_noalloc(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                              const kvc_segment* segs, int32_t n_segs, float* out, float* lse,
                              hipStream_t stream) {
  try {
    // the same validation and plan as kvc_attend; only the workspace differs
    const size_t need = kvc_attend_workspace_bytes(heads, n_q, dim, q_dtype, segs, n_segs);
    KVC_REQUIRE(need <= size_t(KVC_NOALLOC_SCRATCH_BYTES), KVC_ERR_WORKSPACE,
                "kvc_attend_noalloc: this call needs %zu bytes of workspace, above the %zu-byte static scratch "
                "array (use kvc_attend with a caller workspace)",
                need, size_t(KVC_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    if (need > 0) {
      kvc_status st = KVC_OK;
      ws = scratch_on_current_device(&st);
      if (ws == nullptr) return st;
    }
    return attend_impl(heads, n_q, dim, q_dtype, q, segs, n_segs, out, lse, ws, need, stream, nullptr, nullptr);
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_attend_noalloc");
  }
}

// ------------------------------------------------------------------------------ logit compensation
kvc_status kvc_attend_psac(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                           const float* u, int32_t r, const kvc_segment* segs, const uint16_t* const* coefs,
                           int32_t n_segs, float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  KVC_REQUIRE(r == kvc::kPsacRank, KVC_ERR_UNSUPPORTED, "the compensation rank must be %d", kvc::kPsacRank);
  KVC_REQUIRE(n_segs == 0 || coefs != nullptr, KVC_ERR_INVALID_ARG, "coefs is NULL");
  KVC_REQUIRE(u != nullptr || heads == 0 || n_q == 0, KVC_ERR_INVALID_ARG, "u is NULL");
  return attend_impl(heads, n_q, dim, q_dtype, q, segs, n_segs, out, lse, ws, ws_bytes, stream, u, coefs);
}

size_t kvc_attend_psac_workspace_bytes(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype,
                                       const kvc_segment* segs, int32_t n_segs) {
  return kvc_attend_workspace_bytes(heads, n_q, dim, q_dtype, segs, n_segs);
}

kvc_status kvc_query_moments(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                             int64_t n_prev, float* m, hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_q >= 0 && n_prev >= 0, KVC_ERR_INVALID_ARG, "heads, n_q and n_prev must be >= 0");
    KVC_REQUIRE(heads <= 65535, KVC_ERR_UNSUPPORTED, "at most 65535 heads per call");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(valid_dtype(q_dtype), KVC_ERR_INVALID_ARG, "bad dtype");
    const bool work = heads > 0 && n_q > 0;
    KVC_PTR(q, work, "q");
    KVC_PTR(m, work, "m");
    if (!work) return ok();
    return hip_status(kvc::launch_query_moments(heads, n_q, dim, q_dtype, q, n_prev, m, stream), "query moments");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_query_moments");
  }
}

kvc_status kvc_psac_basis(int32_t heads, int32_t dim, const float* m, int32_t r, int32_t n_iter,
                          const float* u_prev, float* u, float* lam, hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_iter >= 0, KVC_ERR_INVALID_ARG, "heads and n_iter must be >= 0");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(r == kvc::kPsacRank, KVC_ERR_UNSUPPORTED, "the compensation rank must be %d", kvc::kPsacRank);
    const bool work = heads > 0;
    KVC_PTR(m, work, "m");
    KVC_PTR(u, work, "u");
    KVC_PTR(lam, work, "lam");
    if (u_prev) KVC_PTR(u_prev, work, "u_prev");
    if (!work) return ok();
    return hip_status(kvc::launch_psac_basis(heads, dim, m, n_iter, u_prev, u, lam, stream), "psac basis");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_psac_basis");
  }
}

kvc_status kvc_psac_coeffs(int32_t heads, int64_t n_tokens, int32_t dim, kvc_dtype dt, const void* x,
                           int32_t n_centroids, const void* centroids, const uint8_t* ids, const uint8_t* codes,
                           const uint16_t* meta, int32_t bits, int32_t group, const float* u, int32_t r,
                           uint16_t* coef, hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_tokens >= 0, KVC_ERR_INVALID_ARG, "heads and n_tokens must be >= 0");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(valid_dtype(dt), KVC_ERR_INVALID_ARG, "bad dtype");
    KVC_REQUIRE(n_centroids >= 1 && n_centroids <= 256, KVC_ERR_INVALID_ARG, "n_centroids must be in [1, 256]");
    KVC_REQUIRE(bits == 2 || bits == 4, KVC_ERR_UNSUPPORTED, "bits must be 2 or 4");
    KVC_REQUIRE(group > 0 && dim % group == 0, KVC_ERR_INVALID_ARG, "group must divide dim");
    KVC_REQUIRE(group == 16 || group == 32, KVC_ERR_UNSUPPORTED, "group must be 16 or 32");
    KVC_REQUIRE(r == kvc::kPsacRank, KVC_ERR_UNSUPPORTED, "the compensation rank must be %d", kvc::kPsacRank);
    KVC_REQUIRE(heads <= 65535, KVC_ERR_UNSUPPORTED, "at most 65535 heads per call");
    const bool work = heads > 0 && n_tokens > 0;
    KVC_PTR(x, work, "x");
    KVC_PTR(centroids, work, "centroids");
    KVC_PTR(ids, work, "ids");
    KVC_PTR(codes, work, "codes");
    KVC_PTR(meta, work, "meta");
    KVC_PTR(u, work, "u");
    KVC_PTR(coef, work, "coef");
    if (!work) return ok();
    return hip_status(kvc::launch_psac_coeffs(heads, n_tokens, dim, dt, x, n_centroids, centroids, ids, codes, meta,
                                              bits, group, u, coef, stream),
                      "psac coefficients");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_psac_coeffs");
  }
}

size_t kvc_attend_lowdim_workspace_bytes(int32_t heads, int64_t n_q, int32_t dim, int32_t rank,
                                         const kvc_segment* segs, int32_t n_segs) {
  if (heads <= 0 || n_q <= 0 || dim != 128 || (rank != 32 && rank != 64)) return 0;
  size_t b = align_up(size_t(heads) * size_t(n_q) * rank * 4);   // projected queries (fp16 hi + lo)
  b += table_bytes(heads, rank, segs, n_segs);                      // projected centres (fp16)
  const int s = kvc::attend_split_plan(heads, n_q, total_tiles_of(segs, n_segs), kvc::kLowdimRows);
  return b + split_bytes(heads, n_q, dim, s);
}

kvc_status kvc_attend_lowdim(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                             const float* basis_k, const float* basis_v, int32_t rank, const kvc_segment* segs,
                             int32_t n_segs, float* out, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_q >= 0, KVC_ERR_INVALID_ARG, "heads and n_q must be >= 0");
    KVC_REQUIRE(dim == 64 || dim == 128, KVC_ERR_INVALID_ARG, "dim must be 64 or 128");
    KVC_REQUIRE(valid_dtype(q_dtype), KVC_ERR_INVALID_ARG, "bad q dtype");
    KVC_REQUIRE(rank > 0 && rank <= dim, KVC_ERR_INVALID_ARG, "rank must be in [1, dim]");
    KVC_REQUIRE(dim == 128 && (rank == 32 || rank == 64), KVC_ERR_UNSUPPORTED, "low-dim path needs dim 128, rank 32 or 64");
    KVC_REQUIRE(q_dtype == KVC_BF16, KVC_ERR_UNSUPPORTED, "low-dim path needs bf16 queries");
    kvc::SegList sl;
    CodecKey codecs[kvc::kMaxSegs];
    int n_codecs = 0;
    int codec_of_seg[kvc::kMaxSegs];
    kvc_status st = check_segments(heads, dim, segs, n_segs, rank, /*allow_mixed=*/false, &sl, codecs, &n_codecs,
                                   codec_of_seg);
    if (st != KVC_OK) return st;
    const bool work = heads > 0 && n_q > 0;
    KVC_PTR(q, work, "q");
    KVC_PTR(basis_k, work, "basis_k");
    KVC_PTR(basis_v, work, "basis_v");
    KVC_PTR(out, work, "out");
    KVC_PTR(lse, work, "lse");
    if (!work) return ok();
    // one workgroup of 512 work-items per (256-query block, head, history split of at
    // most 8): the dispatch's work-item count must fit 32 bits
    KVC_REQUIRE(heads <= 65535 && (n_q + 255) / 256 * heads <= (int64_t(1) << 20), KVC_ERR_UNSUPPORTED,
                "at most 65535 heads and 2^20 blocks of 256 queries per call");
    const CodecKey c = n_codecs ? codecs[0] : CodecKey{2, 2, 16, KVC_BF16};
    if (sl.total_tiles > 0) {
      KVC_REQUIRE(c.g == 16 || c.g == 32, KVC_ERR_UNSUPPORTED, "group must be 16 or 32");
      KVC_REQUIRE(c.cdt == KVC_BF16, KVC_ERR_UNSUPPORTED, "low-dim path needs bf16 centres");
    }
    const int kb = c.kb, vb = c.vb, g = c.g;
    const kvc_dtype cdt = c.cdt;
    const size_t need = kvc_attend_lowdim_workspace_bytes(heads, n_q, dim, rank, segs, n_segs);
    KVC_REQUIRE(ws_bytes >= need, KVC_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    KVC_PTR(ws, true, "ws");
    char* w = static_cast<char*>(ws);
    auto* q_proj = reinterpret_cast<uint16_t*>(w);
    w += align_up(size_t(heads) * size_t(n_q) * rank * 4);
    hipError_t e = kvc::launch_project_queries(heads, n_q, dim, rank, q, basis_k, q_proj, stream);
    if (e != hipSuccess) return hip_status(e, "project queries");
    int di = 0;
    for (int i = 0; i < n_segs; ++i) {
      if (segs[i].n_tokens == 0) continue;
      const int C = segs[i].n_centroids;
      const size_t tb = align_up(size_t(heads) * C * rank * 2);
      auto* pk = reinterpret_cast<uint16_t*>(w);
      auto* pv = reinterpret_cast<uint16_t*>(w + tb);
      w += 2 * tb;
      e = kvc::launch_project_centres(heads, C, dim, rank, cdt, segs[i].k_cent, basis_k, pk, stream);
      if (e != hipSuccess) return hip_status(e, "project centres");
      e = kvc::launch_project_centres(heads, C, dim, rank, cdt, segs[i].v_cent, basis_v, pv, stream);
      if (e != hipSuccess) return hip_status(e, "project centres");
      sl.s[di].k_tab = pk;
      sl.s[di].v_tab = pv;
      ++di;
    }
    const int n_split = kvc::attend_split_plan(heads, n_q, sl.total_tiles, kvc::kLowdimRows);
    float* part_out = out;
    float* part_lse = lse;
    if (n_split > 1) {
      part_out = reinterpret_cast<float*>(w);
      w += align_up(size_t(n_split) * heads * n_q * dim * 4);
      part_lse = reinterpret_cast<float*>(w);
    }
    e = kvc::launch_attend_lowdim(heads, n_q, dim, rank, q_proj, basis_v, sl, kb, vb, g, n_split, part_out, part_lse,
                                  stream);
    if (e != hipSuccess) return hip_status(e, "attend low-dim");
    if (n_split > 1) {
      e = kvc::launch_lse_merge_strided(heads, n_q, dim, n_split, part_out, part_lse, out, lse, stream);
      if (e != hipSuccess) return hip_status(e, "split merge");
    }
    return ok();
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_attend_lowdim");
  }
}

// ------------------------------------------------------------------------------ merge
kvc_status kvc_lse_merge(int32_t heads, int64_t n_q, int32_t dim, int32_t n_parts, const float* const* outs,
                         const float* const* lses, float* out, float* lse, hipStream_t stream) {
  try {
    KVC_REQUIRE(heads >= 0 && n_q >= 0, KVC_ERR_INVALID_ARG, "heads and n_q must be >= 0");
    KVC_REQUIRE(dim > 0 && dim % 4 == 0 && 256 % (dim / 4) == 0, KVC_ERR_INVALID_ARG,
                "dim must be a multiple of 4 dividing 1024");
    KVC_REQUIRE(n_parts >= 1, KVC_ERR_INVALID_ARG, "n_parts must be >= 1");
    const bool work = heads > 0 && n_q > 0;
    KVC_REQUIRE(!work || (outs != nullptr && lses != nullptr), KVC_ERR_INVALID_ARG, "outs/lses is NULL");
    KVC_PTR(out, work, "out");
    KVC_PTR(lse, work, "lse");
    if (!work) return ok();
    for (int p = 0; p < n_parts; ++p) {
      KVC_PTR(outs[p], true, "outs[p]");
      KVC_PTR(lses[p], true, "lses[p]");
      if (p > 0)
        KVC_REQUIRE(outs[p] != out && lses[p] != lse, KVC_ERR_INVALID_ARG,
                    "only part 0 may alias the output");
    }
    return hip_status(kvc::launch_lse_merge(heads, n_q, dim, n_parts, outs, lses, out, lse, stream), "lse merge");
  } catch (...) {
    return fail(KVC_ERR_HIP, "unexpected exception in kvc_lse_merge");
  }
}

}  // extern "C"
