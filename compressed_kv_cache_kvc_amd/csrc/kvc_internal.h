// Internal declarations shared by the host dispatcher and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/kvc.h"

namespace kvc {

constexpr int kMaxSegs = 24;        // history segments walked by one attention launch (kernel-argument size)
constexpr int kMaxMergeParts = 32;  // parts merged by one launch of the merge kernel

// Device-side view of one segment (kernel argument).
struct SegDev {
  int64_t n_tokens;
  int64_t tile_begin;               // first global tile index of this segment
  int64_t n_centroids;              // C: head stride of the centre tables
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint32_t* k_meta;           // one 32-bit word (scale | zero << 16) per group
  const uint32_t* v_meta;
  const uint8_t* k_ids;
  const uint8_t* v_ids;
  const void* k_cent;
  const void* v_cent;
  // fp16 centre tables in tile channel order [heads][C][code dim] (workspace):
  // the centres themselves (full dim) or their projections (low dim)
  const uint16_t* k_tab;
  const uint16_t* v_tab;
  // kept key-error coefficients of the logit compensation [heads][n][8] fp16, or NULL
  const uint16_t* psac;
};

struct SegList {
  SegDev s[kMaxSegs];
  int n;
  int64_t total_tiles;
};

// ---------------------------------------------------------------- launchers (return hipError_t)
hipError_t launch_encode(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C,
                         const void* cent, const uint8_t* ids, const float* basis, int rank,
                         int bits, int group, uint8_t* codes, uint16_t* meta, hipStream_t st);

// Nearest-centre ids; the centre norms are computed inside the kernel.
hipError_t launch_assign(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C,
                         const void* cent, uint8_t* ids, hipStream_t st);
constexpr int kAssignMinGroups = 1024;  // assignment workgroups a launch aims for (2 per compute unit, 2 rounds)
// k-means update (per-centre means over the members in a fixed order); ws of
// kmeans_update_workspace(heads, n, C) bytes holds the member lists of long
// heads (update_global_lists) and is otherwise reserved.
hipError_t launch_kmeans_update(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C,
                                void* cent, const uint8_t* ids, void* ws, hipStream_t st);
size_t kmeans_update_workspace(int heads, int64_t n, int C);
bool update_global_lists(int heads, int64_t n);
constexpr int kSortedUpdateMaxTokens = 32768;   // heads up to this length: member lists sorted in LDS,
constexpr int kGlobalListTokens = 8192;         // unless longer than this and at most kGlobalListMaxHeads
constexpr int kGlobalListMaxHeads = 511;        // of them: then sorted once per head in the workspace
constexpr int kUpdateMinGroups = 1024;          // centre-update workgroups a launch aims for
constexpr int kGlobalListMaxSplit = 64;         // workgroups per head of the update over global lists, at most
constexpr int kListMinGroups = 512;             // member-list sort: workgroups a launch aims for,
constexpr int kListChunkTokens = 4096;          // chunks of at least this many tokens,
constexpr int kListChunkWaves = 4;              // of this many wavefronts

// Query-aware assignment (QSAC) of key tokens; n_cand in {1, 2, 4, 8}, group 16 or 32;
// w [heads][dim] fp32 or NULL (all ones).
hipError_t launch_assign_qsac(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C,
                              const void* cent, const float* w, int n_cand, int group, uint8_t* ids,
                              hipStream_t st);
// Logit compensation: running query second-moment matrices [heads][dim][dim], their
// top-kPsacRank eigenvectors [heads][dim][kPsacRank] (+ eigenvalues), and the kept
// key-error coefficients [heads][n][kPsacRank] fp16.
hipError_t launch_query_moments(int heads, int64_t n_q, int dim, kvc_dtype dt, const void* q, int64_t n_prev,
                                float* m, hipStream_t st);
hipError_t launch_psac_basis(int heads, int dim, const float* m, int n_iter, const float* u_prev, float* u,
                             float* lam, hipStream_t st);
hipError_t launch_psac_coeffs(int heads, int64_t n, int dim, kvc_dtype dt, const void* x, int C, const void* cent,
                              const uint8_t* ids, const uint8_t* codes, const uint16_t* meta, int bits, int group,
                              const float* u, uint16_t* coef, hipStream_t st);
// Running per-channel second moments of the queries (w updated in place); ws holds
// query_stats_workspace(heads, n_q, dim) bytes of per-block fp64 partial sums.
hipError_t launch_query_stats(int heads, int64_t n_q, int dim, kvc_dtype dt, const void* q, int64_t n_prev,
                              float* w, void* ws, hipStream_t st);
size_t query_stats_workspace(int heads, int64_t n_q, int dim);

hipError_t launch_lse_merge(int heads, int64_t n_q, int dim, int n_parts, const float* const* outs,
                            const float* const* lses, float* out, float* lse, hipStream_t st);
hipError_t launch_lse_merge_strided(int heads, int64_t n_q, int dim, int n_parts,
                                    const float* outs, const float* lses, float* out, float* lse,
                                    hipStream_t st);

// Full-dim attention.  If n_split > 1, writes partial (out, lse) for split s at
// part_out + s*heads*n_q*dim and part_lse + s*heads*n_q.
// u_psac: NULL, or [heads][dim][kPsacRank] fp32 principal query directions; then
// every segment carries its kept key-error coefficients (SegDev::psac).
hipError_t launch_attend(int heads, int64_t n_q, int dim, kvc_dtype q_dtype, const void* q,
                         const SegList& segs, int k_bits, int v_bits, int group, kvc_dtype cdt,
                         int n_split, float* out, float* lse, hipStream_t st, const float* u_psac = nullptr);
constexpr int kPsacRank = 8;           // kept directions of the logit compensation

// Reduced queries q' = U^T q as two fp16 arrays [heads][n_q][rank] (tile channel
// order): q_proj holds fp16(q') and q_proj + heads*n_q*rank the fp16 rounding of
// the remainder q' - fp16(q'), so that their sum carries q' to about 2^-22.
hipError_t launch_project_queries(int heads, int64_t n_q, int dim, int rank, const void* q,
                                  const float* basis, uint16_t* q_proj, hipStream_t st);
hipError_t launch_project_centres(int heads, int C, int dim, int rank, kvc_dtype cdt,
                                  const void* cent, const float* basis, uint16_t* tab,
                                  hipStream_t st);
// fp16 centre tables (k_tab, v_tab, already pointed into the workspace) of every
// segment from its bf16 centres, in one launch
hipError_t launch_centre_tables(int heads, int dim, const SegList& segs, hipStream_t st);
hipError_t launch_attend_lowdim(int heads, int64_t n_q, int dim, int rank,
                                const uint16_t* q_proj, const float* basis_v,
                                const SegList& segs, int k_bits, int v_bits, int group,
                                int n_split, float* out, float* lse, hipStream_t st);

// Predictive residual codec over latent frames (encode, or decode to fp16
// reconstructions); k/v are read only when encoding, k_hat/v_hat written only
// when decoding; the state [heads][S][3][dim] fp32 is read when first_frame > 0
// and written at the end.
hipError_t launch_tempo(bool decode, int heads, int S, int first_frame, int n_frames, int dim, kvc_dtype dt,
                        const void* k, const void* v, const float* prm, int kb, int vb, int g, uint8_t* k_codes,
                        uint16_t* k_meta, uint8_t* v_codes, uint16_t* v_meta, float* state, uint16_t* k_hat,
                        uint16_t* v_hat, hipStream_t st);

// Split plan shared by the dispatcher and the workspace-size queries.
int attend_split_plan(int heads, int64_t n_q, int64_t total_tiles, int rows_per_block);

constexpr int kAttendTile = 64;        // history tokens per tile
constexpr int kAttendRows = 256;       // queries per workgroup (full-dim path)
constexpr int kLowdimRows = 256;       // queries per workgroup (low-dim path)

}  // namespace kvc
