/*
 * kvc.h -- C ABI of the compressed KV-cache hot path on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources: the text of web pages on compressed KV
 * caches for autoregressive video generation):
 *   - each head's cached key and value tokens are stored as the id of their
 *     nearest centre plus a 2- or 4-bit residual (QuantWM, section 4.1, on the
 *     centroid-residual scheme of QVG; NanoKV, Table 4: 256 centres per head
 *     for K and V, two k-means iterations);
 *   - the residual against the centre (TempoKV, section 3.3, Eq. 2) is
 *     quantized per group of g channels by the affine min/max quantizer of
 *     TempoKV, section 3.1, Eq. 1, with an fp16 scale and zero-point per group;
 *   - the current chunk's queries attend over the history reconstructed on the
 *     fly as centre + dequantized residual, returning the outputs and the
 *     log-sum-exp (LSE) of each row so that parts of the history can be merged
 *     (NanoKV, Figure 4d);
 *   - far history can instead be held as quantized coefficients in a reduced
 *     basis and read in low dimension (NanoKV, Figure 4a and 4d).
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers owned by the caller.  Pointer
 *     arrays (kvc_segment lists, the per-part pointers of kvc_lse_merge) are
 *     HOST arrays holding device pointers; they are read before the call
 *     returns and may be released afterwards.
 *   - Every call is asynchronous on `stream` (0 = the null stream).  The
 *     library never allocates, frees or synchronizes; scratch memory comes from
 *     the caller as a workspace whose size the matching *_workspace_bytes
 *     function returns.
 *   - Arrays are dense, row-major, with the head index outermost:
 *       x, centroids ....... [heads][n][dim] in the storage dtype (fp32 or bf16)
 *       ids ................ [heads][n] uint8 (C <= 256)
 *       codes .............. [heads][n][code_dim * bits / 8] uint8; code_dim = dim,
 *                            or rank for coefficient codes.  Channel c of a row
 *                            sits in byte c / (8/bits) at bit offset
 *                            bits * (c % (8/bits)), least significant first.
 *       meta ............... [heads][n][code_dim / group][2] fp16 bit patterns
 *                            (scale, zero-point) per group, scale first.
 *       q, out ............. [heads][n_q][dim]; lse [heads][n_q] fp32, natural log.
 *       basis .............. [heads][dim][rank] fp32, orthonormal columns.
 *   - Every pointer must be 16-byte aligned.  Outputs must not alias inputs.
 *   - Inputs are read only; outputs are fully overwritten (code padding = 0).
 *   - Errors are returned before any launch: KVC_ERR_INVALID_ARG for malformed
 *     arguments, KVC_ERR_UNSUPPORTED for valid combinations without a built
 *     kernel, KVC_ERR_WORKSPACE when the workspace is too small, KVC_ERR_HIP
 *     when the HIP runtime reports a launch error.  kvc_last_error() then holds
 *     a thread-local message.  No C++ exception crosses this interface.
 *   - Results are deterministic: assignment and encoding bit for bit, fitting
 *     with fixed-order fp64 sums, attention for a given split plan.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = 1,
  KVC_ERR_UNSUPPORTED = 2,
  KVC_ERR_WORKSPACE = 3,
  KVC_ERR_HIP = 4
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* One contiguous run of encoded history that shares one centre table per head
 * and tensor (a cache block, compressed as a unit).  rank = 0 means full-dim
 * codes; rank > 0 means coefficient codes in a rank-dimensional basis.  All
 * arrays cover every head of the call, head-major, with n_tokens per head. */
typedef struct {
  int64_t n_tokens;
  int32_t n_centroids;          /* C, 1..256 */
  int32_t rank;                 /* 0 or the coefficient dimension */
  int32_t k_bits, v_bits;       /* 2 or 4 each */
  int32_t group;                /* channel-group size g of the quantizer */
  kvc_dtype cent_dtype;         /* dtype of the centre tables */
  const uint8_t *k_codes, *v_codes;
  const uint16_t *k_meta, *v_meta;
  const uint8_t *k_ids, *v_ids;
  const void *k_cent, *v_cent;  /* [heads][C][dim], full dimension even when rank > 0 */
} kvc_segment;

/* Lloyd k-means per head (QuantWM, section 4.1; NanoKV, Table 4: two
 * iterations), then a final assignment.
 *   x          [heads][n_tokens][dim], dtype dt.
 *   centroids  [heads][n_centroids][dim], dtype dt; in: initial centres, out:
 *              fitted centres.  Each iteration moves a centre to the mean of its
 *              members (fp64 sum in a fixed order, one division, rounded to
 *              nearest even in dt); a centre without members keeps its value.
 *   n_iters    >= 0 (0 = assignment only).
 *   ids_out    [heads][n_tokens]: argmin over centres of the squared L2 distance,
 *              ties to the lowest index.
 *   ws         workspace of at least kvc_fit_assign_workspace_bytes(...) bytes:
 *              with n_tokens > 32768, or n_tokens > 8192 and heads <= 511, it
 *              holds every head's member lists, sorted once per head (4 * heads
 *              * (n_tokens + n_centroids + 1) bytes), the sort's per-chunk counts
 *              when a head is sorted in several chunks, and 256 bytes; otherwise
 *              256 bytes, reserved (the update keeps its member lists in LDS).
 * dim must be 64 or 128; n_centroids 1..256; n_tokens < 2^31 (token indices
 * are 32-bit); heads <= 65535 (KVC_ERR_UNSUPPORTED above); n_tokens >=
 * n_centroids is not required.  Tokens must be finite: a token with a NaN or an infinite value has
 * no finite distance and is assigned id 0 (its codes and the centre update are
 * then meaningless, but every id stays a valid index). */
kvc_status kvc_fit_assign(int32_t heads, int64_t n_tokens, int32_t dim, kvc_dtype dt,
                          const void* x, int32_t n_centroids, void* centroids,
                          int32_t n_iters, uint8_t* ids_out,
                          void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvc_fit_assign_workspace_bytes(int32_t heads, int64_t n_tokens, int32_t dim,
                                      int32_t n_centroids);

/* Query-aware assignment of key tokens, QSAC (QuantWM, section 4.1, Eqs. 9-12).
 * Per token x: the n_cand centres nearest in d_w(x, mu) = sum_c w_c (x_c - mu_c)^2
 * are candidates (ties to the lower index); each is scored by
 * S = sum_g (sum_{c in g} w_c) (max_{c in g} r_c - min_{c in g} r_c)^2 with
 * r = x - mu and g the channel groups of the residual codec; the token takes the
 * smallest score, ties to the lower index.  n_cand = 1 with w = NULL is the plain
 * nearest-centre assignment.
 *   x, centroids  [heads][n_tokens][dim] / [heads][n_centroids][dim], dtype dt.
 *   w          NULL (all channel weights 1: the cold start) or [heads][dim] fp32
 *              non-negative weights, e.g. from kvc_query_stats.
 *   n_cand     1, 2, 4 or 8 (others: KVC_ERR_UNSUPPORTED).
 *   group      16 or 32, dividing dim.
 *   ids_out    [heads][n_tokens].
 * bf16 candidate sets are exact (a near tie at the candidate boundary is
 * re-scored in fp64); candidate scores are fp32 for bf16 and fp64 for fp32
 * tokens.  No workspace; dim 64 or 128; heads <= 65535. */
kvc_status kvc_assign_qsac(int32_t heads, int64_t n_tokens, int32_t dim, kvc_dtype dt,
                           const void* x, int32_t n_centroids, const void* centroids,
                           const float* w, int32_t n_cand, int32_t group, uint8_t* ids_out,
                           hipStream_t stream);

/* Running second moments of the queries per head and channel (QuantWM, section
 * 4.1, Eqs. 6-8, diagonal): w <- (n_prev * w + sum_i q_ic^2) / (n_prev + n_q),
 * summed in fp64 in a fixed order.  With n_prev = 0 the previous contents of w
 * are ignored.
 *   q   [heads][n_q][dim], dtype q_dtype;  w  [heads][dim] fp32, in/out.
 *   ws  at least kvc_query_stats_workspace_bytes(...) bytes (fp64 partial sums of
 *       blocks of queries, added in block order). */
kvc_status kvc_query_stats(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype,
                           const void* q, int64_t n_prev, float* w, void* ws, size_t ws_bytes,
                           hipStream_t stream);
size_t kvc_query_stats_workspace_bytes(int32_t heads, int64_t n_q, int32_t dim);

/* Principal-subspace logit compensation, PSAC (QuantWM, section 4.2, Eqs. 13-17;
 * r = 8 kept directions).
 * kvc_query_moments: running second-moment matrices of the queries,
 *   M <- (n_prev * M + sum_i q_i q_i^T) / (n_prev + n_q); q [heads][n_q][dim],
 *   m [heads][dim][dim] fp32 in/out (ignored on input when n_prev = 0).
 * kvc_psac_basis: the r eigenvectors of the largest eigenvalues of each M, as
 *   u [heads][dim][r] fp32 (column k = k-th largest; its largest component
 *   positive) and lam [heads][r]; subspace iteration (n_iter products with M and
 *   re-orthonormalization, then Rayleigh-Ritz), started from u_prev when given.
 * kvc_psac_coeffs: kept coefficients of the keys' remaining quantization error,
 *   coef [heads][n][r] fp16 = (x - (c[id] + q*s + z)) u, from the same x,
 *   centroids, ids, codes and meta (2/4-bit, group 16/32) that kvc_encode used.
 * kvc_attend_psac: kvc_attend with every logit corrected by (u^T q) . coef_j,
 *   i.e. attention on k_hat_j + u u^T (k_j - k_hat_j); coefs is a HOST array of
 *   n_segs device pointers (one per segment, [heads][n_tokens][r] fp16); dim 128,
 *   bf16 queries, 2/4-bit segments.  Workspace as for kvc_attend. */
kvc_status kvc_query_moments(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype,
                             const void* q, int64_t n_prev, float* m, hipStream_t stream);
kvc_status kvc_psac_basis(int32_t heads, int32_t dim, const float* m, int32_t r, int32_t n_iter,
                          const float* u_prev, float* u, float* lam, hipStream_t stream);
kvc_status kvc_psac_coeffs(int32_t heads, int64_t n_tokens, int32_t dim, kvc_dtype dt,
                           const void* x, int32_t n_centroids, const void* centroids,
                           const uint8_t* ids, const uint8_t* codes, const uint16_t* meta,
                           int32_t bits, int32_t group, const float* u, int32_t r,
                           uint16_t* coef, hipStream_t stream);
kvc_status kvc_attend_psac(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype,
                           const void* q, const float* u, int32_t r, const kvc_segment* segs,
                           const uint16_t* const* coefs, int32_t n_segs, float* out, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvc_attend_psac_workspace_bytes(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype,
                                       const kvc_segment* segs, int32_t n_segs);

/* Frame routing of mixed-dimensional attention (NanoKV, Figure 4 and appendix
 * Table 7): frame f of a history of n_frames latent frames (0 = oldest) is read
 * at full dimension (full_dim[f] = 1) when n_frames <= all_full_until, or f >=
 * n_frames - n_recent, or f < n_sink, or period > 0 and f % period == 0 (one
 * anchor per `period` older frames, the first of each window); otherwise through
 * the reduced maps (0).  Host memory; no GPU work. */
kvc_status kvc_route_frames(int32_t n_frames, int32_t n_recent, int32_t period, int32_t n_sink,
                            int32_t all_full_until, uint8_t* full_dim);
/* Anchor precision (TempoKV, section 3.3 and Table 7): b_a = max(4, b_K, b_V). */
int32_t kvc_anchor_bits(int32_t k_bits, int32_t v_bits);

/* Predictive residual coding over latent frames (TempoKV, section 3.3, Eqs. 2-4
 * and "Anchor frames").  A head's tokens are frames of frame_tokens = S spatial
 * tokens, token f*S + s being spatial token s of frame f of the call; a call
 * codes frames first_frame .. first_frame + n_frames - 1.  Per token and frame t:
 *   keys (Eq. 3):    K~ = beta_K + A1 (.) K^[t-1] + A2 (.) K^[t-2]; frame 1 uses its
 *                    own (beta_K1, A_K1) and no A2 term; the anchor frame 0 has K~ = 0;
 *   values (Eq. 4):  V~ = beta_V + W K^[t] + A_V (.) V^[t-1]; frame 0 has V~ = 0;
 *   both (Eq. 2):    r = x - x~ quantized by the group quantizer of kvc_encode
 *                    (fp16 scale rounded up, fp16 zero-point rounded down, codes
 *                    and metadata laid out as for kvc_encode), x^ = x~ + (q*s + z).
 * fp32 arithmetic in one fixed order, no fused multiply-add: x~ of a key is
 * ((beta + A1*k1) + A2*k2); the W term adds W[c][j]*K^[j] for j ascending to beta_V,
 * then A_V*v1 is added; r = x - x~; x^ = x~ + (q*s + z).
 *   params   [heads][kvc_tempo_param_count(dim)] fp32 per head: beta_K1, A_K1,
 *            beta_K2, A_K21, A_K22, beta_V, A_V (dim values each), then W row-major
 *            (W[c][j] multiplies K^[j] into channel c), e.g. fitted offline by ridge
 *            regression (TempoKV, Eq. 5).
 *   state    [heads][S][3][dim] fp32: K^[f-1], K^[f-2], V^[f-1] before the call's
 *            first frame f (read when first_frame > 0, ignored for the anchor);
 *            overwritten with the same three rows after its last frame, so
 *            consecutive calls continue the sequence.
 *   The anchor frame is coded alone (first_frame = 0 needs n_frames = 1) at
 *   b_a = max(4, b_K, b_V) = 4 bits: k_bits = v_bits = 4 in that call.
 * kvc_tempo_encode: k, v [heads][n_frames*S][dim] (dtype dt) -> k_codes/v_codes
 *   [heads][n_frames*S][dim*bits/8], k_meta/v_meta [heads][n_frames*S][dim/group][2].
 * kvc_tempo_decode: the same codes (and the same state before the call) ->
 *   k_hat, v_hat [heads][n_frames*S][dim] as fp16 bit patterns (x^ rounded to
 *   nearest), bit for bit the encoder's reconstruction; the result reads through
 *   kvc_attend as a 16-bit residual segment over a zero centre table.
 * dim 64 or 128; bits 2 or 4; group 16 or 32.  No workspace. */
int32_t kvc_tempo_param_count(int32_t dim);
kvc_status kvc_tempo_encode(int32_t heads, int32_t frame_tokens, int32_t first_frame, int32_t n_frames,
                            int32_t dim, kvc_dtype dt, const void* k, const void* v, const float* params,
                            int32_t k_bits, int32_t v_bits, int32_t group, uint8_t* k_codes, uint16_t* k_meta,
                            uint8_t* v_codes, uint16_t* v_meta, float* state, hipStream_t stream);
kvc_status kvc_tempo_decode(int32_t heads, int32_t frame_tokens, int32_t first_frame, int32_t n_frames,
                            int32_t dim, const float* params, int32_t k_bits, int32_t v_bits, int32_t group,
                            const uint8_t* k_codes, const uint16_t* k_meta, const uint8_t* v_codes,
                            const uint16_t* v_meta, float* state, uint16_t* k_hat, uint16_t* v_hat,
                            hipStream_t stream);

/* Encode tokens against their centres (TempoKV, section 3.1 Eq. 1 and section
 * 3.3 Eq. 2).  Per token: r = fl32(x - c[id]); with a basis, r is replaced by
 * its coefficients a_k = sum_i fl32(U[i][k] * r[i]) accumulated in fp32 over
 * i ascending (multiply and add rounded separately).  Per group of `group`
 * coded channels: z = fp16 round-down of the minimum, s = fp16 round-up of
 * fl32((max - z) / (2^bits - 1)), zero values stored as +0; code q =
 * clamp(round-half-even(fl32(fl32(r - z) * fl32(1/s))), 0, 2^bits - 1), q = 0
 * when s = 0.
 *   ids_in     [heads][n_tokens] or NULL; NULL runs the assignment first.
 *   ws         kvc_encode_workspace_bytes(...) bytes (currently 0: encode keeps
 *              the argument so that a later version may stage data in it).
 *   ids_out    NULL, or where the ids used are written (may equal ids_in only
 *              when ids_in is NULL).
 *   basis      NULL or [heads][dim][rank] fp32; rank = 0 without a basis.
 *   bits       2 or 4; group divides the coded dimension (dim or rank).
 *              bits = 16 stores the residual itself, fp16 nearest-even per
 *              element ([heads][n_tokens][dim] fp16 in `codes`, 2*dim bytes a
 *              row), with no groups and no metadata (meta may be NULL; group is
 *              ignored); full dimension only (TempoKV, Table 7: 16-bit anchors).
 *   codes, meta  outputs as laid out above.
 * Supported: dim 64 or 128; group 16 or 32 (and group <= coded dimension);
 * rank 0, or 32 or 64 with dim 128. */
kvc_status kvc_encode(int32_t heads, int64_t n_tokens, int32_t dim, kvc_dtype dt,
                      const void* x, int32_t n_centroids, const void* centroids,
                      const uint8_t* ids_in, uint8_t* ids_out,
                      const float* basis, int32_t rank, int32_t bits, int32_t group,
                      uint8_t* codes, uint16_t* meta,
                      void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvc_encode_workspace_bytes(int32_t heads, int64_t n_tokens, int32_t dim,
                                  int32_t n_centroids, int32_t ids_given);

/* Attention of n_q queries per head over the concatenation of n_segs history
 * segments (full-dimensional codes, rank = 0), each token reconstructed on
 * demand as its prediction plus the dequantized residual (TempoKV, section 3.3,
 * Eq. 2, with the centre as the prediction; QuantWM, Figure 9: packed storage
 * read back by on-demand reconstruction during streaming inference):
 * S = q . k_hat / sqrt(dim), k_hat = c_K[id] + q*s + z, likewise v_hat;
 * out = softmax(S) V_hat, lse = ln sum exp(S), the log-sum-exp by which parts of
 * the history merge (NanoKV, Figure 4d).  No mask.  An empty history gives
 * out = 0, lse = -inf.
 *   q          [heads][n_q][dim], dtype q_dtype (bf16; fp32 selects an fp32 path).
 *   segs       host array of n_segs descriptors; every segment must share the
 *              codec parameters (k_bits, v_bits, group, cent_dtype); each has its
 *              own centre tables.
 *   out, lse   fp32 outputs.
 *   ws         at least kvc_attend_workspace_bytes(...) bytes (partial results of
 *              the split over history, merged by LSE inside the call).
 * Limits: heads <= 65535 and ceil(n_q / 256) * heads <= 2^20; fp32 queries
 * n_q <= 2^26; a 2/4-bit segment holds at most 2^25 tokens per head, a 16-bit
 * residual segment at most 2^24 (else KVC_ERR_UNSUPPORTED); the same limits hold
 * for kvc_attend_lowdim. */
kvc_status kvc_attend(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                      const kvc_segment* segs, int32_t n_segs, float* out, float* lse,
                      void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvc_attend_workspace_bytes(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype,
                                  const kvc_segment* segs, int32_t n_segs);

/* kvc_attend for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace kvc_attend would take (kvc_attend_workspace_bytes) is instead a
 * static device array of KVC_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held from the first use on that GPU until the process ends; the call
 * itself allocates and frees nothing.  Same arguments (minus the workspace),
 * validation, kernels and results as kvc_attend.  A call whose workspace would
 * exceed the array returns KVC_ERR_WORKSPACE before any launch (e.g. 24 heads
 * over ten 256-centre segments need 31 MiB and fit; 720 heads over ten do not).
 * Every call on one GPU shares that GPU's array and leaves its contents behind
 * (nothing in it needs to start at zero), so calls that overlap on one GPU, on
 * different streams or from different threads, race: serialize them. */
#define KVC_NOALLOC_SCRATCH_BYTES (64u << 20)
kvc_status kvc_attend_noalloc(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype, const void* q,
                              const kvc_segment* segs, int32_t n_segs, float* out, float* lse,
                              hipStream_t stream);

/* Low-dimensional attention over coefficient-coded segments (NanoKV, Figure 4a
 * and 4d): q' = U_K^T q; k' = U_K^T c_K[id] + a_hat_K; S = q'.k' / sqrt(dim);
 * O' = softmax(S) (U_V^T c_V[id] + a_hat_V); out = U_V O'.  Returns lse as
 * kvc_attend does, so that the result LSE-merges with a full-dim part.
 *   basis_k, basis_v  [heads][dim][rank] fp32, the bases the segments were
 *                     encoded with (every segment must have this rank).
 * Supported: dim 128, rank 32 or 64, bf16 queries and centres. */
kvc_status kvc_attend_lowdim(int32_t heads, int64_t n_q, int32_t dim, kvc_dtype q_dtype,
                             const void* q, const float* basis_k, const float* basis_v,
                             int32_t rank, const kvc_segment* segs, int32_t n_segs,
                             float* out, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream);
size_t kvc_attend_lowdim_workspace_bytes(int32_t heads, int64_t n_q, int32_t dim, int32_t rank,
                                         const kvc_segment* segs, int32_t n_segs);

/* Merge n_parts attention results of the same queries (NanoKV, Figure 4d):
 * lse = ln sum_p exp(lse_p), out = sum_p exp(lse_p - lse) out_p.  Parts with
 * lse = -inf contribute nothing; if every part is -inf the result is
 * out = 0, lse = -inf.
 *   outs, lses  HOST arrays of n_parts device pointers ([heads][n_q][dim] and
 *               [heads][n_q] fp32).  out/lse may alias outs[0]/lses[0]. */
kvc_status kvc_lse_merge(int32_t heads, int64_t n_q, int32_t dim, int32_t n_parts,
                         const float* const* outs, const float* const* lses,
                         float* out, float* lse, hipStream_t stream);

const char* kvc_status_string(kvc_status status);
/* Message of the last failed call on this thread ("" if none). */
const char* kvc_last_error(void);
/* Library version string. */
const char* kvc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
