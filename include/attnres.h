/*
 * attnres.h -- C ABI of the MI355X (gfx950) Block / Full Attention Residuals
 * depth-aggregation library (libattnres.so).
 *
 * What it computes.  For every token t and every target sublayer l, a learned,
 * input-independent pseudo-query w_l scores each depth source u as
 *     z(u) = w_l^T ( g_l (.) u / r(u) ),   r(u) = sqrt(mean_k u_k^2 + eps),
 * the scores are softmaxed over the site's sources and weight the raw sources:
 *     h_l = sum_u softmax(z)_u * u.
 * Sources: "Attention Residuals" (structured notes on arXiv 2603.15031),
 * section 7 "Full AttnRes" for the score/softmax/aggregation, and
 * "Attention Residuals 阅读补充", section "RMSNorm 的数学原理" for RMSNorm.
 * In Block AttnRes (same notes, section 8) the sources of a sublayer in block
 * n are the embedding b_0, the completed block sums b_1..b_{n-1} and, after
 * the block's first sublayer, the running partial sum of block n.
 *
 * The work is split as in the notes' section 10 (two-phase inference) and the
 * reading notes' section on static queries and two-phase computation:
 *   - attnres_phase1: one batched pass per block; each completed-block source
 *     row is read once and serves all S pseudo-queries of the block.  Returns
 *     the normalised partial outputs and their softmax statistics.
 *   - attnres_phase2_merge: one call per sublayer; adds the previous
 *     sublayer's output to the partial sum, scores the partial sum, merges it
 *     with the phase-1 partition exactly (online softmax), and applies the
 *     consuming sublayer's PreNorm RMSNorm in the same pass.
 *   - attnres_block_accumulate: b_n = partial + last output of the block.
 *   - attnres_full: one-shot aggregation of n sources with one query (Full
 *     AttnRes, or the final aggregation over b_0..b_N), optional PreNorm.
 *
 * Conventions for every entry point:
 *  - Storage dtype `dt` (fp32 or bf16) for rows of sources and outputs; all
 *    arithmetic is fp32; bf16 results are rounded to nearest even.
 *    Parameters (w, key_gain, prenorm_gain) are fp32 [.., d] rows.
 *  - Layout: row-major, token-major rows of d channels.  A row set [T][d] is
 *    contiguous.  Multi-source inputs are slabs src + i*src_stride (elements).
 *  - d must be a multiple of 8 and at most 16384; strides multiples of 8,
 *    in [0, ATTNRES_MAX_STRIDE]; 0 <= T <= ATTNRES_MAX_T (anything else is
 *    ATTNRES_EINVAL); row and parameter pointers 16-byte aligned, statistics
 *    ([T] / [S][T] fp32) pointers 4-byte aligned.
 *  - All pointers except `stream` are device pointers owned by the caller.
 *    The library allocates nothing and keeps no state beyond loaded kernels.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Calls
 *    are asynchronous; argument errors are reported synchronously before any
 *    launch; a failed launch reports ATTNRES_EHIP.
 *  - T == 0 is valid and launches nothing; it returns ATTNRES_OK once the
 *    scalar arguments (dtype, d, counts, eps) are valid, whatever the
 *    pointers are (empty tensors may have null data pointers).
 *  - Kernels use no atomics: results are bitwise reproducible run to run and
 *    independent of how tokens are split over calls.
 */
#ifndef ATTNRES_H
#define ATTNRES_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTNRES_OK = 0,
    ATTNRES_EINVAL = 1,  /* null pointer, bad size, unsupported size combination */
    ATTNRES_EDTYPE = 2,  /* unknown dtype */
    ATTNRES_EALIGN = 3,  /* d or a stride not a multiple of 8, pointer not 16-byte aligned */
    ATTNRES_EALIAS = 4,  /* an output overlaps an input (other than the allowed in-place case) */
    ATTNRES_EHIP = 5,    /* the HIP runtime reported an error at launch */
    ATTNRES_ESCRATCH = 6 /* more workspace than attnres_phase1_noalloc holds */
} attnres_status_t;

/* Storage formats.  ATTNRES_P24 and ATTNRES_Q16 are only valid for the
 * running partial sum of a block (partial_in / partial_out).
 * P24: the fp32 value rounded to nearest even at bit 8 of its encoding and
 * kept as its upper 24 bits, stored as two planes -- T*d 16-bit upper halves
 * followed by T*d bytes holding bits 8..15 (3 bytes per element; full fp32
 * range, relative step 2^-16).
 * Q16: 16-bit fixed point with one power-of-two scale per row -- T*d int16
 * values q followed by T int32 row exponents e (2 bytes per element plus 4
 * per row); element k of row t is q[t][k] * 2^(e[t] - 15), where e[t] is
 * the smallest exponent with every |value| of the row below 2^e[t], and q is
 * the value times 2^(15 - e[t]) rounded to nearest even (|q| <= 32767): every
 * element is kept to within 2^-15 of the row's largest magnitude.  Finite
 * values only.  The buffer must be 16-byte aligned. */
typedef enum { ATTNRES_F32 = 0, ATTNRES_BF16 = 1, ATTNRES_P24 = 2, ATTNRES_Q16 = 3 } attnres_dtype_t;

/* Largest supported values. */
#define ATTNRES_MAX_D 16384
#define ATTNRES_MAX_SOURCES 32          /* attnres_full / phase 1 with S == 1 */
#define ATTNRES_MAX_SOURCES_MULTI 16    /* phase 1 with S >= 2 */
#define ATTNRES_MAX_GROUP_SOURCES 16    /* attnres_phase2_merge_multi */
#define ATTNRES_MAX_T 2147483647LL      /* tokens per call */
#define ATTNRES_MAX_QUERIES 4096        /* S of phase 1 */
#define ATTNRES_MAX_STRIDE (1LL << 40)  /* slab strides, in elements; strides are >= 0 */

/*
 * Phase 1 of a block ("Attention Residuals" notes, section 10, first phase;
 * "Attention Residuals 阅读补充", static-query batching Q K^T).
 * For each token t and each query s < S, over the n_src completed sources
 * u_i = src + i*src_stride (each [T][d], dtype src_dt):
 *     z_si = w_s^T (key_gain_s (.) u_i / r(u_i)),  m_s = max_i z_si,
 *     lse_s = m_s + ln sum_i e^{z_si - m_s},
 *     out[s][t][:] = sum_i e^{z_si - lse_s} u_i        (normalised)
 *   w, key_gain: [S][d] fp32 (key_gain NULL = ones).
 *   out: [S][T][d] dtype dt, or NULL to compute the statistics only (with a
 *   single source every output equals that source, so a caller can use the
 *   source row itself in phase 2).  m_out, lse_out: [S][T] fp32 (m_out may
 *   be NULL).
 * Limits: 1 <= n_src <= ATTNRES_MAX_SOURCES_MULTI when S >= 2, <=
 * ATTNRES_MAX_SOURCES when S == 1; 1 <= S <= ATTNRES_MAX_QUERIES (queries are processed 32 at a
 * time; each group of 32 reads the sources once for the scores and once for
 * the outputs).
 * workspace: caller-owned device memory of at least
 * attnres_phase1_workspace_bytes(T, d, n_src, S) bytes, 16-byte aligned,
 * used for the queries packed as matrix-core operands and for the scores or
 * softmax weights between the scoring and output kernels (its contents
 * afterwards are unspecified).  Required for S >= 2.  For S == 1 it is not used (may be
 * NULL): one pass over the sources computes the site with an online softmax
 * (the running maximum and normaliser rescaled batch by batch, as in the
 * notes' log-sum-exp merge), reading every source row once.
 * out must not overlap src; m_out, lse_out and workspace must not overlap
 * anything.
 * src_dt: the sources' dtype, dt itself, or ATTNRES_F32 with dt ==
 * ATTNRES_BF16 (fp32 sources, bf16 outputs; then 1 <= n_src <=
 * ATTNRES_MAX_SOURCES_MULTI and the workspace is required for S == 1 too).
 * A training forward keeps the block sums exact this way: the notes'
 * section 8 defines b_n as the sum of the block's outputs, and storing it in
 * bf16 would change what the backward differentiates.  Any other pair is
 * ATTNRES_EDTYPE.
 */
attnres_status_t attnres_phase1(attnres_dtype_t dt, attnres_dtype_t src_dt,
                                const void* src, int64_t n_src, int64_t src_stride,
                                int64_t T, int64_t d,
                                const float* w, const float* key_gain, int64_t S, float eps,
                                void* out, float* m_out, float* lse_out,
                                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * attnres_phase1 without the caller's workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results (bit for bit),
 * limits and errors as attnres_phase1, except that the workspace is a device
 * array of ATTNRES_NOALLOC_SCRATCH_BYTES inside the library: one copy per
 * GPU, held until the process ends, its address looked up on the first call
 * on each device.  The call allocates nothing and calls no allocating
 * routine.  A call whose attnres_phase1_workspace_bytes(T, d, n_src, S)
 * exceeds ATTNRES_NOALLOC_SCRATCH_BYTES returns ATTNRES_ESCRATCH (64 MiB
 * covers, e.g., 16384 tokens with up to 16 sources and 32 queries, or 32768
 * tokens with 8 sources and 24 queries).  Every call on one GPU shares that
 * GPU's array, which keeps whatever the last call left there (nothing in it
 * needs to start at zero): calls that overlap in time on one GPU -- on
 * different streams, or from different host threads -- race on it and must
 * be serialised by the caller.
 */
#define ATTNRES_NOALLOC_SCRATCH_BYTES (64LL << 20)
attnres_status_t attnres_phase1_noalloc(attnres_dtype_t dt,
                                        const void* src, int64_t n_src, int64_t src_stride,
                                        int64_t T, int64_t d,
                                        const float* w, const float* key_gain, int64_t S, float eps,
                                        void* out, float* m_out, float* lse_out, void* stream);

/*
 * Phase 1 of a block with the first sublayer's input finished in the same
 * pass ("Attention Residuals" notes, section 10: the block's first sublayer
 * has no partial-sum source and takes the phase-1 result as is; its PreNorm,
 * fused as in "ML 研究者的三层基本功", system layer).  Computes everything
 * attnres_phase1 does, except that query 0's output o_0 is not written to
 * out: instead
 *     x_out[t][:] = prenorm_gain (.) h / r(h),   h = o_0 rounded to dt,
 * i.e. exactly what attnres_phase2_merge with sublayer_prev == NULL gives
 * from a stored o_0 (up to the order of the sum of squares).
 *   prenorm_gain: [d] fp32 (NULL = ones).  x_out: [T][d] dtype dt, required.
 *   h_out: [T][d] dtype dt or NULL; when given it receives o_0 (= h of the
 *   first sublayer).
 *   out: [S][T][d] as for attnres_phase1, slabs 1..S-1 hold queries
 *   1..S-1; slab 0 is scratch (its contents afterwards are unspecified).
 *   out may be NULL only when n_src == 1 (every query's output is then the
 *   source row itself).  m_out, lse_out: [S][T] fp32 for every query.
 * Limits and workspace as attnres_phase1 with S >= 2 (also required for
 * S == 1; n_src <= ATTNRES_MAX_SOURCES_MULTI).  x_out and h_out must not
 * overlap any input or other output.
 */
attnres_status_t attnres_phase1_first_prenorm(attnres_dtype_t dt,
                                              const void* src, int64_t n_src, int64_t src_stride,
                                              int64_t T, int64_t d,
                                              const float* w, const float* key_gain, int64_t S, float eps,
                                              void* out, float* m_out, float* lse_out,
                                              const float* prenorm_gain, void* x_out, void* h_out,
                                              void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Phase 1 of a block whose newest source, the previous block's sum, is
 * formed in the same call ("Attention Residuals" notes, section 8: b_n is the
 * sum of block n's sublayer outputs; "Attention Residuals 阅读补充", "如何解
 * 释小于 2% 的延迟": the small overhead rests on fusing such operators).
 * First
 *     u_{n_src-1} = ((partial_in or 0) + (sublayer_prev2 or 0)) + sublayer_prev,
 * summed in fp32 in that order and stored to source slab n_src-1 as src_dt --
 * the same values attnres_block_accumulate(sublayer_dt, T, d, partial_dt,
 * partial_in, sublayer_prev2, sublayer_prev, that slab, src_dt) stores -- then
 * everything attnres_phase1_first_prenorm does (x_out != NULL; src_dt must
 * equal dt) or attnres_phase1 does (x_out == NULL; prenorm_gain and h_out
 * must be NULL too), bit for bit, reading sources 0..n_src-2 from src.
 *   src: the n_src source slabs as for attnres_phase1; slab n_src-1 is
 *   written (its previous contents are not read).
 *   partial_in (format partial_dt, NULL = none), sublayer_prev2 (NULL =
 *   none), sublayer_prev (required): [T][d] pieces, the outputs of dtype
 *   sublayer_dt, as for attnres_block_accumulate; src_dt is sublayer_dt, or
 *   ATTNRES_F32 with bf16 outputs (exact block sums).  dt and src_dt pair as
 *   for attnres_phase1 (a training forward's final site: fp32 sources and
 *   outputs, bf16 pieces).
 * Over long token ranges (at least 64 tokens per compute unit) with a
 * partial_in in ATTNRES_Q16 or ATTNRES_F32 the sum is formed inside the
 * scoring pass, which reads the pieces instead of the slab and writes the
 * slab once; otherwise the call runs the block-sum kernel first.
 * Limits and workspace as the call it stands for, with 2 <= n_src.  No piece
 * may overlap slab n_src-1 or any output; the outputs follow the rules of
 * attnres_phase1 / attnres_phase1_first_prenorm against all of src.
 */
attnres_status_t attnres_phase1_accumulate(attnres_dtype_t dt, attnres_dtype_t src_dt, void* src, int64_t n_src,
                                           int64_t src_stride, int64_t T, int64_t d, const float* w,
                                           const float* key_gain, int64_t S, float eps, attnres_dtype_t partial_dt,
                                           const void* partial_in, attnres_dtype_t sublayer_dt,
                                           const void* sublayer_prev2, const void* sublayer_prev, void* out,
                                           float* m_out, float* lse_out, const float* prenorm_gain, void* x_out,
                                           void* h_out, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes attnres_phase1 uses: 16384 * ceil(d / 128) (packed
 * queries) + T * n_src * min(S, 32) * 4 (softmax weights); 0 for S == 1 with
 * more than ATTNRES_MAX_SOURCES_MULTI sources; -1 for invalid sizes. */
int64_t attnres_phase1_workspace_bytes(int64_t T, int64_t d, int64_t n_src, int64_t S);

/*
 * Phase 2 for one sublayer j of a block ("Attention Residuals" notes,
 * section 10, second phase; "Attention Residuals 阅读补充", merge of two
 * disjoint partitions; PreNorm fusion as in "ML 研究者的三层基本功", system
 * layer, and the CSDN summary section 4.2 on kernel fusion).
 *   o = p1_out [T][d] (dt), lse = p1_lse [T] fp32: this sublayer's phase-1
 *   partition (output normalised, lse = its log-sum-exp).
 *   If sublayer_prev == NULL (first sublayer of the block): h = o.
 *   Otherwise the partial sum is
 *       p = ((partial_in or 0) + (sublayer_prev2 or 0)) + sublayer_prev
 *   in fp32 arithmetic, in that order.  partial_in: [T][d] in format
 *   partial_dt (F32, P24, Q16, or dt itself for a sublayer output; NULL =
 *   zero);
 *   sublayer_prev, sublayer_prev2: [T][d] of dtype dt (the outputs of the
 *   previous and the one-before-previous sublayer; sublayer_prev2 NULL =
 *   zero).  With sublayer_prev2 a caller can store the running partial only
 *   at every second sublayer.  p is written to partial_out in format
 *   partial_out_dt (F32, P24 or Q16; NULL = not stored); partial_out may be the
 *   same pointer as partial_in when both formats are the same (in place).
 *   Merge: zc = w^T(key_gain (.) p / r(p)), M = max(lse, zc),
 *       h = (e^{lse-M} o + e^{zc-M} p) / (e^{lse-M} + e^{zc-M}).
 *   PreNorm: x = prenorm_gain (.) h / r(h)  (prenorm_gain NULL = ones).
 *   h_out, x_out: [T][d] dtype dt, either may be NULL but not both.
 *   w, key_gain, prenorm_gain: [d] fp32 (key_gain NULL = ones).
 * Passing partial_in, sublayer_prev2 or partial_out without sublayer_prev
 * is ATTNRES_EINVAL.
 */
attnres_status_t attnres_phase2_merge(attnres_dtype_t dt, int64_t T, int64_t d,
                                      const void* p1_out, const float* p1_lse,
                                      attnres_dtype_t partial_dt, const void* partial_in,
                                      const void* sublayer_prev2, const void* sublayer_prev,
                                      attnres_dtype_t partial_out_dt, void* partial_out,
                                      const float* w, const float* key_gain,
                                      const float* prenorm_gain, float eps,
                                      void* h_out, void* x_out, void* stream);

/*
 * Phase 2 of the grouped two-phase Full AttnRes ("Attention Residuals" notes,
 * section 7 for the sources, section 10 for the two phases; "Attention
 * Residuals 阅读补充", static queries and two-phase computation): the
 * sublayer's phase-1 partition (o = p1_out [T][d], lse = p1_lse [T], over the
 * sources completed before its group) is merged with the n_src outputs
 * produced inside the group so far, each its own source:
 *     u_i = src + i*src_stride ([T][d] dtype dt), i < n_src,
 *     z_i = w^T(key_gain (.) u_i / r(u_i)),  M = max(lse, z_i),
 *     h = (e^{lse-M} o + sum_i e^{z_i-M} u_i) / (e^{lse-M} + sum_i e^{z_i-M}),
 *     x = prenorm_gain (.) h / r(h).
 *   0 <= n_src <= ATTNRES_MAX_GROUP_SOURCES (n_src = 0: h = o; src and w may
 *   then be NULL).  w, key_gain, prenorm_gain: [d] fp32 (gains NULL = ones).
 *   h_out, x_out: [T][d] dtype dt, either may be NULL but not both (x_out
 *   NULL: no PreNorm).  Outputs must not overlap any input or each other.
 */
attnres_status_t attnres_phase2_merge_multi(attnres_dtype_t dt, int64_t T, int64_t d,
                                            const void* p1_out, const float* p1_lse,
                                            const void* src, int64_t n_src, int64_t src_stride,
                                            const float* w, const float* key_gain,
                                            const float* prenorm_gain, float eps,
                                            void* h_out, void* x_out, void* stream);

/*
 * One-shot depth aggregation with a single query ("Attention Residuals"
 * notes, section 7, Full AttnRes; also the final aggregation over
 * b_0..b_N of section 8).  Sources u_i = src + i*src_stride, i < n_src.
 *   h = sum_i softmax_i(z) u_i,  x = prenorm_gain (.) h / r(h).
 *   h_out, x_out: [T][d] dtype dt, either may be NULL but not both (x_out
 *   NULL: no PreNorm).  lse_out: [T] fp32 or NULL.
 *   w, key_gain, prenorm_gain: [d] fp32 (gains NULL = ones).
 * Limits: 1 <= n_src <= ATTNRES_MAX_SOURCES.  Outputs must not overlap src.
 */
attnres_status_t attnres_full(attnres_dtype_t dt,
                              const void* src, int64_t n_src, int64_t src_stride,
                              int64_t T, int64_t d,
                              const float* w, const float* key_gain,
                              const float* prenorm_gain, float eps,
                              void* h_out, void* x_out, float* lse_out, void* stream);

/*
 * Backward of one depth-aggregation site, for training ("Attention
 * Residuals" notes, section 7: the logit gradient dL/dz_i = alpha_i
 * G_h^T (u_i - h); "Attention Residuals 阅读补充", gradients along the
 * tangent: the RMSNorm Jacobian).  The site's forward over the sources
 * u_i = src + i*src_stride (i < n_src, each [T][d] dtype dt) is
 *     z_i = w^T(key_gain (.) u_i / r(u_i)),  alpha = softmax(z),
 *     h = sum_i alpha_i u_i,  x = prenorm_gain (.) h / r(h)  (prenorm != 0;
 *     x = h otherwise),
 * recomputed here.  Given dx = dL/dx [T][d] (dtype dt), writes
 *     dsrc + i*dsrc_stride = dL/du_i  ([T][d] dtype dt, i < n_src),
 *     dw = dL/dw, dkey_gain = dL/dkey_gain (NULL: not computed),
 *     dprenorm_gain = dL/dprenorm_gain (NULL or prenorm == 0: not computed),
 * each [d] fp32, summed over the T tokens in a fixed order (bitwise
 * reproducible).  key_gain, prenorm_gain NULL mean ones.
 * Limits: 1 <= n_src <= ATTNRES_MAX_SOURCES.  The dsrc rows must not
 * overlap any input; the [d] outputs must not overlap anything.
 * workspace: at least attnres_site_backward_workspace_bytes(T, d) bytes of
 * caller-owned device memory, 16-byte aligned (per-team partial sums).
 */
int64_t attnres_site_backward_workspace_bytes(int64_t T, int64_t d);
attnres_status_t attnres_site_backward(attnres_dtype_t dt,
                                       const void* src, int64_t n_src, int64_t src_stride,
                                       int64_t T, int64_t d,
                                       const float* w, const float* key_gain,
                                       const float* prenorm_gain, int prenorm, float eps,
                                       const void* dx, void* dsrc, int64_t dsrc_stride,
                                       float* dw, float* dkey_gain, float* dprenorm_gain,
                                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * As attnres_site_backward, but dL/du_i is ADDED to fp32 rows:
 *     dsrc + i*dsrc_stride += dL/du_i  ([T][d] fp32, i < n_src).
 * A source feeds every later site of Full AttnRes ("Attention Residuals"
 * notes, section 7: layer l attends over all earlier outputs), so its
 * gradient is the sum of one contribution per site; the sites' backward
 * passes accumulate into one fp32 row per source in reverse site order.
 * dw, dkey_gain, dprenorm_gain are written, not accumulated (each site has
 * its own parameters).  Same limits, alignment, aliasing rules and
 * workspace as attnres_site_backward; dsrc_stride counts fp32 elements.
 */
attnres_status_t attnres_site_backward_accumulate(attnres_dtype_t dt,
                                                  const void* src, int64_t n_src, int64_t src_stride,
                                                  int64_t T, int64_t d,
                                                  const float* w, const float* key_gain,
                                                  const float* prenorm_gain, int prenorm, float eps,
                                                  const void* dx, float* dsrc, int64_t dsrc_stride,
                                                  float* dw, float* dkey_gain, float* dprenorm_gain,
                                                  void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Backward through the block structure, in the two phases of the forward
 * (training).  Site j of a block reads the block sources u_i (b_0..b_{n-1})
 * and, after the block's first sublayer, the partial sum p_j ("Attention
 * Residuals" notes, section 8).  With the site's phase-1 partition (o_j
 * normalised, lse_j) and beta_j the softmax weight of p_j, the forward is
 * h_j = o_j + beta_j (p_j - o_j) ("Attention Residuals 阅读补充",
 * two-phase merge).  The sites of a block run in reverse order, each through
 * attnres_phase2_backward (the sublayer output gradients are complete only
 * once every later site has run); the block sources' gradients of all S
 * sites then come from one attnres_phase1_backward.  The logit gradient is
 * the notes' (section 7) and the RMSNorm Jacobian the reading notes'
 * (gradients along the tangent).
 *
 * attnres_phase2_backward: one site.
 *   p1_out [T][d] (dt), p1_lse [T]: the site's phase-1 partition, as
 *   attnres_phase1 returned it.  partial_in, sublayer_prev2, sublayer_prev:
 *   the partial source, composed exactly as attnres_phase2_merge composes it
 *   (sublayer_prev == NULL: the block's first sublayer, no partial source;
 *   p1_lse and dpartial may then be NULL).  w, key_gain, prenorm_gain: [d]
 *   fp32 (gains NULL = ones).  dx = dL/dx [T][d] (dt); prenorm == 0 means
 *   x = h.  Writes
 *     g_out = G = dL/dh [T][d] (dt),  c_out = 1 - beta, gp_out = G.p [T] fp32
 *   (G as stored; 0 without a partial source), and ADDS
 *     dpartial += dL/dp [T][d] fp32 (the partial source's gradient: the
 *       running gradient of the block's earlier sublayer outputs),
 *     dw += dL/dw, dkey_gain += dL/dkey_gain of the partial source's score
 *       (NULL: not computed; untouched without a partial source),
 *     dprenorm_gain += dL/dprenorm_gain (NULL or prenorm == 0: not computed),
 *   the [d] sums over the tokens in a fixed order.  dpartial is read and
 *   written in place; every other output must not overlap anything.
 *   workspace: attnres_phase2_backward_workspace_bytes(T, d) bytes, 16-byte
 *   aligned (per-team sums).
 *
 * attnres_phase1_backward: the block sources' part of S sites at once.
 *   src, n_src, src_stride: the block sources as for attnres_phase1, of
 *   dtype src_dt: dt, or ATTNRES_F32 with dt == ATTNRES_BF16 (the exact
 *   block sums a training forward keeps; then n_src <=
 *   ATTNRES_MAX_SOURCES_MULTI also for one site).  dt is G's dtype.
 *   w, key_gain: [S][d] fp32 (key_gain NULL = ones).  g_in + j*g_stride:
 *   G_j [T][d] (dt) of site j.  c_in, gp_in: [S][T] fp32 from the sites'
 *   attnres_phase2_backward (both NULL: each site is its phase-1 partition
 *   alone, c = 1, e.g. the final aggregation with G = dL/dh_final; c_in
 *   without gp_in is EINVAL).  Recomputes the scores and alpha1 of every
 *   site and G_j.h_j = c_j sum_i alpha1_ji G_j.u_i + (1 - c_j) G_j.p_j from
 *   the same dot products (not from the stored phase-1 output, whose
 *   rounding would dominate u_i - h_j when one source dominates), and
 *     dsrc + i*dsrc_stride  [T][d] fp32: dL/du_i of the S sites, written
 *       (accumulate == 0) or added (accumulate != 0),
 *     dw += dL/dw, dkey_gain += dL/dkey_gain ([S][d] fp32) of the block
 *       sources' scores (dkey_gain NULL: not computed),
 *   the [S][d] sums over the tokens in a fixed order.  Limits: 1 <= n_src <=
 *   ATTNRES_MAX_SOURCES_MULTI (ATTNRES_MAX_SOURCES for one site without
 *   c_in and gp_in), 1 <= S <= 32.  Outputs must not overlap any
 *   input or each other.  workspace:
 *   attnres_phase1_backward_workspace_bytes(T, d, n_src, S) bytes, 16-byte
 *   aligned (per-token coefficients, w (.) key_gain, per-range sums, the
 *   queries packed as matrix-core operands; for
 *   S == 1 at least the site backward's per-team sums, since one site
 *   without c_in and gp_in -- the final aggregation -- is computed as
 *   attnres_site_backward without PreNorm would, into the fp32 rows).
 */
int64_t attnres_phase2_backward_workspace_bytes(int64_t T, int64_t d);
attnres_status_t attnres_phase2_backward(attnres_dtype_t dt, int64_t T, int64_t d,
                                         const void* p1_out, const float* p1_lse,
                                         attnres_dtype_t partial_dt, const void* partial_in,
                                         const void* sublayer_prev2, const void* sublayer_prev,
                                         const float* w, const float* key_gain,
                                         const float* prenorm_gain, int prenorm, float eps,
                                         const void* dx, float* dpartial,
                                         void* g_out, float* c_out, float* gp_out,
                                         float* dw, float* dkey_gain, float* dprenorm_gain,
                                         void* workspace, int64_t workspace_bytes, void* stream);

int64_t attnres_phase1_backward_workspace_bytes(int64_t T, int64_t d, int64_t n_src, int64_t S);
attnres_status_t attnres_phase1_backward(attnres_dtype_t dt, attnres_dtype_t src_dt,
                                         const void* src, int64_t n_src, int64_t src_stride,
                                         int64_t T, int64_t d,
                                         const float* w, const float* key_gain, int64_t S, float eps,
                                         const void* g_in, int64_t g_stride,
                                         const float* c_in, const float* gp_in,
                                         float* dsrc, int64_t dsrc_stride, int accumulate,
                                         float* dw, float* dkey_gain,
                                         void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Block completion ("Attention Residuals" notes, section 8: b_n is the sum of
 * the block's sublayer outputs):
 *     out = ((partial_in or 0) + (v2 or 0)) + v      (fp32, in that order)
 *   partial_in: [T][d] in format partial_dt (F32, P24, Q16 or dt; NULL =
 *   zero);
 *   v2 (NULL = zero), v: [T][d] dtype dt.  out: [T][d] of dtype out_dt, dt
 *   itself or ATTNRES_F32 with dt == ATTNRES_BF16 (the exact fp32 sum, kept
 *   by a training forward; any other pair is ATTNRES_EDTYPE).  out may be
 *   the same pointer as partial_in when partial_dt == out_dt; out must not
 *   overlap v or v2.
 */
attnres_status_t attnres_block_accumulate(attnres_dtype_t dt, int64_t T, int64_t d,
                                          attnres_dtype_t partial_dt, const void* partial_in,
                                          const void* v2, const void* v, void* out, attnres_dtype_t out_dt,
                                          void* stream);

/*
 * Streaming-bandwidth probe: a measurement aid that computes nothing of the
 * aggregation.  It bounds the HBM rate a kernel with a given mix of read and
 * write streams can reach, the way the aggregation kernels move rows (the
 * reading notes, "静态 Query 与两阶段计算", ask for the benefit of the
 * two-phase scheme to be verified against DRAM reads and kernel latency).
 * Reads n_read streams of stream_bytes each, consecutive from src, and
 * writes n_write streams, consecutive from dst (16-byte accesses, a wave
 * covering 1 KiB of consecutive bytes of each stream per instruction), with
 * workgroups_per_cu 256-thread workgroups per compute unit in a grid-stride
 * loop, `unroll` chunks of each stream in flight per thread (1, 2, 4 or 8),
 * and non-temporal loads and stores when `nontemporal` is nonzero.
 *   0 <= n_read <= 4, 0 <= n_write <= 2, not both zero, or one of the
 *   many-stream mixes (n_read, n_write) = (8, 0) (the scoring pass over a
 *   block's sources), (9, 1) (the final aggregation: nine sources, one
 *   output) and (7, 24) (the phase-1 output pass of a block with seven
 *   sources and 24 sublayers); 1 <= workgroups_per_cu <= 16; stream_bytes a
 *   positive multiple of 16 (at most 2^40).  With n_write == 0, dst must
 *   still point at 16 writable bytes (kept as the loads' sink; not written
 *   for any data these probes read).  The read and written ranges must not
 *   overlap.  Asynchronous on `stream`, like every other entry point.
 */
attnres_status_t attnres_stream_probe(int64_t n_read, int64_t n_write, const void* src, void* dst,
                                      int64_t stream_bytes, int64_t workgroups_per_cu, int64_t unroll,
                                      int64_t nontemporal, void* stream);

/* Human-readable name of a status code (static string). */
const char* attnres_status_string(attnres_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* ATTNRES_H */
