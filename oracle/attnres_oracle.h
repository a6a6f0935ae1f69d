/*
 * Block / Full Attention Residuals (AttnRes) -- reference oracle, fp64, CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is a plain, slow, obviously correct
 * statement of what the depth aggregation computes.  It is loaded by the test
 * suite, by the smoke check and by the benchmark's CPU-baseline leg, and by
 * nothing else.  It shares no code, header, table or helper with the HIP
 * library; neither includes or links the other.
 *
 * Sources followed (page title, section):
 *  - "Attention Residuals 阅读补充", section "RMSNorm 的数学原理":
 *      r_eps(x) = sqrt(mean_i x_i^2 + eps),  RMSNorm(x) = gamma (.) x / r_eps(x).
 *  - "Attention Residuals" (structured notes on arXiv 2603.15031), section 7
 *    "Full AttnRes": one input-independent pseudo-query w_l per target
 *    sublayer; score z_{i,l} = w_l^T RMSNorm(v_i); alpha = softmax over depth;
 *    h_l = sum_i alpha_{i->l} v_i with the *unnormalised* v_i; no 1/sqrt(d),
 *    no temperature; tokens never interact.
 *  - same page, section 8 "Block AttnRes": b_0 = embedding; b_n = sum of the
 *    outputs of block n; the first sublayer of block n sees [b_0..b_{n-1}],
 *    later sublayers also see the partial sum b_n^{i-1}; the final output
 *    reads b_0..b_N.
 *  - same page, section 10 (two-phase inference): the softmax statistics of
 *    a source partition (max, shifted exp-sum, output) and the exact merge of
 *    two disjoint partitions.  In this library the merge is used only by the
 *    tests that check it against the one-shot softmax; the forward functions
 *    compute every site in one shot.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Key RMSNorm gain: each target sublayer l owns a key gain g_l, so
 *    z = w_l^T (g_l (.) u / r_eps(u)).
 *  - eps inside the square root with the mean, same eps for key norm and
 *    PreNorm.
 *  - x_l = RMSNorm_{gamma_l}(h_l) is the PreNorm input of sublayer l.
 *  - The final aggregation has its own (w_{L+1}, g_{L+1}) and no PreNorm.
 *  - lse = m + ln(sum_i exp(z_i - m)) (a true log-sum-exp).
 *
 * Conventions: inputs are fp32 arrays (bf16 inputs are widened exactly);
 * every computation and every output is fp64.  Row-major, token-major rows of
 * d channels.  All functions return 0 on success and a negative value on an
 * invalid argument.
 */
#ifndef ATTNRES_ORACLE_H
#define ATTNRES_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* r_eps(x) = sqrt(sum_i x_i^2 / d + eps). */
double oracle_rms(int64_t d, const double* x, double eps);

/* y = gain (.) x / r_eps(x); gain NULL means all ones. */
int oracle_rmsnorm(int64_t d, const double* x, const double* gain, double eps, double* y);

/* One depth-aggregation site for one token.
 * src[i] (i < n) are the source rows, w the pseudo-query, g the key gain (NULL
 * means ones).  Outputs (any may be NULL): z[n] scores, alpha[n] softmax
 * weights, h[d] aggregated row, *m = max z, *lse = log-sum-exp of z. */
int oracle_depth_softmax(int64_t n, int64_t d, const double* const* src,
                         const double* w, const double* g, double eps,
                         double* z, double* alpha, double* h, double* m, double* lse);

/* Softmax statistics of one source partition in the two-phase notation:
 * m = max z, ell = sum exp(z - m), o = sum exp(z - m) v (unnormalised). */
int oracle_partition_stats(int64_t n, int64_t d, const double* const* src,
                           const double* w, const double* g, double eps,
                           double* m, double* ell, double* o);

/* Merge of two disjoint partitions A and B:
 * h = (e^{mA-M} oA + e^{mB-M} oB) / (e^{mA-M} lA + e^{mB-M} lB), M = max(mA, mB). */
int oracle_merge_two(int64_t d, double mA, double lA, const double* oA,
                     double mB, double lB, const double* oB, double* h);

/* Block AttnRes forward over n_tok tokens (each token independently).
 *  blocks:      n_blocks block sizes (sublayers per block); L = their sum.
 *  n_given:     completed block sums supplied as inputs (b_1..b_{n_given}),
 *               so the first computed block is block n_given+1.
 *  emb  [n_tok][d]            b_0
 *  given[n_given][n_tok][d]   (NULL if n_given == 0)
 *  v    [L][n_tok][d]         sublayer outputs v_l
 *  w, g [L+1][d]              pseudo-queries and key gains; row L belongs to
 *                             the final site (g may be NULL: ones)
 *  gamma[L][d]                PreNorm gains (NULL: ones)
 * Outputs (each may be NULL):
 *  x_out, h_out [L][n_tok][d]     PreNorm input and aggregation of each site
 *  o1_out [L][n_tok][d], m1_out, lse1_out [L][n_tok]
 *        the same softmax restricted to the completed-block sources
 *        [b_0..b_{n-1}] of the site (the phase-1 quantities), normalised
 *  lse_out [L][n_tok]             log-sum-exp over all of the site's sources
 *  hfinal_out [n_tok][d]          final aggregation over b_0..b_N (if final)
 *  reps_out [1+n_given+n_blocks][n_tok][d]   b_0..b_N (exact sums)
 * Threads: tokens are distributed over OpenMP threads when available. */
int oracle_block_forward(int64_t n_tok, int64_t d, int64_t n_blocks, const int64_t* blocks,
                         int64_t n_given, const float* emb, const float* given, const float* v,
                         const float* w, const float* g, const float* gamma, double eps,
                         int final_site,
                         double* x_out, double* h_out, double* o1_out, double* m1_out,
                         double* lse1_out, double* lse_out, double* hfinal_out, double* reps_out);

/* Full AttnRes forward: sublayer l (1..L) aggregates v_0 = emb, v_1..v_{l-1}
 * each as its own source; the final site aggregates v_0..v_L.  Same layouts
 * as oracle_block_forward. */
int oracle_full_forward(int64_t n_tok, int64_t d, int64_t L, const float* emb, const float* v,
                        const float* w, const float* g, const float* gamma, double eps,
                        int final_site, double* x_out, double* h_out, double* lse_out,
                        double* hfinal_out);

/* Backward of one aggregation site for one token.  Forward:
 *   y_i = u_i / r_eps(u_i),  z_i = w^T (g (.) y_i),  alpha = softmax(z),
 *   h = sum_i alpha_i u_i,   x = gamma (.) h / r_eps(h)  (prenorm != 0)
 *                            x = h                        (prenorm == 0)
 * Given dx = dL/dx, writes du[i] = dL/du_i (n rows of d) and ADDS this
 * token's dL/dw, dL/dg, dL/dgamma to dw, dg, dgamma (dgamma may be NULL
 * without PreNorm).  g, gamma NULL mean ones.  Steps, in the pages' order:
 *   RMSNorm backward ("Attention Residuals 阅读补充", section on gradients
 *   propagating along the tangent: the upstream gradient is multiplied by
 *   gamma, then dL/dx = (G - y (y^T G)/d) / r), the logit gradient
 *   dL/dz_i = alpha_i G_h^T (u_i - h) ("Attention Residuals" notes, section
 *   7), the value path alpha_i G_h, and the score path through w, g and the
 *   key RMSNorm (the same Jacobian). */
int oracle_site_backward(int64_t n, int64_t d, const double* const* src, const double* w,
                         const double* g, const double* gamma, int prenorm, double eps,
                         const double* dx, double* const* du, double* dw, double* dg,
                         double* dgamma);

/* oracle_site_backward over n_tok tokens of fp32 inputs (src [n][n_tok][d],
 * dx [n_tok][d]); du [n][n_tok][d]; dw, dg, dgamma [d] are the sums over the
 * tokens (overwritten). */
int oracle_site_backward_tokens(int64_t n_tok, int64_t n, int64_t d, const float* src,
                                const float* w, const float* g, const float* gamma, int prenorm,
                                double eps, const float* dx, double* du, double* dw, double* dg,
                                double* dgamma);

/* Backward of the whole Block AttnRes forward of oracle_block_forward, with
 * the sublayer outputs v_l treated as inputs: the loss is
 *   L = sum_l sum_t dx_l[t] . x_l[t]  +  sum_t dhf[t] . hfinal[t]
 * (the second term only with final_site and dhf != NULL).  Every site's
 * backward is oracle_site_backward over that site's own sources; the chain
 * rule through the sums of the block structure ("Attention Residuals" notes,
 * section 8: b_n is the sum of block n's sublayer outputs and the partial
 * sum of a block is the sum of its outputs so far) gives
 *   dL/dv_l = dL/db_n + sum over later sites j of the same block of dL/dp_j,
 * where b_n is l's block sum and p_j the partial-sum source of site j.
 * Outputs (fp64): dv [L][n_tok][d]; dreps [1 + n_given][n_tok][d] (the
 * embedding, then the given block sums); dw, dg [L+1][d] and dgamma [L][d],
 * summed over the tokens (overwritten).  dx [L][n_tok][d], dhf [n_tok][d].
 * Block sums are exact fp64 sums, as the notes define them. */
int oracle_block_backward(int64_t n_tok, int64_t d, int64_t n_blocks, const int64_t* blocks,
                          int64_t n_given, const float* emb, const float* given, const float* v,
                          const float* w, const float* g, const float* gamma, double eps,
                          int final_site, const float* dx, const float* dhf, double* dv_out,
                          double* dreps_out, double* dw_out, double* dg_out, double* dgamma_out);

/* Number of OpenMP threads the forward functions use (1 without OpenMP). */
int oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
