/*
 * Block / Full Attention Residuals -- reference oracle, fp64, plain C.
 * TEST INFRASTRUCTURE ONLY (see attnres_oracle.h for the sources followed and
 * the readings taken where the pages are silent).
 *
 * Everything here is the plain definition computed per token and per
 * aggregation site, in the order the pages state it: RMSNorm each key,
 * score it against the site's pseudo-query, softmax over depth, weight the
 * unnormalised sources, then apply the consuming sublayer's PreNorm.
 * There is no blocking, no fusion and no two-phase evaluation in the forward
 * functions.
 */
#include "attnres_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* "Attention Residuals 阅读补充", RMSNorm section: mean square over the d
 * features of one token, eps inside the root. */
double oracle_rms(int64_t d, const double* x, double eps) {
    double s = 0.0;
    for (int64_t k = 0; k < d; ++k) s += x[k] * x[k];
    return sqrt(s / (double)d + eps);
}

int oracle_rmsnorm(int64_t d, const double* x, const double* gain, double eps, double* y) {
    if (d <= 0 || !x || !y) return -1;
    double r = oracle_rms(d, x, eps);
    for (int64_t k = 0; k < d; ++k) y[k] = (gain ? gain[k] : 1.0) * (x[k] / r);
    return 0;
}

/* "Attention Residuals" notes, section 7: z_i = w^T RMSNorm_g(src_i);
 * alpha = softmax(z); h = sum_i alpha_i src_i (values are the raw sources). */
int oracle_depth_softmax(int64_t n, int64_t d, const double* const* src,
                         const double* w, const double* g, double eps,
                         double* z, double* alpha, double* h, double* m, double* lse) {
    if (n <= 0 || d <= 0 || !src || !w) return -1;
    double* zz = (double*)malloc(sizeof(double) * (size_t)n * 2);
    double* key = (double*)malloc(sizeof(double) * (size_t)d);
    if (!zz || !key) { free(zz); free(key); return -2; }
    double* aa = zz + n;
    for (int64_t i = 0; i < n; ++i) {
        oracle_rmsnorm(d, src[i], g, eps, key);          /* key = RMSNorm_g(v_i) */
        double s = 0.0;
        for (int64_t k = 0; k < d; ++k) s += w[k] * key[k];
        zz[i] = s;                                         /* z_i = w^T key */
    }
    double mx = zz[0];
    for (int64_t i = 1; i < n; ++i) if (zz[i] > mx) mx = zz[i];
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) { aa[i] = exp(zz[i] - mx); sum += aa[i]; }
    for (int64_t i = 0; i < n; ++i) aa[i] /= sum;
    if (h) {
        for (int64_t k = 0; k < d; ++k) {
            double acc = 0.0;
            for (int64_t i = 0; i < n; ++i) acc += aa[i] * src[i][k];
            h[k] = acc;
        }
    }
    if (z) memcpy(z, zz, sizeof(double) * (size_t)n);
    if (alpha) memcpy(alpha, aa, sizeof(double) * (size_t)n);
    if (m) *m = mx;
    if (lse) *lse = mx + log(sum);
    free(zz);
    free(key);
    return 0;
}

/* "Attention Residuals" notes, section 10: per-partition (m, ell, o). */
int oracle_partition_stats(int64_t n, int64_t d, const double* const* src,
                           const double* w, const double* g, double eps,
                           double* m, double* ell, double* o) {
    if (n <= 0 || d <= 0 || !m || !ell || !o) return -1;
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    if (!z) return -2;
    int rc = oracle_depth_softmax(n, d, src, w, g, eps, z, NULL, NULL, NULL, NULL);
    if (rc) { free(z); return rc; }
    double mx = z[0];
    for (int64_t i = 1; i < n; ++i) if (z[i] > mx) mx = z[i];
    double l = 0.0;
    for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double e = exp(z[i] - mx);
        l += e;
        for (int64_t k = 0; k < d; ++k) o[k] += e * src[i][k];
    }
    *m = mx;
    *ell = l;
    free(z);
    return 0;
}

/* "Attention Residuals 阅读补充", two-phase section: merge of two disjoint
 * partitions under their common maximum. */
int oracle_merge_two(int64_t d, double mA, double lA, const double* oA,
                     double mB, double lB, const double* oB, double* h) {
    if (d <= 0 || !oA || !oB || !h) return -1;
    double M = mA > mB ? mA : mB;
    double a = exp(mA - M), b = exp(mB - M);
    double den = a * lA + b * lB;
    for (int64_t k = 0; k < d; ++k) h[k] = (a * oA[k] + b * oB[k]) / den;
    return 0;
}

static void widen(int64_t d, const float* x, double* y) {
    for (int64_t k = 0; k < d; ++k) y[k] = (double)x[k];
}

int oracle_block_forward(int64_t n_tok, int64_t d, int64_t n_blocks, const int64_t* blocks,
                         int64_t n_given, const float* emb, const float* given, const float* v,
                         const float* w, const float* g, const float* gamma, double eps,
                         int final_site,
                         double* x_out, double* h_out, double* o1_out, double* m1_out,
                         double* lse1_out, double* lse_out, double* hfinal_out, double* reps_out) {
    if (n_tok < 0 || d <= 0 || n_blocks < 0 || n_given < 0 || !emb || !w) return -1;
    if (n_given > 0 && !given) return -1;
    int64_t L = 0;
    for (int64_t b = 0; b < n_blocks; ++b) {
        if (blocks[b] <= 0) return -1;
        L += blocks[b];
    }
    if (L > 0 && !v) return -1;
    const int64_t R = 1 + n_given + n_blocks;   /* b_0 .. b_N */
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_tok; ++t) {
        double* reps = (double*)malloc(sizeof(double) * (size_t)(R * d));
        double* partial = (double*)malloc(sizeof(double) * (size_t)d);
        double* wq = (double*)malloc(sizeof(double) * (size_t)(2 * d));
        double* gam = (double*)malloc(sizeof(double) * (size_t)d);
        double* h = (double*)malloc(sizeof(double) * (size_t)d);
        double* x = (double*)malloc(sizeof(double) * (size_t)d);
        const double** srcs = (const double**)malloc(sizeof(double*) * (size_t)(R + 1));
        if (!reps || !partial || !wq || !gam || !h || !x || !srcs) {
#pragma omp atomic write
            bad = 1;
        } else {
            double* gk = wq + d;
            /* b_0 is the token embedding; b_1..b_{n_given} are supplied. */
            widen(d, emb + t * d, reps);
            for (int64_t n = 0; n < n_given; ++n)
                widen(d, given + (n * n_tok + t) * d, reps + (1 + n) * d);
            int64_t have = 1 + n_given;   /* completed sources so far */
            int64_t l = 0;                /* 0-based sublayer index */
            for (int64_t b = 0; b < n_blocks; ++b) {
                for (int64_t j = 0; j < blocks[b]; ++j, ++l) {
                    /* Sources: [b_0..b_{n-1}] and, after the block's first
                     * sublayer, the partial sum of the block so far. */
                    int64_t ns = 0;
                    for (int64_t i = 0; i < have; ++i) srcs[ns++] = reps + i * d;
                    if (j > 0) srcs[ns++] = partial;
                    widen(d, w + l * d, wq);
                    if (g) widen(d, g + l * d, gk);
                    double lse_full = 0.0;
                    oracle_depth_softmax(ns, d, srcs, wq, g ? gk : NULL, eps,
                                         NULL, NULL, h, NULL, &lse_full);
                    if (gamma) widen(d, gamma + l * d, gam);
                    oracle_rmsnorm(d, h, gamma ? gam : NULL, eps, x);
                    const int64_t row = (l * n_tok + t) * d;
                    if (x_out) memcpy(x_out + row, x, sizeof(double) * (size_t)d);
                    if (h_out) memcpy(h_out + row, h, sizeof(double) * (size_t)d);
                    if (lse_out) lse_out[l * n_tok + t] = lse_full;
                    if (o1_out || m1_out || lse1_out) {
                        /* The same site restricted to the completed blocks. */
                        double m1 = 0.0, lse1 = 0.0;
                        oracle_depth_softmax(have, d, srcs, wq, g ? gk : NULL, eps,
                                             NULL, NULL, h, &m1, &lse1);
                        if (o1_out) memcpy(o1_out + row, h, sizeof(double) * (size_t)d);
                        if (m1_out) m1_out[l * n_tok + t] = m1;
                        if (lse1_out) lse1_out[l * n_tok + t] = lse1;
                    }
                    /* The sublayer's output joins the block's running sum. */
                    const float* vl = v + (l * n_tok + t) * d;
                    for (int64_t k = 0; k < d; ++k)
                        partial[k] = (j == 0 ? 0.0 : partial[k]) + (double)vl[k];
                }
                memcpy(reps + have * d, partial, sizeof(double) * (size_t)d);
                ++have;
            }
            if (final_site && hfinal_out) {
                for (int64_t i = 0; i < have; ++i) srcs[i] = reps + i * d;
                widen(d, w + L * d, wq);
                if (g) widen(d, g + L * d, gk);
                oracle_depth_softmax(have, d, srcs, wq, g ? gk : NULL, eps,
                                     NULL, NULL, hfinal_out + t * d, NULL, NULL);
            }
            if (reps_out)
                for (int64_t i = 0; i < have; ++i)
                    memcpy(reps_out + (i * n_tok + t) * d, reps + i * d, sizeof(double) * (size_t)d);
        }
        free(reps); free(partial); free(wq); free(gam); free(h); free(x); free((void*)srcs);
    }
    return bad ? -2 : 0;
}

int oracle_full_forward(int64_t n_tok, int64_t d, int64_t L, const float* emb, const float* v,
                        const float* w, const float* g, const float* gamma, double eps,
                        int final_site, double* x_out, double* h_out, double* lse_out,
                        double* hfinal_out) {
    if (n_tok < 0 || d <= 0 || L < 0 || !emb || !w || (L > 0 && !v)) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_tok; ++t) {
        /* v_0 = embedding, v_i = output of sublayer i: every one kept. */
        double* hist = (double*)malloc(sizeof(double) * (size_t)((L + 1) * d));
        double* wq = (double*)malloc(sizeof(double) * (size_t)(2 * d));
        double* gam = (double*)malloc(sizeof(double) * (size_t)d);
        double* h = (double*)malloc(sizeof(double) * (size_t)d);
        double* x = (double*)malloc(sizeof(double) * (size_t)d);
        const double** srcs = (const double**)malloc(sizeof(double*) * (size_t)(L + 1));
        if (!hist || !wq || !gam || !h || !x || !srcs) {
#pragma omp atomic write
            bad = 1;
        } else {
            double* gk = wq + d;
            widen(d, emb + t * d, hist);
            for (int64_t i = 0; i <= L; ++i) srcs[i] = hist + i * d;
            for (int64_t l = 0; l < L; ++l) {
                /* sublayer l+1 attends over v_0..v_l */
                widen(d, w + l * d, wq);
                if (g) widen(d, g + l * d, gk);
                double lse = 0.0;
                oracle_depth_softmax(l + 1, d, srcs, wq, g ? gk : NULL, eps, NULL, NULL, h, NULL, &lse);
                if (gamma) widen(d, gamma + l * d, gam);
                oracle_rmsnorm(d, h, gamma ? gam : NULL, eps, x);
                const int64_t row = (l * n_tok + t) * d;
                if (x_out) memcpy(x_out + row, x, sizeof(double) * (size_t)d);
                if (h_out) memcpy(h_out + row, h, sizeof(double) * (size_t)d);
                if (lse_out) lse_out[l * n_tok + t] = lse;
                widen(d, v + (l * n_tok + t) * d, hist + (l + 1) * d);
            }
            if (final_site && hfinal_out) {
                widen(d, w + L * d, wq);
                if (g) widen(d, g + L * d, gk);
                oracle_depth_softmax(L + 1, d, srcs, wq, g ? gk : NULL, eps, NULL, NULL,
                                     hfinal_out + t * d, NULL, NULL);
            }
        }
        free(hist); free(wq); free(gam); free(h); free(x); free((void*)srcs);
    }
    return bad ? -2 : 0;
}

/* "Attention Residuals 阅读补充", gradients along the tangent: for
 * y = x / r_eps(x) and an upstream gradient G = dL/dy,
 * dL/dx = (G - y (y^T G) / d) / r_eps(x). */
static void rms_core_backward(int64_t d, const double* x, double eps, const double* G, double* dx_out) {
    const double r = oracle_rms(d, x, eps);
    double yg = 0.0;
    for (int64_t k = 0; k < d; ++k) yg += (x[k] / r) * G[k];
    for (int64_t k = 0; k < d; ++k) dx_out[k] = (G[k] - (x[k] / r) * yg / (double)d) / r;
}

int oracle_site_backward(int64_t n, int64_t d, const double* const* src, const double* w,
                         const double* g, const double* gamma, int prenorm, double eps,
                         const double* dx, double* const* du, double* dw, double* dg,
                         double* dgamma) {
    if (n <= 0 || d <= 0 || !src || !w || !dx || !du || !dw || !dg) return -1;
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    double* alpha = (double*)malloc(sizeof(double) * (size_t)n);
    double* h = (double*)malloc(sizeof(double) * (size_t)d);
    double* Gh = (double*)malloc(sizeof(double) * (size_t)d);
    double* G = (double*)malloc(sizeof(double) * (size_t)d);
    double* t = (double*)malloc(sizeof(double) * (size_t)d);
    int rc = (!z || !alpha || !h || !Gh || !G || !t) ? -2 : 0;
    /* forward of the site */
    if (!rc) rc = oracle_depth_softmax(n, d, src, w, g, eps, z, alpha, h, NULL, NULL);
    if (rc) {
        free(z); free(alpha); free(h); free(Gh); free(G); free(t);
        return rc;
    }
    /* PreNorm: x = gamma (.) y_h with y_h = h / r(h) */
    if (prenorm) {
        const double rh = oracle_rms(d, h, eps);
        for (int64_t k = 0; k < d; ++k) {
            G[k] = (gamma ? gamma[k] : 1.0) * dx[k];
            if (dgamma) dgamma[k] += dx[k] * (h[k] / rh);
        }
        rms_core_backward(d, h, eps, G, Gh);
    } else {
        for (int64_t k = 0; k < d; ++k) Gh[k] = dx[k];
    }
    for (int64_t i = 0; i < n; ++i) {
        /* logit gradient: alpha_i G_h^T (u_i - h) */
        double s = 0.0;
        for (int64_t k = 0; k < d; ++k) s += Gh[k] * (src[i][k] - h[k]);
        const double dz = alpha[i] * s;
        /* score path: z_i = w^T (g (.) y_i) */
        const double r = oracle_rms(d, src[i], eps);
        for (int64_t k = 0; k < d; ++k) {
            const double gk = g ? g[k] : 1.0;
            const double y = src[i][k] / r;
            G[k] = dz * w[k] * gk;       /* dL/dy_i */
            dw[k] += dz * gk * y;
            dg[k] += dz * w[k] * y;
        }
        rms_core_backward(d, src[i], eps, G, t);
        /* value path + score path */
        for (int64_t k = 0; k < d; ++k) du[i][k] = alpha[i] * Gh[k] + t[k];
    }
    free(z); free(alpha); free(h); free(Gh); free(G); free(t);
    return 0;
}

int oracle_site_backward_tokens(int64_t n_tok, int64_t n, int64_t d, const float* src,
                                const float* w, const float* g, const float* gamma, int prenorm,
                                double eps, const float* dx, double* du, double* dw, double* dg,
                                double* dgamma) {
    if (n_tok < 0 || n <= 0 || d <= 0 || !src || !w || !dx || !du || !dw || !dg) return -1;
    double* wd = (double*)malloc(sizeof(double) * (size_t)d);
    double* gd = g ? (double*)malloc(sizeof(double) * (size_t)d) : NULL;
    double* gmd = gamma ? (double*)malloc(sizeof(double) * (size_t)d) : NULL;
    widen(d, w, wd);
    if (gd) widen(d, g, gd);
    if (gmd) widen(d, gamma, gmd);
    for (int64_t k = 0; k < d; ++k) {
        dw[k] = 0.0;
        dg[k] = 0.0;
        if (dgamma) dgamma[k] = 0.0;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* rows = (double*)malloc(sizeof(double) * (size_t)(n * d));
        double* dxt = (double*)malloc(sizeof(double) * (size_t)d);
        const double** sp = (const double**)malloc(sizeof(double*) * (size_t)n);
        double** dp = (double**)malloc(sizeof(double*) * (size_t)n);
        double* lw = (double*)calloc((size_t)d, sizeof(double));
        double* lg = (double*)calloc((size_t)d, sizeof(double));
        double* lgm = (double*)calloc((size_t)d, sizeof(double));
        double* dut = (double*)malloc(sizeof(double) * (size_t)(n * d));
#pragma omp for schedule(static)
        for (int64_t tk = 0; tk < n_tok; ++tk) {
            for (int64_t i = 0; i < n; ++i) {
                widen(d, src + ((size_t)i * (size_t)n_tok + (size_t)tk) * (size_t)d, rows + i * d);
                sp[i] = rows + i * d;
                dp[i] = dut + i * d;
            }
            widen(d, dx + (size_t)tk * (size_t)d, dxt);
            if (oracle_site_backward(n, d, sp, wd, gd, gmd, prenorm, eps, dxt, dp, lw, lg, lgm)) bad = 1;
            for (int64_t i = 0; i < n; ++i)
                memcpy(du + ((size_t)i * (size_t)n_tok + (size_t)tk) * (size_t)d, dut + i * d,
                       sizeof(double) * (size_t)d);
        }
#pragma omp critical
        {
            for (int64_t k = 0; k < d; ++k) {
                dw[k] += lw[k];
                dg[k] += lg[k];
                if (dgamma) dgamma[k] += lgm[k];
            }
        }
        free(rows); free(dxt); free(sp); free(dp); free(lw); free(lg); free(lgm); free(dut);
    }
    free(wd); free(gd); free(gmd);
    return bad ? -3 : 0;
}

int oracle_block_backward(int64_t n_tok, int64_t d, int64_t n_blocks, const int64_t* blocks,
                          int64_t n_given, const float* emb, const float* given, const float* v,
                          const float* w, const float* g, const float* gamma, double eps,
                          int final_site, const float* dx, const float* dhf, double* dv_out,
                          double* dreps_out, double* dw_out, double* dg_out, double* dgamma_out) {
    if (n_tok < 0 || d <= 0 || n_blocks < 0 || n_given < 0 || !emb || !w || !dv_out || !dreps_out ||
        !dw_out || !dg_out || !dgamma_out)
        return -1;
    if (n_given > 0 && !given) return -1;
    int64_t L = 0;
    for (int64_t b = 0; b < n_blocks; ++b) {
        if (blocks[b] <= 0) return -1;
        L += blocks[b];
    }
    if (L > 0 && (!v || !dx)) return -1;
    const int64_t R = 1 + n_given + n_blocks;   /* b_0 .. b_N */
    for (int64_t k = 0; k < (L + 1) * d; ++k) dw_out[k] = dg_out[k] = 0.0;
    for (int64_t k = 0; k < L * d; ++k) dgamma_out[k] = 0.0;
    int bad = 0;

#pragma omp parallel
    {
        double* reps = (double*)malloc(sizeof(double) * (size_t)(R * d));
        double* parts = (double*)malloc(sizeof(double) * (size_t)((L > 0 ? L : 1) * d));
        double* db = (double*)calloc((size_t)(R * d), sizeof(double));
        double* du = (double*)malloc(sizeof(double) * (size_t)((R + 1) * d));
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        double* wq = (double*)malloc(sizeof(double) * (size_t)(3 * d));
        double* dxt = (double*)malloc(sizeof(double) * (size_t)d);
        double* lw = (double*)calloc((size_t)((L + 1) * d), sizeof(double));
        double* lg = (double*)calloc((size_t)((L + 1) * d), sizeof(double));
        double* lgm = (double*)calloc((size_t)((L > 0 ? L : 1) * d), sizeof(double));
        const double** srcs = (const double**)malloc(sizeof(double*) * (size_t)(R + 1));
        double** dus = (double**)malloc(sizeof(double*) * (size_t)(R + 1));
        if (!reps || !parts || !db || !du || !acc || !wq || !dxt || !lw || !lg || !lgm || !srcs || !dus) {
#pragma omp atomic write
            bad = 1;
        } else {
            double* gk = wq + d;
            double* gm = wq + 2 * d;
            for (int64_t i = 0; i <= R; ++i) dus[i] = du + i * d;
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < n_tok; ++t) {
                /* forward: block sums and the partial-sum source of every site */
                widen(d, emb + t * d, reps);
                for (int64_t n = 0; n < n_given; ++n)
                    widen(d, given + (n * n_tok + t) * d, reps + (1 + n) * d);
                int64_t l = 0;
                for (int64_t b = 0; b < n_blocks; ++b) {
                    double* bs = reps + (1 + n_given + b) * d;
                    for (int64_t k = 0; k < d; ++k) bs[k] = 0.0;
                    for (int64_t j = 0; j < blocks[b]; ++j, ++l) {
                        /* parts[l] = v_{l0} + ... + v_{l-1} (the partial source of site l) */
                        memcpy(parts + l * d, bs, sizeof(double) * (size_t)d);
                        const float* vl = v + (l * n_tok + t) * d;
                        for (int64_t k = 0; k < d; ++k) bs[k] += (double)vl[k];
                    }
                }
                for (int64_t k = 0; k < R * d; ++k) db[k] = 0.0;
                /* the final site reads b_0 .. b_N, no PreNorm */
                if (final_site && dhf) {
                    for (int64_t i = 0; i < R; ++i) srcs[i] = reps + i * d;
                    widen(d, w + L * d, wq);
                    if (g) widen(d, g + L * d, gk);
                    widen(d, dhf + t * d, dxt);
                    if (oracle_site_backward(R, d, srcs, wq, g ? gk : NULL, NULL, 0, eps, dxt, dus,
                                             lw + L * d, lg + L * d, NULL))
                        bad = 1;
                    for (int64_t i = 0; i < R; ++i)
                        for (int64_t k = 0; k < d; ++k) db[i * d + k] += du[i * d + k];
                }
                /* blocks in reverse; inside a block, sites in reverse */
                int64_t l_end = L;
                for (int64_t b = n_blocks - 1; b >= 0; --b) {
                    const int64_t S = blocks[b];
                    const int64_t l0 = l_end - S;
                    const int64_t n = 1 + n_given + b;   /* sources before block b */
                    /* dL/dv of the block's last output is dL/db_n; each site j
                     * adds dL/dp_j for the outputs before it */
                    memcpy(acc, db + n * d, sizeof(double) * (size_t)d);
                    for (int64_t j = S - 1; j >= 0; --j) {
                        const int64_t ll = l0 + j;
                        memcpy(dv_out + (ll * n_tok + t) * d, acc, sizeof(double) * (size_t)d);
                        int64_t ns = 0;
                        for (int64_t i = 0; i < n; ++i) srcs[ns++] = reps + i * d;
                        if (j > 0) srcs[ns++] = parts + ll * d;
                        widen(d, w + ll * d, wq);
                        if (g) widen(d, g + ll * d, gk);
                        if (gamma) widen(d, gamma + ll * d, gm);
                        widen(d, dx + (ll * n_tok + t) * d, dxt);
                        if (oracle_site_backward(ns, d, srcs, wq, g ? gk : NULL, gamma ? gm : NULL, 1, eps, dxt,
                                                 dus, lw + ll * d, lg + ll * d, lgm + ll * d))
                            bad = 1;
                        for (int64_t i = 0; i < n; ++i)
                            for (int64_t k = 0; k < d; ++k) db[i * d + k] += du[i * d + k];
                        if (j > 0)
                            for (int64_t k = 0; k < d; ++k) acc[k] += du[n * d + k];
                    }
                    l_end = l0;
                }
                for (int64_t i = 0; i < 1 + n_given; ++i)
                    memcpy(dreps_out + (i * n_tok + t) * d, db + i * d, sizeof(double) * (size_t)d);
            }
#pragma omp critical
            {
                for (int64_t k = 0; k < (L + 1) * d; ++k) {
                    dw_out[k] += lw[k];
                    dg_out[k] += lg[k];
                }
                for (int64_t k = 0; k < L * d; ++k) dgamma_out[k] += lgm[k];
            }
        }
        free(reps); free(parts); free(db); free(du); free(acc); free(wq); free(dxt);
        free(lw); free(lg); free(lgm); free((void*)srcs); free(dus);
    }
    return bad ? -2 : 0;
}
