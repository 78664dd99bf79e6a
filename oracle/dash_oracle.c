/*
 * dash_oracle.c -- plain double-precision CPU oracle of the DashAttention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY (see dash_oracle.h): the product library never calls this code.
 * [DA] = "DashAttention: Differentiable and Adaptive Sparse Hierarchical Attention",
 * arXiv 2605.18753v1. Readings of points the pages leave open are marked READING.
 */
#include "dash_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

double orc_load(const void* base, int dtype, int64_t i) {
    if (dtype == ORC_F64) return ((const double*)base)[i];
    if (dtype == ORC_F32) return (double)((const float*)base)[i];
    /* bf16 is the upper half of an IEEE binary32 pattern: widen, then convert exactly. */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int64_t div_ceil(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* ---------------------------------------------------------------- Stage 0 [DA §3.1, Eq. 3] */

int orc_pool_keys(const void* k, int dtype, int batch, int n_kv, int h_kv, int head_dim, int block,
                  double* kbar) {
    if (!k || !kbar || batch <= 0 || n_kv <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0)
        return -1;
    const int tc = n_kv / block; /* complete chunks only [DA App. G, Alg. 1] */
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < batch; ++b)
        for (int c = 0; c < tc; ++c)
            for (int r = 0; r < h_kv; ++r)
                for (int e = 0; e < head_dim; ++e) {
                    double s = 0.0;
                    for (int t = c * block; t < (c + 1) * block; ++t)
                        s += orc_load(k, dtype, (((int64_t)b * n_kv + t) * h_kv + r) * head_dim + e);
                    kbar[(((int64_t)b * tc + c) * h_kv + r) * head_dim + e] = s / block;
                }
    return 0;
}

int orc_pool_keys_query_ex(const void* k, int dtype, const double* qbar, int64_t qbar_batch_stride,
                           int64_t qbar_chunk_stride, int batch, int n_kv, int h_kv, int head_dim,
                           int block, double* kbar) {
    if (!k || !qbar || !kbar || batch <= 0 || n_kv <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0 ||
        qbar_batch_stride < 0 || qbar_chunk_stride < 0)
        return -1;
    const int tc = n_kv / block;
    const double inv_sqrt_d = 1.0 / sqrt((double)head_dim);
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < batch; ++b)
        for (int c = 0; c < tc; ++c)
            for (int r = 0; r < h_kv; ++r) {
                /* the summary query of this chunk and KV head [DA App. G, Alg. 1: one per chunk] */
                const double* qc = qbar + b * qbar_batch_stride + c * qbar_chunk_stride + (int64_t)r * head_dim;
                /* logits <qbar_c^(r), k_t> / sqrt(D) over the chunk's own tokens */
                double* s = malloc(sizeof(double) * block);
                double smax = -INFINITY;
                for (int u = 0; u < block; ++u) {
                    int64_t base = (((int64_t)b * n_kv + c * block + u) * h_kv + r) * head_dim;
                    double dot = 0.0;
                    for (int e = 0; e < head_dim; ++e)
                        dot += qc[e] * orc_load(k, dtype, base + e);
                    s[u] = dot * inv_sqrt_d;
                    if (s[u] > smax) smax = s[u];
                }
                double z = 0.0;
                for (int u = 0; u < block; ++u) z += exp(s[u] - smax);
                for (int e = 0; e < head_dim; ++e) {
                    double acc = 0.0;
                    for (int u = 0; u < block; ++u) {
                        int64_t base = (((int64_t)b * n_kv + c * block + u) * h_kv + r) * head_dim;
                        acc += exp(s[u] - smax) / z * orc_load(k, dtype, base + e);
                    }
                    kbar[(((int64_t)b * tc + c) * h_kv + r) * head_dim + e] = acc;
                }
                free(s);
            }
    return 0;
}

int orc_pool_keys_query(const void* k, int dtype, const double* qbar, int batch, int n_kv,
                        int h_kv, int head_dim, int block, double* kbar) {
    return orc_pool_keys_query_ex(k, dtype, qbar, 0, 0, batch, n_kv, h_kv, head_dim, block, kbar);
}

/* Gradients of Eq. 3's local attention, chunk by chunk: with s_t = <qbar_c, k_t> / sqrt(D),
 * a = softmax(s) over the chunk's keys and kbar_c = sum_t a_t k_t, a gradient dkbar_c gives
 *   g_t = <dkbar_c, k_t>,  ds_t = a_t (g_t - sum_u a_u g_u)          (the softmax Jacobian)
 *   dk_t += a_t dkbar_c + ds_t qbar_c / sqrt(D)                       (the weights, the logits)
 *   dqbar_c = sum_t ds_t k_t / sqrt(D)
 * dk [B, n_kv, h_kv, D] is added to; dqbar_full [B, Tc, h_kv, D] receives each chunk's own
 * dqbar_c (a query shared by several chunks or sequences collects the sum of theirs). */
int orc_pool_keys_query_backward(const void* k, int dtype, const double* qbar,
                                 int64_t qbar_batch_stride, int64_t qbar_chunk_stride,
                                 const double* dkbar, int batch, int n_kv, int h_kv, int head_dim,
                                 int block, double* dk, double* dqbar_full) {
    if (!k || !qbar || !dkbar || !dk || !dqbar_full || batch <= 0 || n_kv <= 0 || h_kv <= 0 ||
        head_dim <= 0 || block <= 0 || qbar_batch_stride < 0 || qbar_chunk_stride < 0)
        return -1;
    const int tc = n_kv / block;
    const double inv_sqrt_d = 1.0 / sqrt((double)head_dim);
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < batch; ++b)
        for (int c = 0; c < tc; ++c)
            for (int r = 0; r < h_kv; ++r) {
                const double* qc = qbar + b * qbar_batch_stride + c * qbar_chunk_stride + (int64_t)r * head_dim;
                const double* dkb = dkbar + (((int64_t)b * tc + c) * h_kv + r) * head_dim;
                double* a = malloc(sizeof(double) * block);
                double* g = malloc(sizeof(double) * block);
                double smax = -INFINITY;
                for (int u = 0; u < block; ++u) {
                    const int64_t base = (((int64_t)b * n_kv + c * block + u) * h_kv + r) * head_dim;
                    double dot = 0.0, gd = 0.0;
                    for (int e = 0; e < head_dim; ++e) {
                        const double kv = orc_load(k, dtype, base + e);
                        dot += qc[e] * kv;
                        gd += dkb[e] * kv;
                    }
                    a[u] = dot * inv_sqrt_d;
                    g[u] = gd;
                    if (a[u] > smax) smax = a[u];
                }
                double z = 0.0;
                for (int u = 0; u < block; ++u) {
                    a[u] = exp(a[u] - smax);
                    z += a[u];
                }
                double gbar = 0.0;
                for (int u = 0; u < block; ++u) {
                    a[u] /= z;
                    gbar += a[u] * g[u];
                }
                double* dq = dqbar_full + (((int64_t)b * tc + c) * h_kv + r) * head_dim;
                for (int e = 0; e < head_dim; ++e) dq[e] = 0.0;
                for (int u = 0; u < block; ++u) {
                    const double ds = a[u] * (g[u] - gbar);
                    const int64_t base = (((int64_t)b * n_kv + c * block + u) * h_kv + r) * head_dim;
                    for (int e = 0; e < head_dim; ++e) {
                        dk[base + e] += a[u] * dkb[e] + ds * qc[e] * inv_sqrt_d;
                        dq[e] += ds * orc_load(k, dtype, base + e) * inv_sqrt_d;
                    }
                }
                free(a);
                free(g);
            }
    return 0;
}

/* ------------------------------------------------ alpha-entmax [DA §2, Eq. 2; App. A, Eq. 13] */

static int cmp_desc(const void* a, const void* b) {
    double x = *(const double*)a, y = *(const double*)b;
    return (x < y) - (x > y);
}

/* Exact threshold by sorting [DA App. A, "Computing the threshold": specialised algorithms
 * exist for alpha = 2 and alpha = 1.5]. With the scores sorted in decreasing order, suppose the
 * support is the top k. Then tau solves
 *   alpha = 2:    sum_{j<=k} (x_(j) - tau)   = 1  ->  tau_k = (S1 - 1) / k
 *   alpha = 1.5:  sum_{j<=k} (x_(j) - tau)^2 = 1  ->  tau_k = M - sqrt((1 - k * V) / k)
 * with S1 the sum, M the mean and V the (population) variance of the top k. A candidate k is
 * consistent when tau_k exists and lies strictly below x_(k); the consistent k form a prefix
 * 1..k* of 1..m (the normalisation function is decreasing and convex), and tau = tau_{k*}. */
double orc_entmax_tau_sort(const double* x, int m, double alpha) {
    if (m <= 0) return INFINITY;
    if (alpha != 2.0 && alpha != 1.5) return NAN;
    double* s = malloc(sizeof(double) * m);
    memcpy(s, x, sizeof(double) * m);
    qsort(s, m, sizeof(double), cmp_desc);
    double s1 = 0.0, s2 = 0.0, tau = NAN;
    for (int k = 1; k <= m; ++k) {
        s1 += s[k - 1];
        s2 += s[k - 1] * s[k - 1];
        double tk;
        if (alpha == 2.0) {
            tk = (s1 - 1.0) / k;
        } else {
            double mean = s1 / k;
            double var = s2 / k - mean * mean;
            double delta = (1.0 - k * var) / k;
            if (delta < 0.0) break;
            tk = mean - sqrt(delta);
        }
        if (!(tk < s[k - 1])) break;
        tau = tk;
    }
    free(s);
    return tau;
}

/* Normalisation residual f(tau) = sum_c [x_c - tau]_+^(1/(alpha-1)) - 1, decreasing in tau. */
static double entmax_residual(const double* x, int m, double alpha, double tau) {
    const double e = 1.0 / (alpha - 1.0);
    double s = 0.0;
    for (int c = 0; c < m; ++c)
        if (x[c] > tau) s += pow(x[c] - tau, e);
    return s - 1.0;
}

/* Bisection [DA App. A: "bisection over a bounded interval"]. READING: the bracket is derived,
 * not printed. At tau = max x - 1 the largest term alone equals 1, so f >= 0; at
 * tau = max x - m^(1-alpha) every term is at most 1/m, so f <= 0. */
double orc_entmax_tau_bisect(const double* x, int m, double alpha, int iters) {
    if (m <= 0) return INFINITY;
    double xmax = -INFINITY;
    for (int c = 0; c < m; ++c)
        if (x[c] > xmax) xmax = x[c];
    double lo = xmax - 1.0, hi = xmax - pow((double)m, 1.0 - alpha);
    for (int it = 0; it < iters; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (entmax_residual(x, m, alpha, mid) >= 0.0)
            lo = mid;
        else
            hi = mid;
    }
    return 0.5 * (lo + hi);
}

double orc_entmax_tau(const double* x, int m, double alpha) {
    if (alpha == 2.0 || alpha == 1.5) return orc_entmax_tau_sort(x, m, alpha);
    return orc_entmax_tau_bisect(x, m, alpha, 200);
}

void orc_entmax_probs(const double* x, int m, double alpha, double tau, double* p) {
    const double e = 1.0 / (alpha - 1.0);
    for (int c = 0; c < m; ++c) p[c] = x[c] > tau ? pow(x[c] - tau, e) : 0.0;
}

/* ------------------------------------------------- Stage 1 [DA §3.2, Eq. 4; App. G, Alg. 2] */

int orc_block_entmax(const void* q, int dtype, const double* kbar, int batch, int n_q, int q_pos0,
                     int n_kv, int h_q, int h_kv, int head_dim, int block, double alpha,
                     double gamma, double sigma, int window, const int64_t* rows, int64_t n_rows,
                     uint32_t* mask, double* bias, double* tau, double* x, double* w) {
    if (!q || !kbar || !mask || !bias || !tau || window < 1) return -1;
    if (batch <= 0 || n_q <= 0 || n_kv <= 0 || h_q <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0)
        return -1;
    if (h_q % h_kv != 0 || q_pos0 < 0 || q_pos0 + n_q > n_kv) return -1;
    if (!(alpha > 1.0 && alpha <= 2.0) || !(gamma > 0.0) || !(sigma > 0.0)) return -1;
    if (!rows) n_rows = (int64_t)batch * n_q;
    const int gq = h_q / h_kv;
    const int tc = n_kv / block;
    const int nc = (int)div_ceil(n_kv, block);
    const int nw = (int)div_ceil(nc, 32);
    const double inv_sqrt_d = 1.0 / sqrt((double)head_dim);

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t kk = 0; kk < n_rows; ++kk) {
        const int64_t rho = rows ? rows[kk] : kk;
        const int b = (int)(rho / n_q), t = (int)(rho % n_q);
        const int pos = q_pos0 + t;
        const int ci = pos / block; /* the query's own (diagonal) chunk */
        /* READING: routing covers the complete chunks strictly before the query's own chunk,
         * c < c_i [DA App. G, Alg. 2]; c_i <= Tc always holds. READING: with a window of W
         * blocks [DA App. B.1.1: the diagonal block and the block before it], the W - 1 blocks
         * before c_i are attended like the diagonal (always, d = 0) and leave the routing
         * candidates, which become c < c_i - W + 1; chunks below 0 do not exist. */
        const int lo = ci - (window - 1) > 0 ? ci - (window - 1) : 0; /* first window chunk */
        const int m = lo < tc ? lo : tc;
        double* xr = malloc(sizeof(double) * (m > 0 ? m : 1) * gq);
        double* pr = malloc(sizeof(double) * (m > 0 ? m : 1) * gq);
        double* wr = malloc(sizeof(double) * (m > 0 ? m : 1));

        for (int r = 0; r < h_kv; ++r) {
            /* chunk logits and per-head entmax [DA Eq. 4] */
            for (int g = 0; g < gq; ++g) {
                const int h = r * gq + g; /* head h belongs to group floor(h / gq) */
                const int64_t qb = (((int64_t)b * n_q + t) * h_q + h) * head_dim;
                for (int c = 0; c < m; ++c) {
                    const double* kb = kbar + (((int64_t)b * tc + c) * h_kv + r) * head_dim;
                    double dot = 0.0;
                    for (int e = 0; e < head_dim; ++e) dot += orc_load(q, dtype, qb + e) * kb[e];
                    /* entmax argument (alpha - 1) * gamma * zbar  [DA Eq. 2 and Eq. 4] */
                    xr[g * m + c] = (alpha - 1.0) * gamma * dot * inv_sqrt_d;
                }
                double th = orc_entmax_tau(xr + g * m, m, alpha);
                tau[kk * h_q + h] = th;
                orc_entmax_probs(xr + g * m, m, alpha, th, pr + g * m);
                if (x) {
                    double* xo = x + (kk * h_q + h) * (int64_t)nc;
                    for (int c = 0; c < nc; ++c) xo[c] = c < m ? xr[g * m + c] : NAN;
                }
            }
            /* GQA: mean of the group's head probabilities; the support is the union [DA §3.2] */
            for (int c = 0; c < m; ++c) {
                double s = 0.0;
                for (int g = 0; g < gq; ++g) s += pr[g * m + c];
                wr[c] = s / gq;
            }
            /* routed set R, mask bits and bias d = (log w - mu) / sigma  [DA Prop. 1; Alg. 2] */
            uint32_t* mw = mask + (kk * h_kv + r) * (int64_t)nw;
            double* bo = bias + (kk * h_kv + r) * (int64_t)nc;
            memset(mw, 0, sizeof(uint32_t) * nw);
            for (int c = 0; c < nc; ++c) bo[c] = 0.0;
            int n_routed = 0;
            double sum_log = 0.0;
            for (int c = 0; c < m; ++c)
                if (wr[c] > 0.0) {
                    ++n_routed;
                    sum_log += log(wr[c]);
                }
            /* READING: with no routed chunk (c_i = 0) mu is never needed; the row attends to
             * its own chunk only. */
            const double mu = n_routed > 0 ? sum_log / n_routed : 0.0;
            for (int c = 0; c < m; ++c)
                if (wr[c] > 0.0) {
                    mw[c / 32] |= 1u << (c % 32);
                    bo[c] = isinf(sigma) ? 0.0 : (log(wr[c]) - mu) / sigma;
                }
            /* the diagonal chunk [DA §3.4; Alg. 2] and the window's chunks before it
             * [DA App. B.1.1]: always attended, no bias */
            for (int c = lo; c <= ci; ++c) {
                mw[c / 32] |= 1u << (c % 32);
                bo[c] = 0.0;
            }
            if (w) {
                double* wo = w + (kk * h_kv + r) * (int64_t)nc;
                for (int c = 0; c < nc; ++c) wo[c] = c < m ? wr[c] : 0.0;
            }
        }
        free(xr);
        free(pr);
        free(wr);
    }
    return 0;
}

/* ---------------------------------------------- Stage 2 [DA §3.3-3.4, Eq. 7-10, Prop. 1] */

static int check_attn_args(const void* q, const void* k, const void* v, int batch, int n_q,
                           int q_pos0, int n_kv, int h_q, int h_kv, int head_dim, int block) {
    if (!q || !k || !v) return -1;
    if (batch <= 0 || n_q <= 0 || n_kv <= 0 || h_q <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0)
        return -1;
    if (h_q % h_kv != 0 || q_pos0 < 0 || q_pos0 + n_q > n_kv) return -1;
    return 0;
}

static int mask_bit(const uint32_t* words, int c) { return (words[c / 32] >> (c % 32)) & 1u; }

int orc_sparse_attn(const void* q, const void* k, const void* v, int dtype, const uint32_t* mask,
                    const double* bias, int batch, int n_q, int q_pos0, int n_kv, int h_q, int h_kv,
                    int head_dim, int block, double scale, const int64_t* rows, int64_t n_rows,
                    double* o, double* lse) {
    if (check_attn_args(q, k, v, batch, n_q, q_pos0, n_kv, h_q, h_kv, head_dim, block) || !mask ||
        !bias || !o)
        return -1;
    if (!rows) n_rows = (int64_t)batch * n_q;
    const int gq = h_q / h_kv;
    const int nc = (int)div_ceil(n_kv, block);
    const int nw = (int)div_ceil(nc, 32);

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t kk = 0; kk < n_rows; ++kk) {
        const int64_t rho = rows ? rows[kk] : kk;
        const int b = (int)(rho / n_q), t = (int)(rho % n_q);
        const int pos = q_pos0 + t;
        const int ci = pos / block;
        /* attended tokens: every token of each routed chunk c < c_i, then the causal prefix
         * c_i*B .. pos of the query's own chunk [DA Prop. 1; Alg. 3] */
        int* tok = malloc(sizeof(int) * (pos + 1));
        double* lg = malloc(sizeof(double) * (pos + 1));
        for (int h = 0; h < h_q; ++h) {
            const int r = h / gq;
            const uint32_t* mw = mask + (kk * h_kv + r) * (int64_t)nw;
            const double* bw = bias + (kk * h_kv + r) * (int64_t)nc;
            const int64_t qb = (((int64_t)b * n_q + t) * h_q + h) * head_dim;
            int nt = 0;
            for (int c = 0; c <= ci; ++c) {
                if (c < ci && !mask_bit(mw, c)) continue;
                const int end = c < ci ? (c + 1) * block : pos + 1;
                const double d = c < ci ? bw[c] : 0.0;
                for (int j = c * block; j < end; ++j) {
                    const int64_t kb = (((int64_t)b * n_kv + j) * h_kv + r) * head_dim;
                    double dot = 0.0;
                    for (int e = 0; e < head_dim; ++e)
                        dot += orc_load(q, dtype, qb + e) * orc_load(k, dtype, kb + e);
                    tok[nt] = j;
                    lg[nt] = scale * dot + d;
                    ++nt;
                }
            }
            double lmax = -INFINITY;
            for (int u = 0; u < nt; ++u)
                if (lg[u] > lmax) lmax = lg[u];
            double z = 0.0;
            for (int u = 0; u < nt; ++u) z += exp(lg[u] - lmax);
            double* oo = o + (kk * h_q + h) * (int64_t)head_dim;
            for (int e = 0; e < head_dim; ++e) {
                double acc = 0.0;
                for (int u = 0; u < nt; ++u)
                    acc += exp(lg[u] - lmax) *
                           orc_load(v, dtype, (((int64_t)b * n_kv + tok[u]) * h_kv + r) * head_dim + e);
                oo[e] = acc / z;
            }
            if (lse) lse[kk * h_q + h] = lmax + log(z);
        }
        free(tok);
        free(lg);
    }
    return 0;
}

int orc_sparse_attn_prior(const void* q, const void* k, const void* v, int dtype, const double* w,
                          int batch, int n_q, int q_pos0, int n_kv, int h_q, int h_kv,
                          int head_dim, int block, double scale, double sigma, const int64_t* rows,
                          int64_t n_rows, double* o) {
    if (check_attn_args(q, k, v, batch, n_q, q_pos0, n_kv, h_q, h_kv, head_dim, block) || !w || !o)
        return -1;
    if (!(sigma > 0.0)) return -1;
    if (!rows) n_rows = (int64_t)batch * n_q;
    const int gq = h_q / h_kv;
    const int nc = (int)div_ceil(n_kv, block);
    const double inv_sigma = isinf(sigma) ? 0.0 : 1.0 / sigma;

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t kk = 0; kk < n_rows; ++kk) {
        const int64_t rho = rows ? rows[kk] : kk;
        const int b = (int)(rho / n_q), t = (int)(rho % n_q);
        const int pos = q_pos0 + t;
        const int ci = pos / block;
        double* g = malloc(sizeof(double) * (pos + 1)); /* prior g over tokens 0..pos */
        double* z = malloc(sizeof(double) * (pos + 1));
        for (int r = 0; r < h_kv; ++r) {
            const double* wr = w + (kk * h_kv + r) * (int64_t)nc;
            /* routed branch R (tokens of chunks with w_c > 0) and diagonal branch D */
            int n_chunks = 0;
            double s_pow = 0.0;
            for (int c = 0; c < ci; ++c)
                if (wr[c] > 0.0) {
                    ++n_chunks;
                    s_pow += pow(wr[c], inv_sigma);
                }
            const double n_r = (double)n_chunks * block; /* |R_i| in tokens */
            const double n_d = (double)(pos - ci * block + 1); /* |D_i| */
            double lambda = 0.0; /* READING: no routed chunk -> all prior mass on D_i */
            if (n_chunks > 0) {
                /* strength-reduced prior w'_j = w_c(j)^(1/sigma) / (B * 1^T w^(1/sigma))  [Eq. 8]
                 * KL(u_R || w'_R) = sum_{j in R} (1/|R|) log((1/|R|) / w'_j) */
                double kl = 0.0;
                for (int c = 0; c < ci; ++c)
                    if (wr[c] > 0.0) {
                        const double wp = pow(wr[c], inv_sigma) / (block * s_pow);
                        kl += block * (1.0 / n_r) * log((1.0 / n_r) / wp);
                    }
                /* lambda = sigmoid(KL + log(|R| / |D|))  [Eq. 10] */
                const double arg = kl + log(n_r / n_d);
                lambda = 1.0 / (1.0 + exp(-arg));
            }
            /* g_j = lambda * w'_j on R, (1 - lambda) / |D| on D, 0 elsewhere  [Eq. 9] */
            for (int j = 0; j <= pos; ++j) {
                const int c = j / block;
                if (c == ci)
                    g[j] = (1.0 - lambda) / n_d;
                else if (wr[c] > 0.0)
                    g[j] = lambda * pow(wr[c], inv_sigma) / (block * s_pow);
                else
                    g[j] = 0.0;
            }
            for (int gg = 0; gg < gq; ++gg) {
                const int h = r * gq + gg;
                const int64_t qb = (((int64_t)b * n_q + t) * h_q + h) * head_dim;
                /* o = sum_j g_j e^{z_j} v_j / sum_j g_j e^{z_j}  [Eq. 7], shifted by max z */
                double zmax = -INFINITY;
                for (int j = 0; j <= pos; ++j) {
                    if (g[j] <= 0.0) continue;
                    const int64_t kb = (((int64_t)b * n_kv + j) * h_kv + r) * head_dim;
                    double dot = 0.0;
                    for (int e = 0; e < head_dim; ++e)
                        dot += orc_load(q, dtype, qb + e) * orc_load(k, dtype, kb + e);
                    z[j] = scale * dot;
                    if (z[j] > zmax) zmax = z[j];
                }
                double den = 0.0;
                for (int j = 0; j <= pos; ++j)
                    if (g[j] > 0.0) den += g[j] * exp(z[j] - zmax);
                double* oo = o + (kk * h_q + h) * (int64_t)head_dim;
                for (int e = 0; e < head_dim; ++e) {
                    double acc = 0.0;
                    for (int j = 0; j <= pos; ++j)
                        if (g[j] > 0.0)
                            acc += g[j] * exp(z[j] - zmax) *
                                   orc_load(v, dtype, (((int64_t)b * n_kv + j) * h_kv + r) * head_dim + e);
                    oo[e] = acc / den;
                }
            }
        }
        free(g);
        free(z);
    }
    return 0;
}

/* ------------------------------------------------ gradients [DA §3.2-3.4, App. A; §3.5 training] */

static double dot_d(const void* a, int dtype, int64_t ia, const void* b, int64_t ib, int d) {
    double s = 0.0;
    for (int e = 0; e < d; ++e) s += orc_load(a, dtype, ia + e) * orc_load(b, dtype, ib + e);
    return s;
}

/* Stage 2 gradients of one query row (sequence b, position t), every head, the selection held
 * fixed [DA Prop. 1, differentiated]: with p_j = exp(scale <q, k_j> + d_c(j) - lse) over the
 * row's tokens, dp_j = <dout, v_j> and ds_j = p_j (dp_j - <dout, o>), it adds
 * dq = scale sum ds_j k_j, dk_j += scale ds_j q, dv_j += p_j dout, and dL/dd_c = sum of ds_j over
 * chunk c's tokens for the routed chunks c < c_i (the own chunk carries the constant d = 0).
 * mw / bo: the row's mask words and bias for each KV head (h_kv * nw, h_kv * nc); dout, o:
 * [h_q, D]; lse [h_q]; dq [h_q, D]; dk, dv [B, n, h_kv, D] or NULL; dbias [h_kv, nc] or NULL. */
static void row_backward(const void* q, const void* k, const void* v, int dtype,
                         const uint32_t* mw, const double* bo, const double* dout,
                         const double* o, const double* lse, int b, int t, int n, int h_q,
                         int h_kv, int D, int block, double scale, double* dq, double* dk,
                         double* dv, double* dbias) {
    const int g = h_q / h_kv, ci = t / block;
    const int nc = (int)div_ceil(n, block), nw = (int)div_ceil(nc, 32);
    const int64_t row = (int64_t)b * n + t;
    for (int h = 0; h < h_q; ++h) {
        const int r = h / g;
        const int64_t qi = (row * h_q + h) * D;
        const double* dh = dout + (int64_t)h * D;
        double dsum = 0.0;
        for (int e = 0; e < D; ++e) dsum += dh[e] * o[(int64_t)h * D + e];
        for (int j = 0; j <= t; ++j) {
            const int c = j / block;
            if (c != ci && !mask_bit(mw + (int64_t)r * nw, c)) continue;
            const int64_t kj = (((int64_t)b * n + j) * h_kv + r) * D;
            const double dval = c == ci ? 0.0 : bo[(int64_t)r * nc + c];
            const double pj = exp(scale * dot_d(q, dtype, qi, k, kj, D) + dval - lse[h]);
            double dp = 0.0;
            for (int e = 0; e < D; ++e) dp += dh[e] * orc_load(v, dtype, kj + e);
            const double ds = pj * (dp - dsum);
            for (int e = 0; e < D; ++e) {
                dq[(int64_t)h * D + e] += scale * ds * orc_load(k, dtype, kj + e);
                if (dk) dk[kj + e] += scale * ds * orc_load(q, dtype, qi + e);
                if (dv) dv[kj + e] += pj * dh[e];
            }
            if (dbias && c != ci) dbias[(int64_t)r * nc + c] += ds;
        }
    }
}

int orc_sparse_attn_backward(const void* q, const void* k, const void* v, int dtype,
                             const uint32_t* mask, const double* bias, const double* dout,
                             int batch, int n, int h_q, int h_kv, int head_dim, int block,
                             double scale, double* dq, double* dk, double* dv, double* dbias) {
    if (check_attn_args(q, k, v, batch, n, 0, n, h_q, h_kv, head_dim, block) || !mask || !bias ||
        !dout || !dq || !dk || !dv)
        return -1;
    const int D = head_dim;
    const int nc = (int)div_ceil(n, block), nw = (int)div_ceil(nc, 32);
    const int64_t R = (int64_t)batch * n;
    double* o = calloc((size_t)R * h_q * D, sizeof(double));
    double* lse = calloc((size_t)R * h_q, sizeof(double));
    if (!o || !lse) {
        free(o);
        free(lse);
        return -1;
    }
    if (orc_sparse_attn(q, k, v, dtype, mask, bias, batch, n, 0, n, h_q, h_kv, D, block, scale,
                        NULL, 0, o, lse)) {
        free(o);
        free(lse);
        return -1;
    }
    memset(dq, 0, sizeof(double) * R * h_q * D);
    memset(dk, 0, sizeof(double) * R * h_kv * D);
    memset(dv, 0, sizeof(double) * R * h_kv * D);
    if (dbias) memset(dbias, 0, sizeof(double) * R * h_kv * nc);
    for (int64_t row = 0; row < R; ++row)
        row_backward(q, k, v, dtype, mask + row * h_kv * nw, bias + row * h_kv * nc,
                     dout + row * h_q * D, o + row * h_q * D, lse + row * h_q, (int)(row / n),
                     (int)(row % n), n, h_q, h_kv, D, block, scale, dq + row * h_q * D, dk, dv,
                     dbias ? dbias + row * h_kv * nc : NULL);
    free(o);
    free(lse);
    return 0;
}

/* dq and dL/dd of the listed rows only (rows[i] = b * n + t, increasing or not): mask, bias,
 * dout, dq and dbias hold one entry per listed row, in list order. */
int orc_sparse_attn_backward_rows(const void* q, const void* k, const void* v, int dtype,
                                  const uint32_t* mask, const double* bias, const double* dout,
                                  int batch, int n, int h_q, int h_kv, int head_dim, int block,
                                  double scale, const int64_t* rows, int64_t n_rows, double* dq,
                                  double* dbias) {
    if (check_attn_args(q, k, v, batch, n, 0, n, h_q, h_kv, head_dim, block) || !mask || !bias ||
        !dout || !dq || !rows || n_rows <= 0)
        return -1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= (int64_t)batch * n) return -1;
    const int D = head_dim;
    const int nc = (int)div_ceil(n, block), nw = (int)div_ceil(nc, 32);
    double* o = calloc((size_t)n_rows * h_q * D, sizeof(double));
    double* lse = calloc((size_t)n_rows * h_q, sizeof(double));
    int rc = -1;
    if (!o || !lse) goto done;
    if (orc_sparse_attn(q, k, v, dtype, mask, bias, batch, n, 0, n, h_q, h_kv, D, block, scale,
                        rows, n_rows, o, lse))
        goto done;
    memset(dq, 0, sizeof(double) * n_rows * h_q * D);
    if (dbias) memset(dbias, 0, sizeof(double) * n_rows * h_kv * nc);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i)
        row_backward(q, k, v, dtype, mask + i * h_kv * nw, bias + i * h_kv * nc,
                     dout + i * h_q * D, o + i * h_q * D, lse + i * h_q, (int)(rows[i] / n),
                     (int)(rows[i] % n), n, h_q, h_kv, D, block, scale, dq + i * h_q * D, NULL,
                     NULL, dbias ? dbias + i * h_kv * nc : NULL);
    rc = 0;
done:
    free(o);
    free(lse);
    return rc;
}

int orc_block_entmax_backward(const void* q, int dtype, const double* kbar, const double* dd,
                              int batch, int n, int h_q, int h_kv, int head_dim, int block,
                              double alpha, double gamma, double sigma, int window,
                              const int64_t* rows, int64_t n_rows, double* dq, double* dkbar) {
    if (!q || !dd || !dq || window < 1) return -1;
    if (batch <= 0 || n <= 0 || h_q <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0 ||
        h_q % h_kv != 0)
        return -1;
    if (!(alpha > 1.0 && alpha <= 2.0) || !(gamma > 0.0) || !(sigma > 0.0)) return -1;
    const int g = h_q / h_kv, tc = n / block, D = head_dim;
    const int nc = (int)div_ceil(n, block), nw = (int)div_ceil(nc, 32);
    if (tc > 0 && !kbar) return -1;
    if (!rows) n_rows = (int64_t)batch * n;
    for (int64_t i = 0; rows && i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= (int64_t)batch * n) return -1;
    uint32_t* mask = calloc((size_t)n_rows * h_kv * nw, sizeof(uint32_t));
    double* bias = calloc((size_t)n_rows * h_kv * nc, sizeof(double));
    double* tau = calloc((size_t)n_rows * h_q, sizeof(double));
    double* x = calloc((size_t)n_rows * h_q * nc, sizeof(double));
    double* w = calloc((size_t)n_rows * h_kv * nc, sizeof(double));
    double* dw = calloc((size_t)n_rows * h_kv * nc, sizeof(double));
    int rc = -1;
    if (!mask || !bias || !tau || !x || !w || !dw) goto done;
    /* the routing of the listed rows, for x, tau and w */
    if (tc > 0 && orc_block_entmax(q, dtype, kbar, batch, n, 0, n, h_q, h_kv, D, block, alpha,
                                   gamma, sigma, window, rows, n_rows, mask, bias, tau, x, w))
        goto done;
    memset(dq, 0, sizeof(double) * n_rows * h_q * D);

    /* d -> w [DA Prop. 1]: d_c = (log w_c - mu) / sigma on R = {c : w_c > 0} (the window's
     * chunks carry the constant d = 0 and have no w) with mu the mean of log w over R, so
     * dL/dlog w_c = (dd_c - mean_R dd) / sigma and dL/dw_c = that / w_c (c in R; 0 elsewhere). */
    if (tc > 0 && !isinf(sigma))
        for (int64_t kk = 0; kk < n_rows; ++kk)
            for (int r = 0; r < h_kv; ++r) {
                const double* wr = w + (kk * h_kv + r) * nc;
                const double* ddr = dd + (kk * h_kv + r) * nc;
                double s = 0.0;
                int nr = 0;
                for (int c = 0; c < nc; ++c)
                    if (wr[c] > 0.0) {
                        s += ddr[c];
                        ++nr;
                    }
                if (nr == 0) continue;
                for (int c = 0; c < nc; ++c)
                    if (wr[c] > 0.0) dw[(kk * h_kv + r) * nc + c] = (ddr[c] - s / nr) / sigma / wr[c];
            }

    /* w -> p_h -> x_h [DA §3.2, Eq. 2; App. A]: w is the mean of the group's heads, so each head
     * receives dp = dw / g; on the support of p = [x - tau]_+^(1/(alpha-1)), with u = p^(2-alpha),
     * the entmax Jacobian gives dx = u (dp - sum(u dp) / sum(u)) / (alpha - 1), 0 off the support.
     * x = coef <q, kbar> with coef = (alpha - 1) gamma / sqrt(D) [Eq. 4]. */
    if (tc > 0) {
        const double coef = (alpha - 1.0) * gamma / sqrt((double)D);
        const double e = 1.0 / (alpha - 1.0);
        for (int64_t kk = 0; kk < n_rows; ++kk) {
            const int64_t rho = rows ? rows[kk] : kk;
            const int b = (int)(rho / n);
            for (int h = 0; h < h_q; ++h) {
                const int r = h / g;
                const double* xr = x + (kk * h_q + h) * nc;
                const double th = tau[kk * h_q + h];
                if (isinf(th)) continue; /* no candidate chunk */
                double su = 0.0, sud = 0.0;
                for (int c = 0; c < nc && !isnan(xr[c]); ++c)
                    if (xr[c] > th) {
                        const double u = pow(pow(xr[c] - th, e), 2.0 - alpha);
                        su += u;
                        sud += u * dw[(kk * h_kv + r) * nc + c] / g;
                    }
                if (su <= 0.0) continue;
                const int64_t qi = (rho * h_q + h) * D;
                for (int c = 0; c < nc && !isnan(xr[c]); ++c) {
                    if (!(xr[c] > th)) continue;
                    const double u = pow(pow(xr[c] - th, e), 2.0 - alpha);
                    const double dx = u * (dw[(kk * h_kv + r) * nc + c] / g - sud / su) / (alpha - 1.0);
                    const int64_t kb = (((int64_t)b * tc + c) * h_kv + r) * D;
                    for (int f = 0; f < D; ++f) {
                        dq[(kk * h_q + h) * D + f] += coef * dx * kbar[kb + f];
                        if (dkbar) dkbar[kb + f] += coef * dx * orc_load(q, dtype, qi + f);
                    }
                }
            }
        }
    }
    rc = 0;
done:
    free(mask); free(bias); free(tau); free(x); free(w); free(dw);
    return rc;
}

int orc_backward(const void* q, const void* k, const void* v, int dtype, const double* dout,
                 int batch, int n, int h_q, int h_kv, int head_dim, int block, double alpha,
                 double gamma, double sigma, int window, double scale, double* dq, double* dk,
                 double* dv, double* dbias) {
    if (check_attn_args(q, k, v, batch, n, 0, n, h_q, h_kv, head_dim, block) || !dout || !dq ||
        !dk || !dv || window < 1)
        return -1;
    if (!(alpha > 1.0 && alpha <= 2.0) || !(gamma > 0.0) || !(sigma > 0.0)) return -1;
    const int tc = n / block;
    const int nc = (int)div_ceil(n, block), nw = (int)div_ceil(nc, 32);
    const int D = head_dim;
    const int64_t R = (int64_t)batch * n;
    double* kbar = calloc((size_t)batch * (tc > 0 ? tc : 1) * h_kv * D, sizeof(double));
    uint32_t* mask = calloc((size_t)R * h_kv * nw, sizeof(uint32_t));
    double* bias = calloc((size_t)R * h_kv * nc, sizeof(double));
    double* tau = calloc((size_t)R * h_q, sizeof(double));
    double* x = calloc((size_t)R * h_q * nc, sizeof(double));
    double* w = calloc((size_t)R * h_kv * nc, sizeof(double));
    double* dd = calloc((size_t)R * h_kv * nc, sizeof(double));
    double* dqr = calloc((size_t)R * h_q * D, sizeof(double));
    double* dkbar = calloc((size_t)batch * (tc > 0 ? tc : 1) * h_kv * D, sizeof(double));
    int rc = -1;
    if (!kbar || !mask || !bias || !tau || !x || !w || !dd || !dqr || !dkbar) goto done;
    /* the forward pass's selection */
    if (tc > 0 && orc_pool_keys(k, dtype, batch, n, h_kv, D, block, kbar)) goto done;
    if (orc_block_entmax(q, dtype, kbar, batch, n, 0, n, h_q, h_kv, D, block, alpha, gamma, sigma,
                         window, NULL, 0, mask, bias, tau, x, w))
        goto done;
    /* Stage 2 with the selection held fixed: dq, dk, dv and dL/dd */
    if (orc_sparse_attn_backward(q, k, v, dtype, mask, bias, dout, batch, n, h_q, h_kv, D, block,
                                 scale, dq, dk, dv, dd))
        goto done;
    /* only the routed chunks' d depends on w (the window's chunks carry the constant d = 0) */
    for (int64_t i = 0; i < R * h_kv * nc; ++i)
        if (!(w[i] > 0.0)) dd[i] = 0.0;
    /* Stage 1: d -> w -> p -> x -> q and kbar */
    if (orc_block_entmax_backward(q, dtype, kbar, dd, batch, n, h_q, h_kv, D, block, alpha, gamma,
                                  sigma, window, NULL, 0, dqr, dkbar))
        goto done;
    for (int64_t i = 0; i < R * h_q * D; ++i) dq[i] += dqr[i];
    /* kbar -> k [DA Eq. 3 with the summary query at zero]: the mean of the chunk's keys */
    for (int b = 0; b < batch; ++b)
        for (int c = 0; c < tc; ++c)
            for (int r = 0; r < h_kv; ++r)
                for (int t = c * block; t < (c + 1) * block; ++t)
                    for (int f = 0; f < D; ++f)
                        dk[(((int64_t)b * n + t) * h_kv + r) * D + f] +=
                            dkbar[(((int64_t)b * tc + c) * h_kv + r) * D + f] / block;
    if (dbias) memcpy(dbias, dd, sizeof(double) * R * h_kv * nc);
    rc = 0;
done:
    free(kbar); free(mask); free(bias); free(tau); free(x); free(w); free(dd); free(dqr);
    free(dkbar);
    return rc;
}
