/*
 * dash_oracle.h -- plain double-precision CPU oracle of the DashAttention forward pass.
 *
 * TEST INFRASTRUCTURE. This code exists to check the GPU library, nothing else. Only the test
 * suite, the smoke check of the package entry module and the CPU-baseline leg of the benchmark
 * may load it. The product library never links, imports or calls it, and shares no code,
 * header, table or helper with it.
 *
 * Source: "DashAttention: Differentiable and Adaptive Sparse Hierarchical Attention"
 * (arXiv 2605.18753v1), cited below as [DA] with section / equation / algorithm numbers:
 *   [DA §2, Eq. 2] and [DA App. A, Eq. 11-13]  alpha-entmax and its threshold tau
 *   [DA §3.1, Eq. 3] and [DA App. G, Alg. 1]   Stage 0, chunk summaries (summary query at zero)
 *   [DA §3.2, Eq. 4] and [DA App. G, Alg. 2]   Stage 1, entmax routing, GQA mean, mask and bias
 *   [DA §3.3-3.4, Eq. 7-10, Prop. 1], [DA App. D] and [DA App. G, Alg. 3]   Stage 2
 *
 * Every routine is a straight transcription of the definition it cites: loops over rows,
 * heads, chunks and tokens in double, no blocking, no fusion, no reordering beyond the
 * definition. Inputs may be fp32 or bf16 (raw 16-bit patterns); both convert to double exactly.
 *
 * Layouts (all row-major, token-major as in the "Require" clauses of [DA App. G, Alg. 1-3]):
 *   q    [batch, n_q,  h_q,  head_dim]      query at row t sits at absolute position q_pos0 + t
 *   k, v [batch, n_kv, h_kv, head_dim]
 *   kbar [batch, Tc,   h_kv, head_dim]      Tc = floor(n_kv / block)   (complete chunks only)
 *   For a list of query rows rho = b * n_q + t (rows == NULL means every row in order), the
 *   per-row outputs are compact, indexed by the position k of rho in the list:
 *   mask [n_rows, h_kv, W] uint32, W = ceil(Nc / 32), Nc = ceil(n_kv / block); chunk c is bit
 *        (c mod 32) of word floor(c / 32)
 *   bias [n_rows, h_kv, Nc]   routing bias d; entries whose mask bit is 0 are written as 0
 *   tau  [n_rows, h_q]        threshold in x-units; +inf for a row with no complete chunk before it
 *   x    [n_rows, h_q, Nc]    entmax argument x_c = (alpha-1) * gamma * <q, kbar_c> / sqrt(D),
 *                             entries c >= c_i written as NaN (optional output)
 *   w    [n_rows, h_kv, Nc]   GQA-averaged chunk probabilities, 0 for c >= c_i (optional output)
 *   o    [n_rows, h_q, head_dim], lse [n_rows, h_q]
 *
 * All functions return 0 on success and a negative value on invalid arguments.
 */
#ifndef DASH_ORACLE_H
#define DASH_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

/* Value i of an fp32, bf16 or fp64 array, exactly, in double. */
double orc_load(const void* base, int dtype, int64_t i);

/* Stage 0 with the learned summary query at zero: Eq. 3 then weighs every token of a chunk
 * equally, so each complete chunk is summarised by the arithmetic mean of its keys. */
int orc_pool_keys(const void* k, int dtype, int batch, int n_kv, int h_kv, int head_dim, int block,
                  double* kbar);

/* Stage 0 with a learned summary query qbar [h_kv, head_dim] (double): the local SDPA of
 * Eq. 3, a softmax over the chunk's own keys of <qbar, k_t>/sqrt(D), used to weigh the keys. */
int orc_pool_keys_query(const void* k, int dtype, const double* qbar, int batch, int n_kv,
                        int h_kv, int head_dim, int block, double* kbar);
/* The same with a summary query per chunk [DA App. G, Alg. 1, which takes qbar with one row per
 * chunk and KV head]: the query of sequence b, chunk c, KV head r is the head_dim values at
 * qbar + b * qbar_batch_stride + c * qbar_chunk_stride + r * head_dim (strides in elements;
 * 0 and 0 give one query per KV head, shared by all chunks). */
int orc_pool_keys_query_ex(const void* k, int dtype, const double* qbar, int64_t qbar_batch_stride,
                           int64_t qbar_chunk_stride, int batch, int n_kv, int h_kv, int head_dim,
                           int block, double* kbar);

/* Gradients of the learned-query pooling (Eq. 3) for dL/dkbar = dkbar [B, Tc, h_kv, D]: adds to
 * dk [B, n_kv, h_kv, D] and writes each chunk's dL/dqbar_c into dqbar_full [B, Tc, h_kv, D]
 * (queries addressed as in orc_pool_keys_query_ex). */
int orc_pool_keys_query_backward(const void* k, int dtype, const double* qbar,
                                 int64_t qbar_batch_stride, int64_t qbar_chunk_stride,
                                 const double* dkbar, int batch, int n_kv, int h_kv, int head_dim,
                                 int block, double* dk, double* dqbar_full);

/* alpha-entmax threshold for x[0..m-1] (x already holds (alpha-1) * scores):
 * the unique tau with sum_c [x_c - tau]_+^(1/(alpha-1)) = 1.
 *   _sort:   exact sort-based solution, alpha = 2 (sparsemax) or alpha = 1.5 only (NaN otherwise)
 *   _bisect: bisection on the bracket [max x - 1, max x - m^(1-alpha)], any alpha in (1, 2]
 *   orc_entmax_tau: _sort for alpha in {1.5, 2}, _bisect (200 halvings) otherwise. */
double orc_entmax_tau_sort(const double* x, int m, double alpha);
double orc_entmax_tau_bisect(const double* x, int m, double alpha, int iters);
double orc_entmax_tau(const double* x, int m, double alpha);
/* p_c = [x_c - tau]_+^(1/(alpha-1)) */
void orc_entmax_probs(const double* x, int m, double alpha, double tau, double* p);

/* Stage 1 for the listed query rows: chunk scores, per-head entmax, GQA mean, mask and bias.
 * window >= 1 blocks are always attended: the query's own chunk and the window - 1 before it
 * (the training window of [DA App. B.1.1] is window = 2); routing covers the complete chunks
 * before them. window = 1 is [DA Alg. 2] as printed. */
int orc_block_entmax(const void* q, int dtype, const double* kbar, int batch, int n_q, int q_pos0,
                     int n_kv, int h_q, int h_kv, int head_dim, int block, double alpha,
                     double gamma, double sigma, int window, const int64_t* rows, int64_t n_rows,
                     uint32_t* mask, double* bias, double* tau, double* x, double* w);

/* Stage 2, bias form (Prop. 1): softmax of scale * <q, k_j> + d_c(j) over the tokens of the
 * routed chunks (mask bits below the query's own chunk) and the causal part of the query's own
 * chunk (d = 0 there), then the weighted sum of values. mask / bias are per listed row, in the
 * compact layout orc_block_entmax writes. */
int orc_sparse_attn(const void* q, const void* k, const void* v, int dtype, const uint32_t* mask,
                    const double* bias, int batch, int n_q, int q_pos0, int n_kv, int h_q, int h_kv,
                    int head_dim, int block, double scale, const int64_t* rows, int64_t n_rows,
                    double* o, double* lse);

/* Stage 2, prior form (Eq. 7 with the prior g of Eq. 8-10), from the GQA-averaged chunk
 * probabilities w of each listed row. Independent of the bias form; Prop. 1 says they agree. */
int orc_sparse_attn_prior(const void* q, const void* k, const void* v, int dtype, const double* w,
                          int batch, int n_q, int q_pos0, int n_kv, int h_q, int h_kv,
                          int head_dim, int block, double scale, double sigma, const int64_t* rows,
                          int64_t n_rows, double* o);

/* Gradients of Stage 2 alone (bias form, Prop. 1) for prefill, every query row, with the mask and
 * the bias held fixed: dq [B, n, H_q, D], dk, dv [B, n, H_kv, D] and, when dbias is not NULL,
 * dL/dd [B, n, H_kv, Nc] for every chunk below the query's own whose mask bit is set (0 elsewhere). */
int orc_sparse_attn_backward(const void* q, const void* k, const void* v, int dtype,
                             const uint32_t* mask, const double* bias, const double* dout,
                             int batch, int n, int h_q, int h_kv, int head_dim, int block,
                             double scale, double* dq, double* dk, double* dv, double* dbias);

/* dq and dL/dd of the listed query rows only (rows[i] = b * n + t); mask [R, H_kv, W], bias
 * [R, H_kv, Nc], dout and dq [R, H_q, D], dbias [R, H_kv, Nc] hold one entry per listed row. */
int orc_sparse_attn_backward_rows(const void* q, const void* k, const void* v, int dtype,
                                  const uint32_t* mask, const double* bias, const double* dout,
                                  int batch, int n, int h_q, int h_kv, int head_dim, int block,
                                  double scale, const int64_t* rows, int64_t n_rows, double* dq,
                                  double* dbias);

/* Gradients of Stage 1 (the routing) for prefill, the selection held fixed: from dd = dL/dd of
 * the listed rows (rows[i] = b * n + t; every row when rows is NULL) [R, H_kv, Nc], the chain
 * d -> log w (mu couples the routed chunks) -> w (the GQA mean) -> each head's entmax (its
 * Jacobian on the support) -> x = coef <q, kbar>. Writes the routing part of dq for the listed
 * rows [R, H_q, D] and, when dkbar is not NULL, adds coef * sum of dx q into dkbar [B, Tc, H_kv, D].
 * kbar [B, Tc, H_kv, D] are the mean-pooled summaries the forward routed with. */
int orc_block_entmax_backward(const void* q, int dtype, const double* kbar, const double* dd,
                              int batch, int n, int h_q, int h_kv, int head_dim, int block,
                              double alpha, double gamma, double sigma, int window,
                              const int64_t* rows, int64_t n_rows, double* dq, double* dkbar);

/* Gradients of the whole forward pass (Stage 0 mean pooling, Stage 1 routing, Stage 2 bias-form
 * attention) for prefill (every query row, q_pos0 = 0), given dout = dL/do [B, n, H_q, D]:
 * dq [B, n, H_q, D], dk, dv [B, n, H_kv, D] and, when dbias is not NULL, dL/dd for every routed
 * chunk [B, n, H_kv, Nc] (0 elsewhere). The selection (the support of each entmax and the routed
 * set R) is piecewise constant, so no gradient flows through which chunks are selected; within a
 * fixed support the chain is d -> log w (mu couples the routed chunks) -> w (the GQA mean) -> each
 * head's entmax (its Jacobian) -> the chunk scores -> q and the summaries -> k (mean pooling). */
int orc_backward(const void* q, const void* k, const void* v, int dtype, const double* dout,
                 int batch, int n, int h_q, int h_kv, int head_dim, int block, double alpha,
                 double gamma, double sigma, int window, double scale, double* dq, double* dk,
                 double* dv, double* dbias);

/* Number of OpenMP threads the oracle's row loops use. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* DASH_ORACLE_H */
