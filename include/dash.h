/*
 * dash.h -- C ABI of libdash, the DashAttention forward pass on AMD Instinct MI355X (gfx950).
 *
 * Method: "DashAttention: Differentiable and Adaptive Sparse Hierarchical Attention"
 * (arXiv 2605.18753v1), cited as [DA]. Three stages over Q, K, V backed by a cache of chunk
 * summaries [DA §3.5]:
 *   Stage 0  dash_pool_keys            chunk summaries kbar              [DA §3.1 Eq. 3; Alg. 1]
 *   Stage 1  dash_block_entmax         alpha-entmax routing: mask, bias   [DA §3.2 Eq. 4; Alg. 2]
 *   Stage 2  dash_sparse_attn_prefill  prior-biased sparse softmax        [DA §3.3-3.4 Prop. 1; Alg. 3]
 *            dash_sparse_attn_decode   the same for one new token per sequence, split over the
 *                                      selected chunks                   [DA §3.5 "split-KV variant"]
 * Incremental decoding with a length per sequence (a cache of capacity n_cap, sequence b holding
 * ctx_lens[b] tokens): dash_pool_keys_append writes the summary of a chunk the newest token
 * completed [DA §3.1, §3.5]; dash_block_entmax_ex and dash_sparse_attn_decode_varlen take the
 * lengths. dash_block_entmax_ex also takes the attention window of [DA App. B.1.1].
 *
 * Notation: B = batch, n = sequence length, H_q / H_kv = query / key-value heads, g = H_q / H_kv
 * (query head h belongs to KV group floor(h / g)), D = head dim, Bc = chunk (block) size,
 * Tc = floor(n_kv / Bc) complete chunks (those with a summary), Nc = ceil(n_kv / Bc) chunk slots,
 * W = ceil(Nc / 32) mask words. A query at absolute position p lies in chunk c_p = floor(p / Bc).
 *
 * Layouts (row-major, token-major as in the "Require" clauses of [DA Alg. 1-3]):
 *   q            [B, n_q, H_q, D]       dtype dt
 *   k, v         [B, n_kv, H_kv, D]     dtype dt
 *   kbar         [B, Tc, H_kv, D]       fp32
 *   mask         [B, n_q, H_kv, W]      uint32; chunk c is bit (c mod 32) of word floor(c / 32)
 *   bias         [B, n_q, H_kv, Nc]     fp32 routing bias d of [DA Prop. 1]
 *   tau          [B, n_q, H_q]          fp32 entmax threshold in x-units (see dash_block_entmax)
 *   o            [B, n_q, H_q, D]       dtype dt;   lse [B, n_q, H_q] fp32
 *
 * Conventions
 *   Ownership:   every pointer is device memory owned by the caller. The library allocates
 *                nothing and keeps no pointer after a call returns.
 *   Asynchrony:  every call enqueues its kernels on `stream` and returns without waiting.
 *                Calls are thread-safe; the only state is the thread-local error string.
 *   Sizes:       batch, lengths and head counts are at least 1; an empty call (a zero size) is
 *                DASH_ERR_INVALID, not a silent no-op.
 *   Errors:      arguments are validated before anything is launched. Invalid arguments give
 *                DASH_ERR_INVALID, valid but unimplemented shapes DASH_ERR_UNSUPPORTED, a short
 *                workspace DASH_ERR_WORKSPACE, a failed launch DASH_ERR_HIP; nothing is launched
 *                on a validation error. dash_last_error() gives the detail. Faults inside a
 *                kernel surface at the caller's next synchronisation. No exception crosses the ABI.
 *   Determinism: the same inputs give bitwise-equal outputs (no floating-point atomics).
 *   Supported:   dt in {DASH_F32, DASH_BF16}; D in {64, 128}; Bc in {32, 64, 128};
 *                g in {1, 2, 4, 8, 16}; Nc <= 8192.
 */
#ifndef DASH_H
#define DASH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DASH_OK = 0,
    DASH_ERR_INVALID = 1,
    DASH_ERR_UNSUPPORTED = 2,
    DASH_ERR_WORKSPACE = 3,
    DASH_ERR_HIP = 4
} dash_status_t;

typedef enum { DASH_F32 = 0, DASH_BF16 = 1 } dash_dtype_t;

/* Static text naming a status code. */
const char* dash_status_string(dash_status_t s);

/* Detail of the calling thread's last non-OK return ("" if none). Valid until the next call. */
const char* dash_last_error(void);

/* Library version, as major * 10000 + minor * 100 + patch. */
int dash_version(void);

/*
 * Stage 0 [DA §3.1, Eq. 3 with the learned summary query at its zero initialisation, where the
 * local softmax is uniform; DA App. G, Alg. 1]: each complete chunk c < Tc of each KV head is
 * summarised by the mean of its Bc keys, accumulated in fp32.
 *   k     [B, n_kv, H_kv, D] (dt)      kbar [B, Tc, H_kv, D] fp32 (written in full)
 * The trailing n_kv - Tc * Bc keys of an incomplete chunk get no summary (kbar may be NULL when
 * Tc = 0, here and in dash_block_entmax). The summaries only
 * depend on their own chunk, so a decode loop can pool once and keep kbar as a cache.
 */
dash_status_t dash_pool_keys(const void* k, dash_dtype_t dt, float* kbar, int batch, int n_kv,
                             int h_kv, int head_dim, int block, hipStream_t stream);

/*
 * Stage 0 with a learned summary query [DA §3.1, Eq. 3; Alg. 1]: kbar_c = sum_t softmax_t(
 * <qbar^(r), k_t> / sqrt(D)) k_t over the chunk's own keys.  qbar [H_kv, D] fp32.
 */
dash_status_t dash_pool_keys_query(const void* k, dash_dtype_t dt, const float* qbar, float* kbar,
                                   int batch, int n_kv, int h_kv, int head_dim, int block,
                                   hipStream_t stream);

/*
 * Stage 0 with one learned summary query per chunk [DA App. G, Alg. 1: qbar has one row per
 * chunk and KV head, rotary position embedding already applied by the caller]: as
 * dash_pool_keys_query, with the query of sequence b, chunk c, KV head r read at
 *   qbar + b * qbar_batch_stride + c * qbar_chunk_stride + r * D      (strides in floats)
 * so qbar [Tc, H_kv, D] shared by the batch is (0, H_kv * D), qbar [B, Tc, H_kv, D] is
 * (Tc * H_kv * D, H_kv * D), and (0, 0) is dash_pool_keys_query's one query per KV head. Strides
 * are non-negative multiples of 4 (16-byte rows); the caller keeps every addressed row in bounds.
 */
dash_status_t dash_pool_keys_query_ex(const void* k, dash_dtype_t dt, const float* qbar,
                                      int64_t qbar_batch_stride, int64_t qbar_chunk_stride,
                                      float* kbar, int batch, int n_kv, int h_kv, int head_dim,
                                      int block, hipStream_t stream);

/*
 * Stage 0, streaming [DA §3.1 (a summary is final once its chunk is complete), §3.5 (the chunk
 * cache persisted across decoding steps)]: after the newest token of sequence b was appended
 * (ctx_lens[b] tokens in the cache, device int32 [B]), the summary of chunk ctx_lens[b] / Bc - 1
 * is written into kbar when ctx_lens[b] is a positive multiple of Bc; otherwise nothing is
 * written for that sequence. The mean (qbar NULL) or the learned-query form (qbar [H_kv, D]
 * fp32), as dash_pool_keys / dash_pool_keys_query.
 *   k_cache [B, n_cap, H_kv, D] (dt)     kbar [B, floor(n_cap / Bc), H_kv, D] fp32
 * Lengths outside [0, n_cap] are clamped into it on the device (no error can be reported there).
 */
dash_status_t dash_pool_keys_append(const void* k_cache, dash_dtype_t dt, const float* qbar,
                                    const int32_t* ctx_lens, float* kbar, int batch, int n_cap,
                                    int h_kv, int head_dim, int block, hipStream_t stream);

/* dash_pool_keys_append with one summary query per chunk, addressed as in
 * dash_pool_keys_query_ex (the query of the chunk being completed is used; qbar NULL: the
 * mean, strides ignored). */
dash_status_t dash_pool_keys_append_ex(const void* k_cache, dash_dtype_t dt, const float* qbar,
                                       int64_t qbar_batch_stride, int64_t qbar_chunk_stride,
                                       const int32_t* ctx_lens, float* kbar, int batch, int n_cap,
                                       int h_kv, int head_dim, int block, hipStream_t stream);

/*
 * Stage 1 [DA §3.2, Eq. 4; DA App. G, Alg. 2]. Query row t (t < n_q) sits at absolute position
 * p = q_pos0 + t of a sequence of n_kv keys (prefill: q_pos0 = 0, n_q = n_kv; decode: n_q = 1,
 * q_pos0 = n_kv - 1, the new token's key and value already appended). For every query head h it
 *   1. scores the complete chunks before its own, c < c_p:
 *        x_c = (alpha - 1) * gamma * <q_p^(h), kbar_c^(h / g)> / sqrt(D)          (x-units)
 *   2. finds the entmax threshold tau with sum_c [x_c - tau]_+^(1/(alpha-1)) = 1 [DA Eq. 2]
 *      (alpha in {1.5, 2}: closed-form roots on the current support inside a shrinking bracket,
 *      ending when the support is stable; other alpha: Newton steps with a bisection guard)
 *      and p_c = [x_c - tau]_+^(1/(alpha-1));
 * then for every KV group r
 *   3. averages the probabilities of the group's g heads, w_c = mean_h p_c [DA §3.2];
 *   4. routes R = {c < c_p : w_c > 0}, sets their mask bits and the bias
 *        d_c = (log w_c - mu) / sigma,  mu = mean_{c in R} log w_c       [DA Prop. 1]
 *      and always sets the bit of the query's own chunk c_p with d = 0  [DA §3.4; Alg. 2].
 * Mask rows are written in full (bits beyond c_p are 0). Bias entries are written only where the
 * mask bit is 1; the others are left untouched. tau may be NULL; a row with c_p = 0 has no
 * candidate and gets tau = +inf. alpha in (1, 2]; gamma > 0; sigma > 0, +inf allowed (d = 0).
 * bf16 queries with n_q > 1 and Tc <= 1024 run in one pass with the scores on chip; their
 * workspace holds the summaries split into three bf16 terms (6 bytes per summary element, Tc
 * rounded up to a multiple of 32). Other calls (fp32, decode, longer rows) first score into `workspace`, fp32
 * [B, n_q, H_q, Nc]. dash_block_entmax_workspace_bytes() gives the bytes a call needs (0 if
 * none); the workspace may be NULL when it is 0.
 * The workspace holds nothing between calls.
 */
size_t dash_block_entmax_workspace_bytes(dash_dtype_t dt, int batch, int n_q, int q_pos0,
                                         int n_kv, int h_q, int h_kv, int head_dim, int block);
dash_status_t dash_block_entmax(const void* q, dash_dtype_t dt, const float* kbar, int batch,
                                int n_q, int q_pos0, int n_kv, int h_q, int h_kv, int head_dim,
                                int block, float alpha, float gamma, float sigma, uint32_t* mask,
                                float* bias, float* tau, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Stage 1 with two more inputs; dash_block_entmax is this call with ctx_lens = NULL and
 * window_blocks = 1.
 * window_blocks (>= 1) [DA App. B.1.1, the training-time window of the diagonal block and the
 * block before it, 64-127 tokens for Bc = 64]: the query's own chunk and the window_blocks - 1
 * chunks before it are always attended with d = 0 (mask bits set); routing scores only the
 * complete chunks before them, c < c_p - window_blocks + 1. window_blocks = 2 is the pages'
 * window. Chunks before 0 do not exist: a query whose window reaches chunk 0 routes nothing.
 * ctx_lens (device int32 [B], or NULL): decode with a length per sequence, n_q = 1; the query of
 * sequence b sits at p = ctx_lens[b] - 1 (q_pos0 is ignored), n_kv is the cache capacity n_cap
 * (kbar, mask and bias are laid out for it), and only the summaries of the complete chunks
 * below ctx_lens[b] / Bc are read. Lengths outside [1, n_cap] are clamped into it on the device.
 * The workspace is the one of dash_block_entmax with the same sizes.
 */
dash_status_t dash_block_entmax_ex(const void* q, dash_dtype_t dt, const float* kbar,
                                   const int32_t* ctx_lens, int batch, int n_q, int q_pos0,
                                   int n_kv, int h_q, int h_kv, int head_dim, int block,
                                   float alpha, float gamma, float sigma, int window_blocks,
                                   uint32_t* mask, float* bias, float* tau, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Stage 2, prefill [DA §3.3-3.4, Prop. 1; DA App. G, Alg. 3]: for every query t of a causal
 * sequence of n tokens and every head h of group r,
 *   o = sum_j softmax_j(scale * <q_t, k_j> + d_c(j)) v_j
 * over the tokens j of the chunks c < c_t whose mask bit is set (bias d_c from `bias`) and the
 * tokens c_t * Bc .. t of the query's own chunk (d = 0). mask / bias as dash_block_entmax writes
 * them for n_q = n, q_pos0 = 0. scale is normally 1/sqrt(D). lse (natural log of the softmax
 * normaliser, bias included) may be NULL. All query heads of a group share one selection.
 * bf16 with D = 128 needs one sequence's keys to fit 2 GiB (n * H_kv * D * 2 bytes), else
 * DASH_ERR_UNSUPPORTED.
 */
dash_status_t dash_sparse_attn_prefill(const void* q, const void* k, const void* v,
                                       dash_dtype_t dt, const uint32_t* mask, const float* bias,
                                       void* o, float* lse, int batch, int n, int h_q, int h_kv,
                                       int head_dim, int block, float scale, hipStream_t stream);

/*
 * Stage 2 for a block of query rows [DA §3.4 Prop. 1]: as dash_sparse_attn_prefill for the rows
 * at positions q_pos0 .. q_pos0 + n_q - 1 of each sequence of n_kv tokens (0 <= q_pos0,
 * q_pos0 + n_q <= n_kv). q, o [B, n_q, H_q, D], lse [B, n_q, H_q], mask and bias [B, n_q, ...]
 * hold those rows (as dash_block_entmax writes them for the same n_q and q_pos0); k, v
 * [B, n_kv, H_kv, D]. The query at position p attends its routed chunks and the keys of its own
 * chunk up to p. Splitting the rows into blocks gives each row the output of one call over all
 * rows for the same mask and bias: bit for bit for bf16, up to the last bit for fp32 (there the
 * row tiling decides whether an exponent is one fused multiply-add or two), so a caller can route
 * one block while attending the previous one.
 */
dash_status_t dash_sparse_attn_prefill_ex(const void* q, const void* k, const void* v,
                                          dash_dtype_t dt, const uint32_t* mask,
                                          const float* bias, void* o, float* lse, int batch,
                                          int n_q, int q_pos0, int n_kv, int h_q, int h_kv,
                                          int head_dim, int block, float scale,
                                          hipStream_t stream);

/*
 * Stage 2 backward for prefill [DA Prop. 1, differentiated], the selection held fixed: with the
 * forward's lse, p_j = exp(scale <q, k_j> + d_c(j) - lse) over the keys the row attends to,
 * dp_j = <dout, v_j> and ds_j = p_j (dp_j - <dout, o>), where <dout, o> = sum_j p_j dp_j is
 * summed in fp32 from the probabilities (the output o itself is not needed), it writes
 *   dq = scale sum_j ds_j k_j,  dk_j = scale sum ds_j q,  dv_j = sum p_j dout  (over every row
 *   and query head of the group that attends key j), and
 *   dbias[c] = sum of ds_j over chunk c's keys and the group's heads, for the chunks c below the
 *   row's own whose mask bit is set (the gradient of the loss with respect to the routing bias
 *   d_c); every other entry of dbias is 0 (the own chunk, and the window chunks Stage 1 marks
 *   with d = 0, are included as the forward used them).
 *   q, dout [B, n, H_q, D] (dt); k, v [B, n, H_kv, D] (dt); lse [B, n, H_q] fp32 as
 *   dash_sparse_attn_prefill returned it for the same mask and bias.
 *   dq [B, n, H_q, D], dk, dv [B, n, H_kv, D], dbias [B, n, H_kv, Nc]: fp32, fully written
 *   (dbias may be NULL: not computed). workspace: device scratch of
 *   dash_sparse_attn_backward_workspace_bytes(B, n, H_q) bytes (<dout, o> per row and head).
 * Each output element is written by one thread, in a fixed order: the result is deterministic.
 */
size_t dash_sparse_attn_backward_workspace_bytes(int batch, int n, int h_q);
dash_status_t dash_sparse_attn_prefill_backward(
    const void* q, const void* k, const void* v, const float* lse, const void* dout,
    dash_dtype_t dt, const uint32_t* mask, const float* bias, float* dq,
    float* dk, float* dv, float* dbias, int batch, int n, int h_q, int h_kv, int head_dim,
    int block, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Stage 1 and Stage 0 backward for prefill [DA §3.1 Eq. 3, §3.2 Eq. 4, Prop. 1; App. A for the
 * entmax Jacobian], the selection held fixed (each head's support and the routed set R are
 * piecewise constant in the inputs, so no gradient flows through which chunks are selected).
 * From dbias = dL/dd of dash_sparse_attn_prefill_backward it ADDS to dq and dk:
 *   dlogw_c = (dd_c - mean over R of dd) / sigma on R = {c < m : mask bit set} (the routed
 *   chunks; the window's chunks carry the constant d = 0), dw_c = dlogw_c / w_c, each head of the
 *   group receives dp = dw / g, the entmax Jacobian gives dx = u (dp - sum(u dp) / sum(u)) /
 *   (alpha - 1) with u = p^(2 - alpha) on the head's support, and with x = coef <q, kbar>,
 *   coef = (alpha - 1) gamma / sqrt(D):  dq += coef sum_c dx_c kbar_c;  dkbar_c = coef sum over
 *   rows and heads of dx_c q;  dk_j += dkbar_c / Bc for the keys j of each complete chunk c.
 * p and w are recomputed from q, kbar and tau (the forward's threshold); a routed chunk whose
 * recomputed w is 0 contributes nothing.
 *   q [B, n, H_q, D] (dt); kbar [B, Tc, H_kv, D] fp32 from dash_pool_keys (mean pooling);
 *   tau [B, n, H_q], mask [B, n, H_kv, W] from dash_block_entmax(_ex) on the same q, kbar, alpha,
 *   gamma, sigma, window_blocks; dbias [B, n, H_kv, Nc] fp32; dq [B, n, H_q, D] and dk
 *   [B, n, H_kv, D] fp32, read and updated in place. workspace: device scratch of
 *   dash_block_entmax_backward_workspace_bytes(B, n, H_q, H_kv) bytes.
 * Deterministic: every element is updated by one thread in a fixed order.
 */
size_t dash_block_entmax_backward_workspace_bytes(int batch, int n, int h_q, int h_kv);
dash_status_t dash_block_entmax_backward(const void* q, dash_dtype_t dt, const float* kbar,
                                         const float* tau, const uint32_t* mask,
                                         const float* dbias, float* dq, float* dk, int batch,
                                         int n, int h_q, int h_kv, int head_dim, int block,
                                         float alpha, float gamma, float sigma,
                                         int window_blocks, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * dash_block_entmax_backward for learned summary queries [DA §3.1 Eq. 3 and Alg. 1: kbar_c is a
 * softmax-weighted sum of chunk c's keys, a = softmax_j(<qbar_c, k_j> / sqrt(D))]: the same
 * routing gradients, then the pooling's own chain rule. With dkbar_c as above and
 * g_j = <dkbar_c, k_j>, ds_j = a_j (g_j - sum_i a_i g_i) (the softmax Jacobian), it ADDS
 *   dk_j += a_j dkbar_c + ds_j qbar_c / sqrt(D)   to the keys of each complete chunk, and WRITES
 *   dqbar = dL/dqbar: sum over the (sequence, chunk) pairs that use a query of their
 *   sum_j ds_j k_j / sqrt(D), summed in a fixed order (deterministic).
 *   k [B, n, H_kv, D] (dt, q's dtype): the keys kbar was pooled from; kbar [B, Tc, H_kv, D] fp32
 *   from dash_pool_keys_query_ex with the same qbar and strides; qbar fp32, the query of
 *   (sequence b, chunk c, KV head r) at qbar + b * qbar_batch_stride + c * qbar_chunk_stride +
 *   r * D (strides in floats, non-negative multiples of 4: 0, 0 for [H_kv, D]; 0, H_kv D for
 *   [Tc, H_kv, D]; Tc H_kv D, H_kv D for [B, Tc, H_kv, D]); queries of distinct (b, c) pairs may
 *   coincide (a zero stride) but not partly overlap (else DASH_ERR_INVALID). dqbar: fp32 with
 *   qbar's addressing, every query's D floats overwritten. qbar, dqbar 16-byte aligned.
 *   workspace: dash_block_entmax_backward_query_workspace_bytes(B, n, H_q, H_kv, D, block)
 *   bytes, 256-byte aligned. Other arguments as for dash_block_entmax_backward.
 */
size_t dash_block_entmax_backward_query_workspace_bytes(int batch, int n, int h_q, int h_kv,
                                                        int head_dim, int block);
dash_status_t dash_block_entmax_backward_query(
    const void* q, const void* k, dash_dtype_t dt, const float* kbar, const float* qbar,
    int64_t qbar_batch_stride, int64_t qbar_chunk_stride, const float* tau, const uint32_t* mask,
    const float* dbias, float* dq, float* dk, float* dqbar, int batch, int n, int h_q, int h_kv,
    int head_dim, int block, float alpha, float gamma, float sigma, int window_blocks,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Stage 2, decode [DA §3.5, split-KV variant]: the Stage 2 output of one new query per sequence
 * at position n_ctx - 1 of its cache. The selected chunks are split over many workgroups; their
 * partial (max, sum, output) triples are merged in a fixed order by the last of them to finish,
 * so the result is deterministic and the call is one launch.
 *   q, o [B, H_q, D] (dt);  k_cache, v_cache [B, n_ctx, H_kv, D] (dt);
 *   mask [B, 1, H_kv, W], bias [B, 1, H_kv, Nc] from dash_block_entmax(n_q = 1,
 *   q_pos0 = n_ctx - 1).  workspace: device scratch of dash_decode_workspace_bytes() bytes: the
 *   one ticket counter per (sequence, group) (the first ceil(4 B H_kv / 256) * 256 bytes), then the
 *   partial triples; the counters must be zero when a call starts, and every call leaves them
 *   zero. Zero the workspace once when it is allocated. Two calls in flight at once on one
 *   workspace race.
 */
size_t dash_decode_workspace_bytes(int batch, int n_ctx, int h_q, int h_kv, int head_dim,
                                   int block);
dash_status_t dash_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                      dash_dtype_t dt, const uint32_t* mask, const float* bias,
                                      void* o, int batch, int n_ctx, int h_q, int h_kv,
                                      int head_dim, int block, float scale, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * Stage 2, decode with a length per sequence [DA §3.5]: as dash_sparse_attn_decode for a cache
 * of capacity n_cap (the row layout of k_cache, v_cache, mask and bias), the query of sequence b
 * at p = ctx_lens[b] - 1 (device int32 [B], clamped into [1, n_cap]), attending to the selected
 * chunks below its own and to the tokens c_p * Bc .. p of its own chunk. mask / bias as
 * dash_block_entmax_ex writes them with the same ctx_lens. Workspace as
 * dash_decode_workspace_bytes(batch, n_cap, ...).
 */
dash_status_t dash_sparse_attn_decode_varlen(const void* q, const void* k_cache,
                                             const void* v_cache, dash_dtype_t dt,
                                             const int32_t* ctx_lens, const uint32_t* mask,
                                             const float* bias, void* o, int batch, int n_cap,
                                             int h_q, int h_kv, int head_dim, int block,
                                             float scale, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/*
 * One whole decode step [DA §3.2 Alg. 2 and §3.4-3.5, one new query per sequence]: Stage 1
 * routing against the cached summaries and Stage 2 split attention, exactly
 * dash_block_entmax_ex(n_q = 1) followed by dash_sparse_attn_decode(_varlen) with the same
 * arguments, in one call with one workspace (convenient to capture in a graph).
 *   q, o [B, H_q, D] (dt); k_cache, v_cache [B, n_ctx, H_kv, D] (dt); kbar [B, floor(n_ctx / Bc),
 *   H_kv, D] fp32 (the summaries of the complete chunks); ctx_lens: NULL (every query at
 *   n_ctx - 1) or device int32 [B] (query b at ctx_lens[b] - 1, n_ctx the capacity), as
 *   dash_block_entmax_ex; alpha, gamma, sigma, window_blocks as dash_block_entmax_ex; scale as
 *   dash_sparse_attn_decode.
 *   mask [B, 1, H_kv, W], bias [B, 1, H_kv, Nc]: written as dash_block_entmax_ex writes them.
 *   workspace: dash_decode_step_workspace_bytes() bytes: dash_sparse_attn_decode's workspace
 *   (ticket counters first) followed by dash_block_entmax's. The ticket counters must be zero
 *   when a call starts and every call leaves them zero: zero the workspace once when it is
 *   allocated. Two calls in flight at once on one workspace race.
 */
size_t dash_decode_step_workspace_bytes(int batch, int n_ctx, int h_q, int h_kv, int head_dim,
                                        int block);
dash_status_t dash_decode_step(const void* q, const void* k_cache, const void* v_cache,
                               dash_dtype_t dt, const float* kbar, const int32_t* ctx_lens,
                               int batch, int n_ctx, int h_q, int h_kv, int head_dim, int block,
                               float alpha, float gamma, float sigma, int window_blocks,
                               float scale, uint32_t* mask, float* bias, void* o, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * dash_decode_step without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Arguments and
 * outputs as dash_decode_step; the workspace is a scratch array of 32 MiB that the library holds
 * on every GPU it runs on until the process ends. Call it with the stream's device current (the
 * scratch's address on that device is looked up on its first call there and kept). A call whose
 * dash_decode_step_workspace_bytes() exceeds 32 MiB returns DASH_ERR_WORKSPACE and launches
 * nothing (16 sequences of 128K tokens at 32 query / 8 KV heads, D 128, chunk 64 need 13 MiB).
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (other streams,
 * other threads) race, so serialise them. The scratch's ticket counters start at zero and every
 * call leaves them zero. Nothing is allocated or freed, by the library or by HIP on its behalf.
 */
dash_status_t dash_decode_step_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       dash_dtype_t dt, const float* kbar, const int32_t* ctx_lens,
                                       int batch, int n_ctx, int h_q, int h_kv, int head_dim,
                                       int block, float alpha, float gamma, float sigma,
                                       int window_blocks, float scale, uint32_t* mask, float* bias,
                                       void* o, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H */
