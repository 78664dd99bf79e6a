// libdash C ABI: argument validation, dispatch and launch (see include/dash.h).
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>

#include "dash.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

dash_status_t fail(dash_status_t s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

dash_status_t ok() {
    g_last_error.clear();
    return DASH_OK;
}

dash_status_t hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return ok();
    return fail(DASH_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr int kMaxChunks = 8192;

// Shape checks shared by every entry point. Returns DASH_OK or the failing status.
dash_status_t check_shape(const char* fn, dash_dtype_t dt, int batch, int n_kv, int h_q, int h_kv,
                          int head_dim, int block) {
    if (dt != DASH_F32 && dt != DASH_BF16) return fail(DASH_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dt);
    if (batch <= 0 || n_kv <= 0 || h_q <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0)
        return fail(DASH_ERR_INVALID, "%s: sizes must be positive (batch=%d n=%d h_q=%d h_kv=%d D=%d block=%d)",
                    fn, batch, n_kv, h_q, h_kv, head_dim, block);
    if (h_q % h_kv != 0)
        return fail(DASH_ERR_INVALID, "%s: h_q=%d is not a multiple of h_kv=%d", fn, h_q, h_kv);
    const int g = h_q / h_kv;
    if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
        return fail(DASH_ERR_UNSUPPORTED, "%s: group size h_q/h_kv=%d not in {1,2,4,8,16}", fn, g);
    if (head_dim != 64 && head_dim != 128)
        return fail(DASH_ERR_UNSUPPORTED, "%s: head_dim=%d not in {64,128}", fn, head_dim);
    if (block != 32 && block != 64 && block != 128)
        return fail(DASH_ERR_UNSUPPORTED, "%s: block=%d not in {32,64,128}", fn, block);
    if (ceil_div(n_kv, block) > kMaxChunks)
        return fail(DASH_ERR_UNSUPPORTED, "%s: %d chunks exceed the limit %d", fn, ceil_div(n_kv, block), kMaxChunks);
    if ((int64_t)batch * n_kv > (int64_t)1 << 31)
        return fail(DASH_ERR_UNSUPPORTED, "%s: batch * n too large", fn);
    return DASH_OK;
}

dash::RouteParams route_params(int batch, int n_q, int q_pos0, int n_kv, int h_q, int h_kv,
                               int head_dim, int block, float alpha, float gamma, float sigma) {
    dash::RouteParams p;
    p.batch = batch; p.n_q = n_q; p.q_pos0 = q_pos0; p.n_kv = n_kv; p.h_q = h_q; p.h_kv = h_kv;
    p.g = h_q / h_kv; p.head_dim = head_dim; p.block = block; p.tc = n_kv / block;
    p.nc = ceil_div(n_kv, block); p.nw = ceil_div(p.nc, 32);
    p.alpha = alpha; p.gamma = gamma; p.inv_sigma = isinf(sigma) ? 0.0f : 1.0f / sigma;
    p.win = 0; p.ctx_lens = nullptr;
    return p;
}

dash::AttnParams attn_params(int batch, int n_q, int q_pos0, int n_kv, int h_q, int h_kv,
                             int head_dim, int block, float scale) {
    dash::AttnParams p;
    p.batch = batch; p.n_q = n_q; p.q_pos0 = q_pos0; p.n_kv = n_kv; p.h_q = h_q; p.h_kv = h_kv;
    p.g = h_q / h_kv; p.head_dim = head_dim; p.block = block;
    p.nc = ceil_div(n_kv, block); p.nw = ceil_div(p.nc, 32); p.scale = scale;
    p.ctx_lens = nullptr;
    return p;
}

// the shared bodies of the entry points with and without per-sequence lengths (defined below)
// Stage 2 prefill over rows q_pos0 .. q_pos0 + n_q - 1 of each sequence (all rows: 0, n_kv).
dash_status_t prefill_call(const char* fn, const void* q, const void* k, const void* v,
                           dash_dtype_t dt, const uint32_t* mask, const float* bias, void* o,
                           float* lse, int batch, int n_q, int q_pos0, int n_kv, int h_q,
                           int h_kv, int head_dim, int block, float scale, hipStream_t stream) {
    dash_status_t s = check_shape(fn, dt, batch, n_kv, h_q, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    if (n_q <= 0 || q_pos0 < 0 || (int64_t)q_pos0 + n_q > n_kv)
        return fail(DASH_ERR_INVALID, "%s: need n_q > 0 and 0 <= q_pos0, q_pos0 + n_q <= n_kv (n_q=%d q_pos0=%d n_kv=%d)",
                    fn, n_q, q_pos0, n_kv);
    if (!(scale > 0.0f) || isinf(scale)) return fail(DASH_ERR_INVALID, "%s: scale=%g must be positive and finite", fn, scale);
    if (!q || !k || !v || !mask || !bias || !o) return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    // bf16 head dim 128 addresses one sequence's keys (and values) with 32-bit byte offsets
    if (dt == DASH_BF16 && head_dim == 128 && (int64_t)n_kv * h_kv * head_dim * 2 > INT32_MAX)
        return fail(DASH_ERR_UNSUPPORTED, "%s: one sequence's keys (n * h_kv * head_dim bf16) exceed 2 GiB", fn);
    dash::AttnParams p = attn_params(batch, n_q, q_pos0, n_kv, h_q, h_kv, head_dim, block, scale);
    return hip_status(dash::launch_attn_prefill(q, k, v, dt, mask, bias, o, lse, p, stream), fn);
}

dash_status_t route_call(const char* fn, const void* q, dash_dtype_t dt, const float* kbar,
                         const int32_t* ctx_lens, int batch, int n_q, int q_pos0, int n_kv,
                         int h_q, int h_kv, int head_dim, int block, float alpha, float gamma,
                         float sigma, int window_blocks, uint32_t* mask, float* bias, float* tau,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);
dash_status_t decode_call(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                          dash_dtype_t dt, const int32_t* ctx_lens, const uint32_t* mask,
                          const float* bias, void* o, int batch, int n_ctx, int h_q, int h_kv,
                          int head_dim, int block, float scale, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);
dash_status_t decode_step_call(const char* fn, const void* q, const void* k_cache,
                               const void* v_cache, dash_dtype_t dt, const float* kbar,
                               const int32_t* ctx_lens, int batch, int n_ctx, int h_q, int h_kv,
                               int head_dim, int block, float alpha, float gamma, float sigma,
                               int window_blocks, float scale, uint32_t* mask, float* bias,
                               void* o, void* workspace, size_t workspace_bytes, bool use_scratch,
                               hipStream_t stream);

}  // namespace

extern "C" {

const char* dash_status_string(dash_status_t s) {
    switch (s) {
        case DASH_OK: return "DASH_OK";
        case DASH_ERR_INVALID: return "DASH_ERR_INVALID";
        case DASH_ERR_UNSUPPORTED: return "DASH_ERR_UNSUPPORTED";
        case DASH_ERR_WORKSPACE: return "DASH_ERR_WORKSPACE";
        case DASH_ERR_HIP: return "DASH_ERR_HIP";
    }
    return "DASH_UNKNOWN_STATUS";
}

const char* dash_last_error(void) { return g_last_error.c_str(); }

int dash_version(void) { return 100; }

dash_status_t dash_pool_keys(const void* k, dash_dtype_t dt, float* kbar, int batch, int n_kv,
                             int h_kv, int head_dim, int block, hipStream_t stream) {
    dash_status_t s = check_shape("dash_pool_keys", dt, batch, n_kv, h_kv, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    // with no complete chunk (n_kv < block) there is nothing to write and kbar may be null
    if (!k || (!kbar && n_kv / block > 0)) return fail(DASH_ERR_INVALID, "dash_pool_keys: null pointer");
    return hip_status(dash::launch_pool_mean(k, dt, kbar, batch, n_kv, h_kv, head_dim, block, stream),
                      "dash_pool_keys");
}

dash_status_t dash_pool_keys_query_ex(const void* k, dash_dtype_t dt, const float* qbar,
                                      int64_t qbar_batch_stride, int64_t qbar_chunk_stride,
                                      float* kbar, int batch, int n_kv, int h_kv, int head_dim,
                                      int block, hipStream_t stream) {
    const char* fn = "dash_pool_keys_query_ex";
    dash_status_t s = check_shape(fn, dt, batch, n_kv, h_kv, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    if (!k || !qbar || (!kbar && n_kv / block > 0)) return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    if (qbar_batch_stride < 0 || qbar_chunk_stride < 0 || qbar_batch_stride % 4 || qbar_chunk_stride % 4)
        return fail(DASH_ERR_INVALID, "%s: qbar strides must be non-negative multiples of 4 (%lld, %lld)",
                    fn, (long long)qbar_batch_stride, (long long)qbar_chunk_stride);
    return hip_status(dash::launch_pool_query(k, dt, qbar, qbar_batch_stride, qbar_chunk_stride, kbar,
                                              batch, n_kv, h_kv, head_dim, block, stream), fn);
}

dash_status_t dash_pool_keys_query(const void* k, dash_dtype_t dt, const float* qbar, float* kbar,
                                   int batch, int n_kv, int h_kv, int head_dim, int block,
                                   hipStream_t stream) {
    const dash_status_t s = dash_pool_keys_query_ex(k, dt, qbar, 0, 0, kbar, batch, n_kv, h_kv,
                                                    head_dim, block, stream);
    if (s != DASH_OK) g_last_error.replace(0, strlen("dash_pool_keys_query_ex"), "dash_pool_keys_query");
    return s;
}

dash_status_t dash_pool_keys_append_ex(const void* k_cache, dash_dtype_t dt, const float* qbar,
                                       int64_t qbar_batch_stride, int64_t qbar_chunk_stride,
                                       const int32_t* ctx_lens, float* kbar, int batch, int n_cap,
                                       int h_kv, int head_dim, int block, hipStream_t stream) {
    const char* fn = "dash_pool_keys_append_ex";
    dash_status_t s = check_shape(fn, dt, batch, n_cap, h_kv, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    if (!k_cache || !ctx_lens || (!kbar && n_cap / block > 0)) return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    if (qbar_batch_stride < 0 || qbar_chunk_stride < 0 || qbar_batch_stride % 4 || qbar_chunk_stride % 4)
        return fail(DASH_ERR_INVALID, "%s: qbar strides must be non-negative multiples of 4 (%lld, %lld)",
                    fn, (long long)qbar_batch_stride, (long long)qbar_chunk_stride);
    return hip_status(dash::launch_pool_append(k_cache, dt, qbar, qbar_batch_stride, qbar_chunk_stride,
                                               ctx_lens, kbar, batch, n_cap, h_kv, head_dim, block,
                                               stream), fn);
}

dash_status_t dash_pool_keys_append(const void* k_cache, dash_dtype_t dt, const float* qbar,
                                    const int32_t* ctx_lens, float* kbar, int batch, int n_cap,
                                    int h_kv, int head_dim, int block, hipStream_t stream) {
    const dash_status_t s = dash_pool_keys_append_ex(k_cache, dt, qbar, 0, 0, ctx_lens, kbar, batch,
                                                     n_cap, h_kv, head_dim, block, stream);
    if (s != DASH_OK) g_last_error.replace(0, strlen("dash_pool_keys_append_ex"), "dash_pool_keys_append");
    return s;
}

size_t dash_block_entmax_workspace_bytes(dash_dtype_t dt, int batch, int n_q, int q_pos0,
                                         int n_kv, int h_q, int h_kv, int head_dim, int block) {
    if (batch <= 0 || n_q <= 0 || n_kv <= 0 || h_q <= 0 || h_kv <= 0 || block <= 0 || h_q % h_kv)
        return 0;
    return dash::route_workspace_bytes(route_params(batch, n_q, q_pos0, n_kv, h_q, h_kv, head_dim,
                                                    block, 1.5f, 1.0f, 1.0f), (int)dt);
}

dash_status_t dash_block_entmax(const void* q, dash_dtype_t dt, const float* kbar, int batch,
                                int n_q, int q_pos0, int n_kv, int h_q, int h_kv, int head_dim,
                                int block, float alpha, float gamma, float sigma, uint32_t* mask,
                                float* bias, float* tau, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    return route_call("dash_block_entmax", q, dt, kbar, nullptr, batch, n_q, q_pos0, n_kv, h_q,
                      h_kv, head_dim, block, alpha, gamma, sigma, 1, mask, bias, tau, workspace,
                      workspace_bytes, stream);
}

dash_status_t dash_block_entmax_ex(const void* q, dash_dtype_t dt, const float* kbar,
                                   const int32_t* ctx_lens, int batch, int n_q, int q_pos0,
                                   int n_kv, int h_q, int h_kv, int head_dim, int block,
                                   float alpha, float gamma, float sigma, int window_blocks,
                                   uint32_t* mask, float* bias, float* tau, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    return route_call("dash_block_entmax_ex", q, dt, kbar, ctx_lens, batch, n_q, q_pos0, n_kv,
                      h_q, h_kv, head_dim, block, alpha, gamma, sigma, window_blocks, mask, bias,
                      tau, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

dash_status_t route_call(const char* fn, const void* q, dash_dtype_t dt, const float* kbar,
                         const int32_t* ctx_lens, int batch, int n_q, int q_pos0, int n_kv,
                         int h_q, int h_kv, int head_dim, int block, float alpha, float gamma,
                         float sigma, int window_blocks, uint32_t* mask, float* bias, float* tau,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    dash_status_t s = check_shape(fn, dt, batch, n_kv, h_q, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    if (ctx_lens) {
        if (n_q != 1) return fail(DASH_ERR_INVALID, "%s: per-sequence lengths need n_q = 1 (n_q=%d)", fn, n_q);
        q_pos0 = n_kv - 1;  // unused on the device; keeps the range check below meaningful
    }
    if (window_blocks < 1) return fail(DASH_ERR_INVALID, "%s: window_blocks=%d must be >= 1", fn, window_blocks);
    if (n_q <= 0 || q_pos0 < 0 || (int64_t)q_pos0 + n_q > n_kv)
        return fail(DASH_ERR_INVALID, "%s: need n_q > 0 and 0 <= q_pos0, q_pos0 + n_q <= n_kv (n_q=%d q_pos0=%d n_kv=%d)",
                    fn, n_q, q_pos0, n_kv);
    if (!(alpha > 1.0f && alpha <= 2.0f)) return fail(DASH_ERR_INVALID, "%s: alpha=%g not in (1, 2]", fn, alpha);
    if (!(gamma > 0.0f) || isinf(gamma)) return fail(DASH_ERR_INVALID, "%s: gamma=%g must be positive and finite", fn, gamma);
    if (!(sigma > 0.0f)) return fail(DASH_ERR_INVALID, "%s: sigma=%g must be positive (or +inf)", fn, sigma);
    if (!q || (!kbar && n_kv / block > 0) || !mask || !bias)
        return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    dash::RouteParams p = route_params(batch, n_q, q_pos0, n_kv, h_q, h_kv, head_dim, block, alpha,
                                       gamma, sigma);
    p.win = window_blocks - 1;
    p.ctx_lens = ctx_lens;
    const size_t need = dash::route_workspace_bytes(p, (int)dt);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DASH_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return hip_status(dash::launch_block_entmax(q, dt, kbar, p, mask, bias, tau, workspace, stream), fn);
}

}  // namespace

extern "C" {

dash_status_t dash_sparse_attn_prefill_ex(const void* q, const void* k, const void* v,
                                          dash_dtype_t dt, const uint32_t* mask,
                                          const float* bias, void* o, float* lse, int batch,
                                          int n_q, int q_pos0, int n_kv, int h_q, int h_kv,
                                          int head_dim, int block, float scale,
                                          hipStream_t stream) {
    return prefill_call("dash_sparse_attn_prefill_ex", q, k, v, dt, mask, bias, o, lse, batch, n_q,
                        q_pos0, n_kv, h_q, h_kv, head_dim, block, scale, stream);
}

dash_status_t dash_sparse_attn_prefill(const void* q, const void* k, const void* v,
                                       dash_dtype_t dt, const uint32_t* mask, const float* bias,
                                       void* o, float* lse, int batch, int n, int h_q, int h_kv,
                                       int head_dim, int block, float scale, hipStream_t stream) {
    return prefill_call("dash_sparse_attn_prefill", q, k, v, dt, mask, bias, o, lse, batch, n, 0, n,
                        h_q, h_kv, head_dim, block, scale, stream);
}

size_t dash_sparse_attn_backward_workspace_bytes(int batch, int n, int h_q) {
    if (batch <= 0 || n <= 0 || h_q <= 0) return 0;
    return (size_t)batch * n * h_q * sizeof(float);
}

dash_status_t dash_sparse_attn_prefill_backward(
    const void* q, const void* k, const void* v, const float* lse, const void* dout,
    dash_dtype_t dt, const uint32_t* mask, const float* bias, float* dq,
    float* dk, float* dv, float* dbias, int batch, int n, int h_q, int h_kv, int head_dim,
    int block, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* fn = "dash_sparse_attn_prefill_backward";
    dash_status_t s = check_shape(fn, dt, batch, n, h_q, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    if (!(scale > 0.0f) || isinf(scale)) return fail(DASH_ERR_INVALID, "%s: scale=%g must be positive and finite", fn, scale);
    if (!q || !k || !v || !lse || !dout || !mask || !bias || !dq || !dk || !dv)
        return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    dash::AttnParams p = attn_params(batch, n, 0, n, h_q, h_kv, head_dim, block, scale);
    const size_t need = dash::attn_backward_workspace_bytes(p);
    if (!workspace || workspace_bytes < need)
        return fail(DASH_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return hip_status(dash::launch_attn_backward(q, k, v, lse, dout, dt, mask, bias, dq, dk, dv,
                                                 dbias, p, workspace, stream), fn);
}

size_t dash_block_entmax_backward_workspace_bytes(int batch, int n, int h_q, int h_kv) {
    if (batch <= 0 || n <= 0 || h_q <= 0 || h_kv <= 0) return 0;
    return (size_t)batch * n * (h_q + h_kv) * sizeof(float);
}

size_t dash_block_entmax_backward_query_workspace_bytes(int batch, int n, int h_q, int h_kv,
                                                        int head_dim, int block) {
    if (batch <= 0 || n <= 0 || h_q <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0) return 0;
    dash::RouteParams p{};
    p.batch = batch;
    p.n_q = n;
    p.h_q = h_q;
    p.h_kv = h_kv;
    p.head_dim = head_dim;
    p.tc = n / block;
    return dash::route_backward_workspace_bytes(p, true);
}

namespace {

dash_status_t route_backward_call(const char* fn, const void* q, dash_dtype_t dt,
                                  const float* kbar, const dash::PoolGrad& pg, const float* tau,
                                  const uint32_t* mask, const float* dbias, float* dq, float* dk,
                                  int batch, int n, int h_q, int h_kv, int head_dim, int block,
                                  float alpha, float gamma, float sigma, int window_blocks,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    dash_status_t s = check_shape(fn, dt, batch, n, h_q, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    if (window_blocks < 1) return fail(DASH_ERR_INVALID, "%s: window_blocks=%d must be >= 1", fn, window_blocks);
    if (!(alpha > 1.0f && alpha <= 2.0f)) return fail(DASH_ERR_INVALID, "%s: alpha=%g not in (1, 2]", fn, alpha);
    if (!(gamma > 0.0f) || isinf(gamma)) return fail(DASH_ERR_INVALID, "%s: gamma=%g must be positive and finite", fn, gamma);
    if (!(sigma > 0.0f)) return fail(DASH_ERR_INVALID, "%s: sigma=%g must be positive (or +inf)", fn, sigma);
    if (!q || (!kbar && n / block > 0) || !tau || !mask || !dbias || !dq || !dk)
        return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    dash::RouteParams p = route_params(batch, n, 0, n, h_q, h_kv, head_dim, block, alpha, gamma,
                                       sigma);
    p.win = window_blocks - 1;
    const size_t need = dash::route_backward_workspace_bytes(p, pg.qbar != nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(DASH_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (pg.qbar && ((uintptr_t)workspace & 255))
        return fail(DASH_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
    return hip_status(dash::launch_route_backward(q, (int)dt, kbar, tau, mask, dbias, dq, dk, pg,
                                                  p, workspace, stream), fn);
}

}  // namespace

dash_status_t dash_block_entmax_backward(const void* q, dash_dtype_t dt, const float* kbar,
                                         const float* tau, const uint32_t* mask,
                                         const float* dbias, float* dq, float* dk, int batch,
                                         int n, int h_q, int h_kv, int head_dim, int block,
                                         float alpha, float gamma, float sigma,
                                         int window_blocks, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    const dash::PoolGrad pg{nullptr, nullptr, 0, 0, nullptr};
    return route_backward_call("dash_block_entmax_backward", q, dt, kbar, pg, tau, mask, dbias,
                               dq, dk, batch, n, h_q, h_kv, head_dim, block, alpha, gamma, sigma,
                               window_blocks, workspace, workspace_bytes, stream);
}

dash_status_t dash_block_entmax_backward_query(
    const void* q, const void* k, dash_dtype_t dt, const float* kbar, const float* qbar,
    int64_t qbar_batch_stride, int64_t qbar_chunk_stride, const float* tau, const uint32_t* mask,
    const float* dbias, float* dq, float* dk, float* dqbar, int batch, int n, int h_q, int h_kv,
    int head_dim, int block, float alpha, float gamma, float sigma, int window_blocks,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* fn = "dash_block_entmax_backward_query";
    if (!k || !qbar || !dqbar) return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    const int64_t sb = qbar_batch_stride, sc = qbar_chunk_stride;
    if (sb < 0 || sc < 0 || sb % 4 || sc % 4)
        return fail(DASH_ERR_INVALID, "%s: qbar strides must be non-negative multiples of 4 (%lld, %lld)",
                    fn, (long long)sb, (long long)sc);
    if (((uintptr_t)qbar & 15) || ((uintptr_t)dqbar & 15))
        return fail(DASH_ERR_INVALID, "%s: qbar and dqbar must be 16-byte aligned", fn);
    // dqbar rows of distinct (sequence, chunk) pairs must not overlap unless they share the query
    if (head_dim > 0 && block > 0 && batch > 0) {
        const int64_t row = (int64_t)h_kv * head_dim, tc = n / block;
        const int64_t eb = batch > 1 ? sb : 0, ec = tc > 1 ? sc : 0;
        const bool ok = (eb == 0 || eb >= row) && (ec == 0 || ec >= row) &&
                        (eb == 0 || ec == 0 || eb >= tc * ec || ec >= (int64_t)batch * eb);
        if (!ok)
            return fail(DASH_ERR_INVALID, "%s: qbar strides (%lld, %lld) make distinct chunks' queries overlap",
                        fn, (long long)sb, (long long)sc);
    }
    const dash::PoolGrad pg{k, qbar, sb, sc, dqbar};
    return route_backward_call(fn, q, dt, kbar, pg, tau, mask, dbias, dq, dk, batch, n, h_q, h_kv,
                               head_dim, block, alpha, gamma, sigma, window_blocks, workspace,
                               workspace_bytes, stream);
}

size_t dash_decode_workspace_bytes(int batch, int n_ctx, int h_q, int h_kv, int head_dim,
                                   int block) {
    if (batch <= 0 || n_ctx <= 0 || h_q <= 0 || h_kv <= 0 || block <= 0 || h_q % h_kv) return 0;
    return dash::decode_workspace_bytes(attn_params(batch, 1, n_ctx - 1, n_ctx, h_q, h_kv, head_dim,
                                                    block, 1.0f));
}

dash_status_t dash_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                      dash_dtype_t dt, const uint32_t* mask, const float* bias,
                                      void* o, int batch, int n_ctx, int h_q, int h_kv,
                                      int head_dim, int block, float scale, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return decode_call("dash_sparse_attn_decode", q, k_cache, v_cache, dt, nullptr, mask, bias, o,
                       batch, n_ctx, h_q, h_kv, head_dim, block, scale, workspace, workspace_bytes,
                       stream);
}

dash_status_t dash_sparse_attn_decode_varlen(const void* q, const void* k_cache,
                                             const void* v_cache, dash_dtype_t dt,
                                             const int32_t* ctx_lens, const uint32_t* mask,
                                             const float* bias, void* o, int batch, int n_cap,
                                             int h_q, int h_kv, int head_dim, int block,
                                             float scale, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
    if (!ctx_lens) return fail(DASH_ERR_INVALID, "dash_sparse_attn_decode_varlen: null pointer");
    return decode_call("dash_sparse_attn_decode_varlen", q, k_cache, v_cache, dt, ctx_lens, mask,
                       bias, o, batch, n_cap, h_q, h_kv, head_dim, block, scale, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"

namespace {

dash_status_t decode_call(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                          dash_dtype_t dt, const int32_t* ctx_lens, const uint32_t* mask,
                          const float* bias, void* o, int batch, int n_ctx, int h_q, int h_kv,
                          int head_dim, int block, float scale, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    dash_status_t s = check_shape(fn, dt, batch, n_ctx, h_q, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    if (!(scale > 0.0f) || isinf(scale)) return fail(DASH_ERR_INVALID, "%s: scale=%g must be positive and finite", fn, scale);
    if (!q || !k_cache || !v_cache || !mask || !bias || !o) return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    dash::AttnParams p = attn_params(batch, 1, n_ctx - 1, n_ctx, h_q, h_kv, head_dim, block, scale);
    p.ctx_lens = ctx_lens;
    const size_t need = dash::decode_workspace_bytes(p);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DASH_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return hip_status(dash::launch_attn_decode(q, k_cache, v_cache, dt, mask, bias, o, p, workspace, stream), fn);
}

}  // namespace

extern "C" {

size_t dash_decode_step_workspace_bytes(int batch, int n_ctx, int h_q, int h_kv, int head_dim,
                                        int block) {
    if (batch <= 0 || n_ctx <= 0 || h_q <= 0 || h_kv <= 0 || block <= 0 || h_q % h_kv) return 0;
    const dash::RouteParams rp = route_params(batch, 1, n_ctx - 1, n_ctx, h_q, h_kv, head_dim,
                                              block, 1.5f, 1.0f, 1.0f);
    const dash::AttnParams p = attn_params(batch, 1, n_ctx - 1, n_ctx, h_q, h_kv, head_dim, block, 1.0f);
    return dash::decode_step_workspace_bytes(rp, p);
}

dash_status_t dash_decode_step(const void* q, const void* k_cache, const void* v_cache,
                               dash_dtype_t dt, const float* kbar, const int32_t* ctx_lens,
                               int batch, int n_ctx, int h_q, int h_kv, int head_dim, int block,
                               float alpha, float gamma, float sigma, int window_blocks,
                               float scale, uint32_t* mask, float* bias, void* o, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    return decode_step_call("dash_decode_step", q, k_cache, v_cache, dt, kbar, ctx_lens, batch,
                            n_ctx, h_q, h_kv, head_dim, block, alpha, gamma, sigma, window_blocks,
                            scale, mask, bias, o, workspace, workspace_bytes, false, stream);
}

}  // extern "C"

namespace {

// Scratch of dash_decode_step_noalloc: one copy on every GPU the library runs on, held until the
// process ends. Its address on the current device is looked up once per device and kept; kernels
// get that address, never the array's host-side name. Zero at load, so its ticket counters start
// at zero, and every call leaves them zero.
constexpr size_t kScratchBytes = (size_t)32 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// the scratch's device address on the current device, or nullptr (with the error recorded)
void* scratch_address(const char* fn) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fail(DASH_ERR_HIP, "%s: no current device", fn);
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(DASH_ERR_HIP, "%s: scratch address: %s", fn, hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

dash_status_t decode_step_call(const char* fn, const void* q, const void* k_cache,
                               const void* v_cache, dash_dtype_t dt, const float* kbar,
                               const int32_t* ctx_lens, int batch, int n_ctx, int h_q, int h_kv,
                               int head_dim, int block, float alpha, float gamma, float sigma,
                               int window_blocks, float scale, uint32_t* mask, float* bias,
                               void* o, void* workspace, size_t workspace_bytes, bool use_scratch,
                               hipStream_t stream) {
    dash_status_t s = check_shape(fn, dt, batch, n_ctx, h_q, h_kv, head_dim, block);
    if (s != DASH_OK) return s;
    if (window_blocks < 1) return fail(DASH_ERR_INVALID, "%s: window_blocks=%d must be >= 1", fn, window_blocks);
    if (!(alpha > 1.0f && alpha <= 2.0f)) return fail(DASH_ERR_INVALID, "%s: alpha=%g not in (1, 2]", fn, alpha);
    if (!(gamma > 0.0f) || isinf(gamma)) return fail(DASH_ERR_INVALID, "%s: gamma=%g must be positive and finite", fn, gamma);
    if (!(sigma > 0.0f)) return fail(DASH_ERR_INVALID, "%s: sigma=%g must be positive (or +inf)", fn, sigma);
    if (!(scale > 0.0f) || isinf(scale)) return fail(DASH_ERR_INVALID, "%s: scale=%g must be positive and finite", fn, scale);
    if (!q || !k_cache || !v_cache || (!kbar && n_ctx / block > 0) || !mask || !bias || !o)
        return fail(DASH_ERR_INVALID, "%s: null pointer", fn);
    dash::RouteParams rp = route_params(batch, 1, n_ctx - 1, n_ctx, h_q, h_kv, head_dim, block,
                                        alpha, gamma, sigma);
    rp.win = window_blocks - 1;
    rp.ctx_lens = ctx_lens;
    dash::AttnParams p = attn_params(batch, 1, n_ctx - 1, n_ctx, h_q, h_kv, head_dim, block, scale);
    p.ctx_lens = ctx_lens;
    const size_t need = dash::decode_step_workspace_bytes(rp, p);
    if (use_scratch) {
        if (need > kScratchBytes)
            return fail(DASH_ERR_WORKSPACE, "%s: the call needs %zu bytes of scratch, more than the "
                        "%zu the library holds per device", fn, need, kScratchBytes);
        workspace = scratch_address(fn);
        if (!workspace) return DASH_ERR_HIP;
        workspace_bytes = kScratchBytes;
    }
    if (!workspace || workspace_bytes < need)
        return fail(DASH_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return hip_status(dash::launch_decode_step(q, k_cache, v_cache, (int)dt, kbar, rp, p, mask,
                                               bias, o, workspace, stream), fn);
}

}  // namespace

extern "C" {

dash_status_t dash_decode_step_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       dash_dtype_t dt, const float* kbar, const int32_t* ctx_lens,
                                       int batch, int n_ctx, int h_q, int h_kv, int head_dim,
                                       int block, float alpha, float gamma, float sigma,
                                       int window_blocks, float scale, uint32_t* mask, float* bias,
                                       void* o, hipStream_t stream) {
    return decode_step_call("dash_decode_step_noalloc", q, k_cache, v_cache, dt, kbar, ctx_lens,
                            batch, n_ctx, h_q, h_kv, head_dim, block, alpha, gamma, sigma,
                            window_blocks, scale, mask, bias, o, nullptr, 0, true, stream);
}

}  // extern "C"
