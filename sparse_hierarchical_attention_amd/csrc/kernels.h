// Kernel launchers behind the libdash C ABI. Arguments are validated by the caller (api.hip);
// every launcher enqueues on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dash {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// ---- Stage 0 (pool_keys.hip)
hipError_t launch_pool_mean(const void* k, int dt, float* kbar, int batch, int n_kv, int h_kv,
                            int head_dim, int block, hipStream_t st);
// qbar of (sequence b, chunk c, KV head r) at qbar + b sb + c sc + r D (sb = sc = 0: per head)
hipError_t launch_pool_query(const void* k, int dt, const float* qbar, int64_t sb, int64_t sc,
                             float* kbar, int batch, int n_kv, int h_kv, int head_dim, int block,
                             hipStream_t st);
hipError_t launch_pool_append(const void* k, int dt, const float* qbar, int64_t sb, int64_t sc,
                              const int* ctx_lens, float* kbar, int batch, int n_cap, int h_kv,
                              int head_dim, int block, hipStream_t st);

// ---- Stage 1 (block_entmax.hip)
// n_kv, tc = n_kv / block, nc and nw describe the key range (for decode: the cache capacity).
// win: blocks before the query's own that are always attended (the window of W = win + 1
// blocks). ctx_lens (decode only, n_q = 1): per-sequence context lengths, the new token at
// ctx_lens[b] - 1; null when every sequence has n_kv tokens.
struct RouteParams {
    int batch, n_q, q_pos0, n_kv, h_q, h_kv, g, head_dim, block, tc, nc, nw;
    float alpha, gamma, inv_sigma;
    int win;
    const int* ctx_lens;
};
size_t route_workspace_bytes(const RouteParams& p, int dt);
bool route_fused_supported(const RouteParams& p, int dt);
size_t route_fused_workspace_bytes(const RouteParams& p);
hipError_t launch_route_fused(const void* q, const float* kbar, uint32_t* mask, float* bias,
                              float* tau, const RouteParams& p, void* ws, hipStream_t st);
hipError_t launch_block_entmax(const void* q, int dt, const float* kbar, const RouteParams& p,
                               uint32_t* mask, float* bias, float* tau, void* ws,
                               hipStream_t st);
hipError_t launch_score_one(const void* q, int dt, const float* kbar, float* x,
                            const RouteParams& p, hipStream_t st);
// Stage 0 of the backward: qbar == nullptr for mean pooling; otherwise learned summary queries,
// the query of (sequence b, chunk c, KV head r) at qbar + b sb + c sc + r D, its gradient written
// at dqbar + b sb + c sc + r D (summed over the (b, c) that share it: sb = 0 or sc = 0)
struct PoolGrad {
    const void* k;  // [B, n, Hkv, D], q's dtype
    const float* qbar;
    int64_t sb, sc;
    float* dqbar;
};
// with_query: room for each chunk's dqbar before the sum over shared queries
size_t route_backward_workspace_bytes(const RouteParams& p, bool with_query);
hipError_t launch_route_backward(const void* q, int dt, const float* kbar, const float* tau,
                                 const uint32_t* mask, const float* dbias, float* dq, float* dk,
                                 const PoolGrad& pg, const RouteParams& p, void* ws,
                                 hipStream_t st);


// ---- Stage 2 (sparse_attn.hip)
struct AttnParams {
    int batch, n_q, q_pos0, n_kv, h_q, h_kv, g, head_dim, block, nc, nw;
    float scale;
    const int* ctx_lens;  // decode only: per-sequence context lengths (null: n_kv for all)
};

// Token position of query t of sequence b. A per-sequence length is clamped into [1, cap].
__device__ __forceinline__ int seq_pos(const int* ctx_lens, int q_pos0, int cap, int b, int t) {
    return ctx_lens ? min(max(ctx_lens[b], 1), cap) - 1 : q_pos0 + t;
}
__device__ __forceinline__ int route_pos(const RouteParams& p, int b, int t) {
    return seq_pos(p.ctx_lens, p.q_pos0, p.n_kv, b, t);
}
// Routing candidates of the query at pos: the complete chunks before its window, c < m. The
// window is chunks m .. pos / block (the query's own chunk and the win before it).
__device__ __forceinline__ int route_cands(const RouteParams& p, int pos) {
    return max(0, min(pos / p.block - p.win, p.tc));
}
// Bits of chunks lo .. hi (inclusive) that fall into mask word wd.
__device__ __forceinline__ uint32_t span_bits(int wd, int lo, int hi) {
    const int a = max(lo, 32 * wd), z = min(hi, 32 * wd + 31);
    if (a > z) return 0u;
    const int n = z - a + 1;
    return (n == 32 ? ~0u : ((1u << n) - 1u)) << (a - 32 * wd);
}
hipError_t launch_attn_prefill(const void* q, const void* k, const void* v, int dt,
                               const uint32_t* mask, const float* bias, void* o, float* lse,
                               const AttnParams& p, hipStream_t st);
hipError_t launch_attn_prefill_mfma(const void* q, const void* k, const void* v,
                                   const uint32_t* mask, const float* bias, void* o, float* lse,
                                   const AttnParams& p, hipStream_t st);
hipError_t launch_attn_prefill_dma(const void* q, const void* k, const void* v,
                                  const uint32_t* mask, const float* bias, void* o, float* lse,
                                  const AttnParams& p, hipStream_t st);
size_t decode_workspace_bytes(const AttnParams& p);
hipError_t launch_attn_decode(const void* q, const void* k, const void* v, int dt,
                              const uint32_t* mask, const float* bias, void* o,
                              const AttnParams& p, void* ws, hipStream_t st);
// the decode step (dash_decode_step): scores, then routing and attention in one kernel
size_t decode_step_workspace_bytes(const RouteParams& rp, const AttnParams& p);
hipError_t launch_decode_step(const void* q, const void* k, const void* v, int dt,
                              const float* kbar, const RouteParams& rp, const AttnParams& p,
                              uint32_t* mask, float* bias, void* o, void* ws, hipStream_t st);
size_t attn_backward_workspace_bytes(const AttnParams& p);
hipError_t launch_attn_backward_mfma(const void* q, const void* k, const void* v,
                                     const float* lse, const void* dout, const uint32_t* mask,
                                     const float* bias, float* dq, float* dk, float* dv,
                                     float* dbias, const AttnParams& p, void* ws, hipStream_t st);
hipError_t launch_attn_backward(const void* q, const void* k, const void* v, const float* lse,
                                const void* dout, int dt, const uint32_t* mask,
                                const float* bias, float* dq, float* dk, float* dv, float* dbias,
                                const AttnParams& p, void* ws, hipStream_t st);

}  // namespace dash
