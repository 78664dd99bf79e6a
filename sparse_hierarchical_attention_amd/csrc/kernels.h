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
hipError_t launch_pool_query(const void* k, int dt, const float* qbar, float* kbar, int batch,
                             int n_kv, int h_kv, int head_dim, int block, hipStream_t st);

// ---- Stage 1 (block_entmax.hip)
struct RouteParams {
    int batch, n_q, q_pos0, n_kv, h_q, h_kv, g, head_dim, block, tc, nc, nw;
    float alpha, gamma, inv_sigma;
};
size_t route_workspace_bytes(const RouteParams& p, int dt);
bool route_fused_supported(const RouteParams& p, int dt);
size_t route_fused_workspace_bytes(const RouteParams& p);
hipError_t launch_route_fused(const void* q, const float* kbar, uint32_t* mask, float* bias,
                              float* tau, const RouteParams& p, void* ws, hipStream_t st);
hipError_t launch_block_entmax(const void* q, int dt, const float* kbar, const RouteParams& p,
                               uint32_t* mask, float* bias, float* tau, void* ws,
                               hipStream_t st);

// ---- Stage 2 (sparse_attn.hip)
struct AttnParams {
    int batch, n_q, q_pos0, n_kv, h_q, h_kv, g, head_dim, block, nc, nw;
    float scale;
};
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

}  // namespace dash
