// Stage 0: chunk summaries ("DashAttention", arXiv 2605.18753v1, §3.1 Eq. 3; App. G Alg. 1).
//
// Mean pooling is a pure HBM stream: a chunk of one sequence is Bc consecutive token rows, each
// holding H_kv * D contiguous elements, so the chunk is one contiguous slab of Bc * H_kv * D
// elements. A workgroup of 4 waves owns one (sequence, chunk, 512-column slab); lane l of wave w
// owns 8 consecutive columns (one 16-byte load per token in bf16) and adds up the tokens
// w, w + 4, ...; the four partial sums meet in LDS and are added in wave order, so the result
// does not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace dash {

constexpr int kPoolCols = kWave * 8;  // columns per workgroup

// Streaming decode: the chunk that sequence b's newest token completed (its length clamped into
// [0, cap] is a positive multiple of the chunk size), or -1 when that token left its chunk open.
// A chunk's summary depends on its own keys only, so it is final from then on [DA §3.1].
__device__ __forceinline__ int completed_chunk(const int* ctx_lens, int b, int cap, int block) {
    const int n = min(max(ctx_lens[b], 0), cap);
    return n > 0 && n % block == 0 ? n / block - 1 : -1;
}

template <typename T>
__global__ __launch_bounds__(256) void pool_mean_kernel(const T* __restrict__ k,
                                                        float* __restrict__ kbar, int n_kv,
                                                        int cols, int block, int tc,
                                                        const int* __restrict__ ctx_lens) {
    const int b = blockIdx.z;
    const int c = ctx_lens ? completed_chunk(ctx_lens, b, n_kv, block) : (int)blockIdx.y;
    if (c < 0) return;  // the whole workgroup
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int col = blockIdx.x * kPoolCols + lane * 8;
    __shared__ float part[4][8][kWave];

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (col < cols) {
        const T* base = k + ((int64_t)b * n_kv + (int64_t)c * block) * cols + col;
#pragma unroll 4
        for (int t = w; t < block; t += 4) {
            float v[8];
            load8(base + (int64_t)t * cols, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[w][i][lane] = acc[i];
    __syncthreads();
    if (w == 0 && col < cols) {
        const float inv = 1.0f / (float)block;
        float s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            s[i] = (((part[0][i][lane] + part[1][i][lane]) + part[2][i][lane]) + part[3][i][lane]) * inv;
        float* out = kbar + ((int64_t)b * tc + c) * cols + col;
        *reinterpret_cast<float4*>(out) = make_float4(s[0], s[1], s[2], s[3]);
        *reinterpret_cast<float4*>(out + 4) = make_float4(s[4], s[5], s[6], s[7]);
    }
}

// Learned summary query (Eq. 3): one wave per (sequence, chunk, KV head). Lanes own tokens for
// the local logits <qbar, k_t> / sqrt(D) and their softmax, then own dimensions for the
// weighted sum of the chunk's keys.
template <typename T, int D>
__global__ __launch_bounds__(64) void pool_query_kernel(const T* __restrict__ k,
                                                        const float* __restrict__ qbar,
                                                        float* __restrict__ kbar, int n_kv,
                                                        int h_kv, int block, int tc,
                                                        const int* __restrict__ ctx_lens) {
    const int r = blockIdx.y, b = blockIdx.z;
    const int c = ctx_lens ? completed_chunk(ctx_lens, b, n_kv, block) : (int)blockIdx.x;
    if (c < 0) return;  // the whole workgroup
    const int lane = threadIdx.x;
    __shared__ float qs[D];
    __shared__ float pw[128];
    for (int e = lane; e < D; e += kWave) qs[e] = qbar[(int64_t)r * D + e];
    __syncthreads();

    const float inv_sqrt_d = rsqrtf((float)D);
    const int64_t row_stride = (int64_t)h_kv * D;
    const T* base = k + ((int64_t)b * n_kv + (int64_t)c * block) * row_stride + (int64_t)r * D;
    float s[2];
    float smax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = lane + i * kWave;
        s[i] = -INFINITY;
        if (u < block) {
            float dot = 0.f;
            for (int e = 0; e < D; e += 8) {
                float kv[8];
                load8(base + u * row_stride + e, kv);
#pragma unroll
                for (int j = 0; j < 8; ++j) dot = fmaf(qs[e + j], kv[j], dot);
            }
            s[i] = dot * inv_sqrt_d;
        }
        smax = fmaxf(smax, s[i]);
    }
    smax = wave_max(smax);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = lane + i * kWave;
        const float p = u < block ? __expf(s[i] - smax) : 0.f;
        if (u < block) pw[u] = p;
        z += p;
    }
    z = wave_sum(z);
    __syncthreads();
    const float inv_z = 1.0f / z;
    for (int e = lane; e < D; e += kWave) {
        float acc = 0.f;
        for (int u = 0; u < block; ++u) acc = fmaf(pw[u], to_f32(base[u * row_stride + e]), acc);
        kbar[(((int64_t)b * tc + c) * h_kv + r) * D + e] = acc * inv_z;
    }
}

hipError_t launch_pool_mean(const void* k, int dt, float* kbar, int batch, int n_kv, int h_kv,
                            int head_dim, int block, hipStream_t st) {
    const int tc = n_kv / block;
    const int cols = h_kv * head_dim;
    if (tc == 0) return hipSuccess;
    dim3 grid(div_up(cols, kPoolCols), tc, batch);
    if (dt == kBF16)
        hipLaunchKernelGGL(pool_mean_kernel<bf16_t>, grid, dim3(256), 0, st,
                           static_cast<const bf16_t*>(k), kbar, n_kv, cols, block, tc, nullptr);
    else
        hipLaunchKernelGGL(pool_mean_kernel<float>, grid, dim3(256), 0, st,
                           static_cast<const float*>(k), kbar, n_kv, cols, block, tc, nullptr);
    return hipGetLastError();
}

hipError_t launch_pool_query(const void* k, int dt, const float* qbar, float* kbar, int batch,
                             int n_kv, int h_kv, int head_dim, int block, hipStream_t st) {
    const int tc = n_kv / block;
    if (tc == 0) return hipSuccess;
    dim3 grid(tc, h_kv, batch);
#define DASH_POOLQ(T, DD)                                                                  \
    hipLaunchKernelGGL((pool_query_kernel<T, DD>), grid, dim3(64), 0, st,                  \
                       static_cast<const T*>(k), qbar, kbar, n_kv, h_kv, block, tc, nullptr)
    if (dt == kBF16) {
        if (head_dim == 64) DASH_POOLQ(bf16_t, 64); else DASH_POOLQ(bf16_t, 128);
    } else {
        if (head_dim == 64) DASH_POOLQ(float, 64); else DASH_POOLQ(float, 128);
    }
#undef DASH_POOLQ
    return hipGetLastError();
}

// Summaries of the chunks completed by each sequence's newest token (streaming decode): one
// workgroup per sequence (and column slab, or KV head), idle where no chunk completed.
hipError_t launch_pool_append(const void* k, int dt, const float* qbar, const int* ctx_lens,
                              float* kbar, int batch, int n_cap, int h_kv, int head_dim, int block,
                              hipStream_t st) {
    const int tc = n_cap / block;
    if (tc == 0) return hipSuccess;
    if (!qbar) {
        const int cols = h_kv * head_dim;
        dim3 grid(div_up(cols, kPoolCols), 1, batch);
        if (dt == kBF16)
            hipLaunchKernelGGL(pool_mean_kernel<bf16_t>, grid, dim3(256), 0, st,
                               static_cast<const bf16_t*>(k), kbar, n_cap, cols, block, tc, ctx_lens);
        else
            hipLaunchKernelGGL(pool_mean_kernel<float>, grid, dim3(256), 0, st,
                               static_cast<const float*>(k), kbar, n_cap, cols, block, tc, ctx_lens);
        return hipGetLastError();
    }
    dim3 grid(1, h_kv, batch);
#define DASH_POOLQ(T, DD)                                                                  \
    hipLaunchKernelGGL((pool_query_kernel<T, DD>), grid, dim3(64), 0, st,                  \
                       static_cast<const T*>(k), qbar, kbar, n_cap, h_kv, block, tc, ctx_lens)
    if (dt == kBF16) {
        if (head_dim == 64) DASH_POOLQ(bf16_t, 64); else DASH_POOLQ(bf16_t, 128);
    } else {
        if (head_dim == 64) DASH_POOLQ(float, 64); else DASH_POOLQ(float, 128);
    }
#undef DASH_POOLQ
    return hipGetLastError();
}

}  // namespace dash
