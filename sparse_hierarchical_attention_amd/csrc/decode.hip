// Stage 2 for one new token per sequence: split-KV sparse attention ("DashAttention",
// arXiv 2605.18753v1, §3.5 "split-KV variant"; the output is that of §3.4 Prop. 1).
//
// decode_split_kernel: workgroup (s, r, b) takes the s-th, (s + S)-th, ... chunk among the
// query's routed chunks and its own chunk (in increasing chunk order), stages each chunk's K and
// V through LDS with coalesced 16-byte loads and keeps, per head of group r, a partial online
// softmax (max, sum, unnormalised output) that it writes to the workspace.
// decode_combine_kernel: merges the S partials of every head in a fixed order (deterministic).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dash {

constexpr int kDecodeSplits = 16;
constexpr float kDecLog2e = 1.4426950408889634f;

// workspace: [B, H_kv, S, g, D + 2] floats: D unnormalised outputs, then max (log2 domain), sum
__host__ __device__ inline int decode_splits(int nc) { return nc < kDecodeSplits ? nc : kDecodeSplits; }

template <typename T, int D, int GQ>
__global__ __launch_bounds__(256) void decode_split_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           const T* __restrict__ v,
                                                           const uint32_t* __restrict__ mask,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ ws, AttnParams p) {
    constexpr int KT = sizeof(T) == 2 ? 64 : 32;  // keys per LDS tile
    constexpr int EPV = 16 / sizeof(T);           // elements per 16-byte load
    constexpr int DPL = D / 64;                   // output dims per lane
    constexpr int HPW = GQ < 4 ? 1 : GQ / 4;      // heads per wave
    constexpr int KS = D + EPV;  // padded K rows: 16 lanes start on 16 different 4-bank groups
    __shared__ __align__(16) T ks[KT * KS];
    __shared__ __align__(16) T vs[KT * D];
    __shared__ float qs[GQ * D];
    __shared__ float ps[GQ][KT];

    const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int S = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = p.n_kv;
    const int pos = n - 1;
    const int cp = pos / p.block;
    const uint32_t* mrow = mask + ((int64_t)b * p.h_kv + r) * p.nw;
    const float* brow = bias + ((int64_t)b * p.h_kv + r) * p.nc;
    const float qk_scale = p.scale * kDecLog2e;

    for (int e = tid; e < GQ * D; e += 256)
        qs[e] = to_f32(q[((int64_t)b * p.h_q + r * GQ) * D + e]) * qk_scale;

    float acc[HPW][DPL];
    float m_run[HPW], l_run[HPW];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.f;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) acc[i][dd] = 0.f;
    }
    const int64_t kv_stride = (int64_t)p.h_kv * D;
    const T* kb = k + (int64_t)b * n * kv_stride + (int64_t)r * D;
    const T* vb = v + (int64_t)b * n * kv_stride + (int64_t)r * D;

    int rank = 0;
    for (int w = 0; w <= cp / 32; ++w) {
        const int hi = cp - 32 * w;
        uint32_t word = mrow[w];
        if (hi < 31) word &= (2u << hi) - 1u;
        if (hi < 32) word |= 1u << hi;
        while (word) {
            const int bit = __builtin_ctz(word);
            word &= word - 1u;
            const int mine = rank % S == s;
            ++rank;
            if (!mine) continue;
            const int c = 32 * w + bit;
            const bool diag = c == cp;
            const float off = diag ? 0.f : brow[c] * kDecLog2e;
            const int kend = diag ? pos + 1 : (c + 1) * p.block;
            for (int k0 = c * p.block; k0 < kend; k0 += KT) {
                __syncthreads();
                for (int e = tid; e < KT * D / EPV; e += 256) {
                    const int kk = e / (D / EPV), dv = e % (D / EPV);
                    const int key = k0 + kk;
                    uint4 uk = make_uint4(0, 0, 0, 0), uv = make_uint4(0, 0, 0, 0);
                    if (key < kend) {
                        uk = *reinterpret_cast<const uint4*>(kb + key * kv_stride + EPV * dv);
                        uv = *reinterpret_cast<const uint4*>(vb + key * kv_stride + EPV * dv);
                    }
                    *reinterpret_cast<uint4*>(&ks[kk * KS + EPV * dv]) = uk;
                    *reinterpret_cast<uint4*>(&vs[kk * D + EPV * dv]) = uv;
                }
                __syncthreads();
                // scores: lane = key, wave owns heads wave, wave + 4, ...
                const int key = k0 + lane;
#pragma unroll
                for (int i = 0; i < HPW; ++i) {
                    const int hh = wave + 4 * i;
                    if (hh >= GQ) break;
                    float sc = -INFINITY;
                    if (lane < KT && key < kend) {
                        float dot = 0.f;
                        for (int e = 0; e < D; e += 8) {
                            float kv[8];
                            load8(&ks[lane * KS + e], kv);
#pragma unroll
                            for (int jj = 0; jj < 8; ++jj) dot = fmaf(qs[hh * D + e + jj], kv[jj], dot);
                        }
                        sc = dot + off;
                    }
                    const float m_new = fmaxf(m_run[i], wave_max(sc));
                    const float pe = __builtin_amdgcn_exp2f(sc - m_new);
                    const float corr = __builtin_amdgcn_exp2f(m_run[i] - m_new);
                    l_run[i] = l_run[i] * corr + wave_sum(pe);
                    m_run[i] = m_new;
#pragma unroll
                    for (int dd = 0; dd < DPL; ++dd) acc[i][dd] *= corr;
                    if (lane < KT) ps[hh][lane] = pe;
                }
                __syncthreads();
                const int nk = min(KT, kend - k0);
#pragma unroll
                for (int i = 0; i < HPW; ++i) {
                    const int hh = wave + 4 * i;
                    if (hh >= GQ) break;
                    for (int kk = 0; kk < nk; ++kk) {
                        const float pk = ps[hh][kk];
#pragma unroll
                        for (int dd = 0; dd < DPL; ++dd)
                            acc[i][dd] = fmaf(pk, to_f32(vs[kk * D + lane + 64 * dd]), acc[i][dd]);
                    }
                }
            }
        }
    }
    // partial results of this split (an empty split leaves max = -inf, sum = 0)
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int hh = wave + 4 * i;
        if (hh >= GQ) break;
        float* out = ws + ((((int64_t)b * p.h_kv + r) * S + s) * GQ + hh) * (D + 2);
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) out[lane + 64 * dd] = acc[i][dd];
        if (lane == 0) {
            out[D] = m_run[i];
            out[D + 1] = l_run[i];
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws,
                                                            T* __restrict__ o, AttnParams p,
                                                            int S) {
    constexpr int DPL = D / 64;
    const int h = blockIdx.x, b = blockIdx.y;
    const int r = h / p.g, hh = h % p.g;
    const int lane = threadIdx.x;
    const float* base = ws + (((int64_t)b * p.h_kv + r) * S * p.g + hh) * (D + 2);
    const int64_t split_stride = (int64_t)p.g * (D + 2);
    // all partial maxima and sums first (independent loads), then the weighted outputs
    float ms[kDecodeSplits], ls[kDecodeSplits];
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < kDecodeSplits; ++s) {
        ms[s] = s < S ? base[s * split_stride + D] : -INFINITY;
        ls[s] = s < S ? base[s * split_stride + D + 1] : 0.f;
    }
#pragma unroll
    for (int s = 0; s < kDecodeSplits; ++s) mx = fmaxf(mx, ms[s]);
    float l = 0.f, acc[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) acc[dd] = 0.f;
#pragma unroll
    for (int s = 0; s < kDecodeSplits; ++s) {
        if (s >= S) break;
        const float f = ms[s] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[s] - mx);
        l = fmaf(f, ls[s], l);
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) acc[dd] = fmaf(f, base[s * split_stride + lane + 64 * dd], acc[dd]);
    }
    const float inv = 1.0f / l;
    T* orow = o + ((int64_t)b * p.h_q + h) * D;
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) store_elem(orow + lane + 64 * dd, acc[dd] * inv);
}

size_t decode_workspace_bytes(const AttnParams& p) {
    return (size_t)p.batch * p.h_kv * decode_splits(p.nc) * p.g * (p.head_dim + 2) * sizeof(float);
}

template <typename T, int D>
static void launch_decode_t(const void* q, const void* k, const void* v, const uint32_t* mask,
                            const float* bias, void* o, const AttnParams& p, float* ws,
                            hipStream_t st) {
    const int S = decode_splits(p.nc);
    dim3 grid(S, p.h_kv, p.batch);
#define DASH_DEC(GG)                                                                        \
    hipLaunchKernelGGL((decode_split_kernel<T, D, GG>), grid, dim3(256), 0, st,             \
                       static_cast<const T*>(q), static_cast<const T*>(k),                  \
                       static_cast<const T*>(v), mask, bias, ws, p)
    switch (p.g) {
        case 1: DASH_DEC(1); break;
        case 2: DASH_DEC(2); break;
        case 4: DASH_DEC(4); break;
        case 8: DASH_DEC(8); break;
        default: DASH_DEC(16); break;
    }
#undef DASH_DEC
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.h_q, p.batch), dim3(64), 0, st, ws,
                       static_cast<T*>(o), p, S);
}

hipError_t launch_attn_decode(const void* q, const void* k, const void* v, int dt,
                              const uint32_t* mask, const float* bias, void* o,
                              const AttnParams& p, void* ws, hipStream_t st) {
    float* w = static_cast<float*>(ws);
    if (dt == kBF16) {
        if (p.head_dim == 64) launch_decode_t<bf16_t, 64>(q, k, v, mask, bias, o, p, w, st);
        else launch_decode_t<bf16_t, 128>(q, k, v, mask, bias, o, p, w, st);
    } else {
        if (p.head_dim == 64) launch_decode_t<float, 64>(q, k, v, mask, bias, o, p, w, st);
        else launch_decode_t<float, 128>(q, k, v, mask, bias, o, p, w, st);
    }
    return hipGetLastError();
}

}  // namespace dash
