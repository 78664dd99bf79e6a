// Stage 2: prior-induced sparse softmax attention ("DashAttention", arXiv 2605.18753v1,
// §3.3-3.4 Eq. 7-10 in the bias form of Prop. 1; App. G Alg. 3).
//
// attn_row_kernel is the fp32 prefill path: one wave per (query, KV group), all g
// heads of the group at once, walking the set bits of the query's mask row chunk by chunk with
// an online softmax. Lanes own keys for the scores and head dimensions for the value
// accumulation. bf16 prefill runs on MFMA tiles (sparse_attn_mfma.hip).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dash {

template <typename T, int D, int G>
__global__ __launch_bounds__(64) void attn_row_kernel(const T* __restrict__ q,
                                                      const T* __restrict__ k,
                                                      const T* __restrict__ v,
                                                      const uint32_t* __restrict__ mask,
                                                      const float* __restrict__ bias,
                                                      T* __restrict__ o, float* __restrict__ lse,
                                                      AttnParams p) {
    constexpr int DPL = D / kWave;  // head dimensions per lane
    const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int pos = p.q_pos0 + t;
    const int cp = pos / p.block;
    const int64_t qrow = (int64_t)b * p.n_q + t;

    __shared__ float qs[G][D];
    __shared__ float ps[G][kWave];
    for (int i = lane; i < G * D; i += kWave) {
        const int gg = i / D, e = i % D;
        qs[gg][e] = to_f32(q[(qrow * p.h_q + r * G + gg) * D + e]) * p.scale;
    }
    __syncthreads();

    float acc[G][DPL];
    float mrun[G], lrun[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
        mrun[gg] = -INFINITY;
        lrun[gg] = 0.f;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) acc[gg][dd] = 0.f;
    }
    const uint32_t* mrow = mask + (qrow * p.h_kv + r) * p.nw;
    const float* brow = bias + (qrow * p.h_kv + r) * p.nc;
    const int64_t kstride = (int64_t)p.h_kv * D;
    const T* kb = k + (int64_t)b * p.n_kv * kstride + (int64_t)r * D;
    const T* vb = v + (int64_t)b * p.n_kv * kstride + (int64_t)r * D;

    for (int c = 0; c <= cp; ++c) {
        if (c < cp && !((mrow[c >> 5] >> (c & 31)) & 1u)) continue;
        const float d = c < cp ? brow[c] : 0.f;  // the query's own chunk carries no bias
        const int kend = c < cp ? (c + 1) * p.block : pos + 1;
        for (int k0 = c * p.block; k0 < kend; k0 += kWave) {
            const int key = k0 + lane;
            const bool valid = key < kend;
            float s[G];
#pragma unroll
            for (int gg = 0; gg < G; ++gg) s[gg] = 0.f;
            if (valid) {
                for (int e = 0; e < D; e += 8) {
                    float kv[8];
                    load8(kb + key * kstride + e, kv);
#pragma unroll
                    for (int gg = 0; gg < G; ++gg)
#pragma unroll
                        for (int j = 0; j < 8; ++j) s[gg] = fmaf(qs[gg][e + j], kv[j], s[gg]);
                }
            }
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
                const float sg = valid ? s[gg] + d : -INFINITY;
                const float mnew = fmaxf(mrun[gg], wave_max(sg));
                const float pe = valid ? __expf(sg - mnew) : 0.f;
                const float corr = __expf(mrun[gg] - mnew);
                lrun[gg] = lrun[gg] * corr + wave_sum(pe);
#pragma unroll
                for (int dd = 0; dd < DPL; ++dd) acc[gg][dd] *= corr;
                mrun[gg] = mnew;
                ps[gg][lane] = pe;
            }
            __syncthreads();
            const int nk = min(kWave, kend - k0);
            for (int j = 0; j < nk; ++j) {
                const T* vr = vb + (int64_t)(k0 + j) * kstride;
                float vv[DPL];
#pragma unroll
                for (int dd = 0; dd < DPL; ++dd) vv[dd] = to_f32(vr[lane + kWave * dd]);
#pragma unroll
                for (int gg = 0; gg < G; ++gg) {
                    const float pj = ps[gg][j];
#pragma unroll
                    for (int dd = 0; dd < DPL; ++dd) acc[gg][dd] = fmaf(pj, vv[dd], acc[gg][dd]);
                }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
        const float inv = 1.0f / lrun[gg];
        T* orow = o + (qrow * p.h_q + r * G + gg) * D;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) store_elem(orow + lane + kWave * dd, acc[gg][dd] * inv);
        if (lse && lane == 0) lse[qrow * p.h_q + r * G + gg] = mrun[gg] + __logf(lrun[gg]);
    }
}

template <typename T, int D>
static void launch_row(const void* q, const void* k, const void* v, const uint32_t* mask,
                       const float* bias, void* o, float* lse, const AttnParams& p,
                       hipStream_t st) {
    dim3 grid(p.n_q, p.h_kv, p.batch);
#define DASH_ROW(GG)                                                                        \
    hipLaunchKernelGGL((attn_row_kernel<T, D, GG>), grid, dim3(kWave), 0, st,               \
                       static_cast<const T*>(q), static_cast<const T*>(k),                  \
                       static_cast<const T*>(v), mask, bias, static_cast<T*>(o), lse, p)
    switch (p.g) {
        case 1: DASH_ROW(1); break;
        case 2: DASH_ROW(2); break;
        case 4: DASH_ROW(4); break;
        case 8: DASH_ROW(8); break;
        default: DASH_ROW(16); break;
    }
#undef DASH_ROW
}

static void launch_row_any(const void* q, const void* k, const void* v, int dt,
                           const uint32_t* mask, const float* bias, void* o, float* lse,
                           const AttnParams& p, hipStream_t st) {
    if (dt == kBF16) {
        if (p.head_dim == 64) launch_row<bf16_t, 64>(q, k, v, mask, bias, o, lse, p, st);
        else launch_row<bf16_t, 128>(q, k, v, mask, bias, o, lse, p, st);
    } else {
        if (p.head_dim == 64) launch_row<float, 64>(q, k, v, mask, bias, o, lse, p, st);
        else launch_row<float, 128>(q, k, v, mask, bias, o, lse, p, st);
    }
}

hipError_t launch_attn_prefill(const void* q, const void* k, const void* v, int dt,
                               const uint32_t* mask, const float* bias, void* o, float* lse,
                               const AttnParams& p, hipStream_t st) {
    if (dt == kBF16) return launch_attn_prefill_mfma(q, k, v, mask, bias, o, lse, p, st);
    launch_row_any(q, k, v, dt, mask, bias, o, lse, p, st);
    return hipGetLastError();
}

}  // namespace dash
