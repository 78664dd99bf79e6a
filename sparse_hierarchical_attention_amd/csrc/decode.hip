// Stage 2 for one new token per sequence: split-KV sparse attention ("DashAttention",
// arXiv 2605.18753v1, §3.5 "split-KV variant"; the output is that of §3.4 Prop. 1).
//
// The units of kDecUnit keys of a (sequence, group)'s selection (decode_common.h) go to
// kDecodeSlots slots, unit u to slot u % kDecodeSlots. decode_split_kernel: each wave owns one
// slot (and, for groups of more than four heads, one set of four heads); the waves of a
// workgroup merge their slots in LDS and write one partial (unnormalised output, max, sum) per
// head to the workspace. decode_combine_kernel merges the workgroups' partials in order.
#include <math.h>

#include "common.h"
#include "decode_common.h"
#include "kernels.h"

namespace dash {

constexpr int kDecodeSlots = 32;   // unit slots per (sequence, group)

// workgroups (of four waves) per (sequence, group)
__host__ __device__ constexpr int dec_workgroups(int g) {
    return kDecodeSlots * dec_waves_per_slot(g) / 4;
}

// workspace: [B, H_kv, dec_workgroups(g), g, D + 4] floats: D unnormalised outputs, max (log2),
// sum, two floats of padding (16-byte aligned records)
template <typename T, int D, int GQ>
__global__ __launch_bounds__(256) void decode_split_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           const T* __restrict__ v,
                                                           const uint32_t* __restrict__ mask,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ ws, AttnParams p) {
    constexpr int WPS = dec_waves_per_slot(GQ);  // waves per slot (sets of four heads)
    constexpr int HPW = dec_heads_per_wave(GQ);  // heads per wave
    constexpr int SPW = 4 / WPS;                 // slots per workgroup
    constexpr int DS = D + 4;                    // workspace record
    using Wave = DecodeWave<T, D, HPW>;
    __shared__ __align__(16) T qs[GQ * D];
    __shared__ __align__(16) float part[4][HPW][DS];
    __shared__ int wtot[4];
    __shared__ uint16_t chunks[kDecMaxWords * 32];  // rank -> chunk

    const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = p.n_kv;  // cache capacity (the row stride of K and V)
    const int pos = seq_pos(p.ctx_lens, n - 1, n, b, 0);
    const int cp = pos / p.block;
    const uint32_t* mrow = mask + ((int64_t)b * p.h_kv + r) * p.nw;
    const float* brow = bias + ((int64_t)b * p.h_kv + r) * p.nc;

    for (int e = tid; e < GQ * D / Wave::EPL; e += 256)
        reinterpret_cast<uint4*>(qs)[e] =
            reinterpret_cast<const uint4*>(q + ((int64_t)b * p.h_q + r * GQ) * D)[e];
    const int total = chunk_list([&](int i) { return mrow[i]; }, cp, wtot, chunks);

    const int cs = wave / WPS;              // slot within the workgroup
    const int h0 = (wave % WPS) * HPW;      // first head of this wave within the group
    const int li = lane % Wave::LPK;
    const int upc = (p.block + kDecUnit - 1) / kDecUnit;  // units per chunk
    const int64_t kv_stride = (int64_t)p.h_kv * D;
    const T* kb = k + (int64_t)b * n * kv_stride + (int64_t)r * D + li * Wave::EPL;
    const T* vb = v + (int64_t)b * n * kv_stride + (int64_t)r * D + li * Wave::EPL;

    uint4 qp[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
        qp[hh] = *reinterpret_cast<const uint4*>(&qs[(h0 + hh) * D + li * Wave::EPL]);
    Wave st;
    st.init();
    st.run(kb, vb, kv_stride, qp, chunks, total * upc, s * SPW + cs, kDecodeSlots, upc, p.block,
           pos, cp, p.scale * kDecLog2e, [&](int c) { return brow[c]; });
    st.store(&part[wave][0][0]);
    __syncthreads();
    // merge the workgroup's slots (waves cs * WPS + set, in slot order) per head; an empty slot
    // has max = -inf and sum = 0
    for (int e = tid; e < GQ * D; e += 256) {
        const int hg = e / D, d = e % D;
        const int set = hg / HPW, hh = hg % HPW;
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < SPW; ++c) mx = fmaxf(mx, part[c * WPS + set][hh][D]);
        const float2 ol = merge_parts([&](int c) { return &part[c * WPS + set][hh][0]; }, SPW, D, d);
        float* out = ws + ((((int64_t)b * p.h_kv + r) * gridDim.x + s) * GQ + hg) * DS;
        out[d] = ol.x;
        if (d == 0) {
            out[D] = mx;
            out[D + 1] = ol.y;
        }
    }
}

template <typename T, int D, int NP>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws,
                                                            T* __restrict__ o, AttnParams p) {
    constexpr int DPL = D / 64;
    const int h = blockIdx.x, b = blockIdx.y;
    const int r = h / p.g, hh = h % p.g;
    const int lane = threadIdx.x;
    const float* base = ws + (((int64_t)b * p.h_kv + r) * NP * p.g + hh) * (D + 4);
    const int64_t part_stride = (int64_t)p.g * (D + 4);
    // all partial maxima, sums and outputs first (independent loads), then the weights
    float ms[NP], ls[NP], os[NP][DPL];
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        ms[s] = base[s * part_stride + D];
        ls[s] = base[s * part_stride + D + 1];
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) os[s][dd] = base[s * part_stride + lane + 64 * dd];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < NP; ++s) mx = fmaxf(mx, ms[s]);
    float l = 0.f, acc[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) acc[dd] = 0.f;
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        const float f = ms[s] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[s] - mx);
        l = fmaf(f, ls[s], l);
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) acc[dd] = f > 0.f ? fmaf(f, os[s][dd], acc[dd]) : acc[dd];
    }
    const float inv = 1.0f / l;
    T* orow = o + ((int64_t)b * p.h_q + h) * D;
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) store_elem(orow + lane + 64 * dd, acc[dd] * inv);
}

size_t decode_workspace_bytes(const AttnParams& p) {
    return (size_t)p.batch * p.h_kv * dec_workgroups(p.g) * p.g * (p.head_dim + 4) * sizeof(float);
}

template <typename T, int D>
static void launch_decode_t(const void* q, const void* k, const void* v, const uint32_t* mask,
                            const float* bias, void* o, const AttnParams& p, float* ws,
                            hipStream_t st) {
#define DASH_DEC(GG)                                                                           \
    hipLaunchKernelGGL((decode_split_kernel<T, D, GG>), dim3(dec_workgroups(GG), p.h_kv, p.batch), \
                       dim3(256), 0, st, static_cast<const T*>(q), static_cast<const T*>(k),     \
                       static_cast<const T*>(v), mask, bias, ws, p);                             \
    hipLaunchKernelGGL((decode_combine_kernel<T, D, dec_workgroups(GG)>), dim3(p.h_q, p.batch),  \
                       dim3(64), 0, st, ws, static_cast<T*>(o), p)
    switch (p.g) {
        case 1: DASH_DEC(1); break;
        case 2: DASH_DEC(2); break;
        case 4: DASH_DEC(4); break;
        case 8: DASH_DEC(8); break;
        default: DASH_DEC(16); break;
    }
#undef DASH_DEC
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
