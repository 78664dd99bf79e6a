// Stage 2 for one new token per sequence: split-KV sparse attention ("DashAttention",
// arXiv 2605.18753v1, §3.5 "split-KV variant"; the output is that of §3.4 Prop. 1).
//
// The units of kDecUnit keys of a (sequence, group)'s selection (decode_common.h) go to S slots,
// unit u to slot u % S, where S grows with the selection: 32 slots up to 256 units, then one per
// 8 units up to 128 (dec_slots), so that a (sequence, group) that routed hundreds of chunks (a
// short sequence whose candidates hold no clear peak) does not serialise the step while the
// others wait. decode_split_kernel: each wave owns one slot (and, for groups of more than four
// heads, one set of four heads); a workgroup whose slots are all past S leaves at once; the waves
// of a workgroup merge their slots in LDS and write one partial (unnormalised output, max, sum)
// per head to the workspace. decode_combine_kernel recounts S from the mask and merges the
// partials of the S / (slots per workgroup) workgroups in order.
#include <math.h>

#include "common.h"
#include "decode_common.h"
#include "kernels.h"

namespace dash {

constexpr int kDecodeSlots = 32;      // unit slots per (sequence, group), at least
constexpr int kDecodeMaxSlots = 128;  // and at most
constexpr int kDecodeUnitsPerSlot = 8;

// slots for a selection of `units` units: a multiple of 4 (the slots of one workgroup)
__host__ __device__ constexpr int dec_slots(int units) {
    return units <= kDecodeSlots * kDecodeUnitsPerSlot ? kDecodeSlots
           : units >= kDecodeMaxSlots * kDecodeUnitsPerSlot
               ? kDecodeMaxSlots
               : ((units + kDecodeUnitsPerSlot - 1) / kDecodeUnitsPerSlot + 3) / 4 * 4;
}

// workgroups (of four waves) per (sequence, group) for S slots
__host__ __device__ constexpr int dec_workgroups(int g, int slots = kDecodeMaxSlots) {
    return slots * dec_waves_per_slot(g) / 4;
}

// units of the (sequence, group)'s selection: its chunks below the own chunk cp whose bit is set
// (whole chunks) and the own chunk (all of its units counted; those past the query are empty)
__device__ __forceinline__ int dec_units(const uint32_t* mrow, int cp) {
    int total = 0;
    for (int wd = threadIdx.x; wd <= cp / 32; wd += blockDim.x) {
        uint32_t word = mrow[wd];
        const int hi = cp - 32 * wd;
        if (hi < 31) word &= (2u << hi) - 1u;
        if (hi < 32) word |= 1u << hi;
        total += __popc(word);
    }
    return total;  // this thread's share; the caller sums over the workgroup
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

    // the slot-set index is the slowest grid dimension: the workgroups every (sequence, group)
    // uses (the first 32 slots) are dispatched first, the extra ones for long selections last
    const int r = blockIdx.x, b = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = p.n_kv;  // cache capacity (the row stride of K and V)
    const int pos = seq_pos(p.ctx_lens, n - 1, n, b, 0);
    const int cp = pos / p.block;
    const uint32_t* mrow = mask + ((int64_t)b * p.h_kv + r) * p.nw;
    const float* brow = bias + ((int64_t)b * p.h_kv + r) * p.nc;

    const int total = chunk_list([&](int i) { return mrow[i]; }, cp, wtot, chunks);
    const int upc = (p.block + kDecUnit - 1) / kDecUnit;  // units per chunk
    const int slots = dec_slots(total * upc);
    if (s * SPW >= slots) return;  // every slot of this workgroup is idle (uniform)
    for (int e = tid; e < GQ * D / Wave::EPL; e += 256)
        reinterpret_cast<uint4*>(qs)[e] =
            reinterpret_cast<const uint4*>(q + ((int64_t)b * p.h_q + r * GQ) * D)[e];
    __syncthreads();

    const int cs = wave / WPS;              // slot within the workgroup
    const int h0 = (wave % WPS) * HPW;      // first head of this wave within the group
    const int li = lane % Wave::LPK;
    const int64_t kv_stride = (int64_t)p.h_kv * D;
    const T* kb = k + (int64_t)b * n * kv_stride + (int64_t)r * D + li * Wave::EPL;
    const T* vb = v + (int64_t)b * n * kv_stride + (int64_t)r * D + li * Wave::EPL;

    uint4 qp[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
        qp[hh] = *reinterpret_cast<const uint4*>(&qs[(h0 + hh) * D + li * Wave::EPL]);
    Wave st;
    st.init();
    st.run(kb, vb, kv_stride, qp, chunks, total * upc, s * SPW + cs, slots, upc, p.block,
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
        float* out = ws + ((((int64_t)b * p.h_kv + r) * gridDim.z + s) * GQ + hg) * DS;
        out[d] = ol.x;
        if (d == 0) {
            out[D] = mx;
            out[D + 1] = ol.y;
        }
    }
}

template <typename T, int D, int WPS>
__global__ __launch_bounds__(64) void decode_combine_kernel(const uint32_t* __restrict__ mask,
                                                            const float* __restrict__ ws,
                                                            T* __restrict__ o, AttnParams p) {
    constexpr int DPL = D / 64;
    const int h = blockIdx.x, b = blockIdx.y;
    const int r = h / p.g, hh = h % p.g;
    const int lane = threadIdx.x;
    const int n = p.n_kv;
    const int cp = seq_pos(p.ctx_lens, n - 1, n, b, 0) / p.block;
    const int upc = (p.block + kDecUnit - 1) / kDecUnit;
    const int units = wave_sum_int(dec_units(mask + ((int64_t)b * p.h_kv + r) * p.nw, cp)) * upc;
    const int np = dec_slots(units) * WPS / 4;  // workgroups that wrote a partial, in order
    const int nmax = dec_workgroups(p.g);
    const float* base = ws + (((int64_t)b * p.h_kv + r) * nmax * p.g + hh) * (D + 4);
    const int64_t part_stride = (int64_t)p.g * (D + 4);
    // batches of 8 partials: their loads are issued together, then merged into a running
    // (max, sum, output) in partial order
    constexpr int NB = 8;
    float mx = -INFINITY, l = 0.f, acc[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) acc[dd] = 0.f;
    for (int s0 = 0; s0 < np; s0 += NB) {
        float ms[NB], ls[NB], os[NB][DPL];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const bool in = s0 + i < np;
            const float* pr = base + (int64_t)(in ? s0 + i : 0) * part_stride;
            ms[i] = in ? pr[D] : -INFINITY;
            ls[i] = in ? pr[D + 1] : 0.f;
#pragma unroll
            for (int dd = 0; dd < DPL; ++dd) os[i][dd] = in ? pr[lane + 64 * dd] : 0.f;
        }
        float bm = mx;
#pragma unroll
        for (int i = 0; i < NB; ++i) bm = fmaxf(bm, ms[i]);
        const float fr = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - bm);
        l *= fr;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) acc[dd] *= fr;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const float f = ms[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[i] - bm);
            l = fmaf(f, ls[i], l);
#pragma unroll
            for (int dd = 0; dd < DPL; ++dd) acc[dd] = f > 0.f ? fmaf(f, os[i][dd], acc[dd]) : acc[dd];
        }
        mx = bm;
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
    hipLaunchKernelGGL((decode_split_kernel<T, D, GG>), dim3(p.h_kv, p.batch, dec_workgroups(GG)), \
                       dim3(256), 0, st, static_cast<const T*>(q), static_cast<const T*>(k),     \
                       static_cast<const T*>(v), mask, bias, ws, p);                             \
    hipLaunchKernelGGL((decode_combine_kernel<T, D, dec_waves_per_slot(GG)>), dim3(p.h_q, p.batch), \
                       dim3(64), 0, st, mask, ws, static_cast<T*>(o), p)
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
