// Stage 2 for one new token per sequence: split-KV sparse attention ("DashAttention",
// arXiv 2605.18753v1, §3.5 "split-KV variant"; the output is that of §3.4 Prop. 1).
//
// The units of kDecUnit keys of a (sequence, group)'s selection (decode_common.h) go to S slots,
// unit u to slot u % S, where S grows with the selection: 32 slots up to 256 units, then one per
// 8 units up to 128 (dec_slots), so that a (sequence, group) that routed hundreds of chunks (a
// short sequence whose candidates hold no clear peak) does not serialise the step while the
// others wait. Each wave owns one slot (and, for groups of more than four heads, one set of four
// heads); a workgroup whose slots are all past S leaves at once; the waves of a workgroup merge
// their slots in LDS and write one partial (unnormalised output, max, sum) per head to the
// workspace as a hand-over (common.h). The last workgroup of a (sequence, group) to finish merges
// the partials of all of them, in slot order, into the output: every workgroup stores its
// partial, then takes a ticket from the (sequence, group)'s counter; the one that draws the last
// ticket merges and resets the counter to zero for the next call. No workgroup ever waits for
// another, and the merge order does not depend on which workgroup is last, so the output is
// deterministic.
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

// LDS of one (sequence, group)'s attention in a workgroup of four waves.
template <typename T, int D, int GQ>
struct DecodeLds {
    static constexpr int HPW = dec_heads_per_wave(GQ);
    T qs[GQ * D];                          // the group's queries
    float part[4][HPW][D + 4];             // the waves' partials
    int wtot[4];
    uint16_t chunks[kDecMaxWords * 32];    // rank -> chunk (then the merge's (max, sum) pairs)
};

// The attention of query (b, r) by slot set s of the grid's gridDim.z (four waves; the group's
// queries already in L.qs, visible after the next barrier): the selected chunks come from
// word_of(i), the mask words, and bias_of(c); the workgroup's partial goes to the group's records
// in ws as a hand-over, and the last of the group's working workgroups merges them into o.
// ws: partial records [B, H_kv, gridDim.z, g, D + 4] floats (D unnormalised outputs, max (log2),
// sum, two floats of padding: 16-byte aligned records); tickets: one counter per (sequence,
// group), zero between calls.
template <typename T, int D, int GQ, class WORD, class BIAS>
__device__ __forceinline__ void decode_attend_group(const T* __restrict__ k, const T* __restrict__ v,
                                                    WORD word_of, BIAS bias_of, float* ws,
                                                    unsigned* tickets, T* __restrict__ o,
                                                    const AttnParams& p, int b, int r, int s,
                                                    DecodeLds<T, D, GQ>& L) {
    constexpr int WPS = dec_waves_per_slot(GQ);  // waves per slot (sets of four heads)
    constexpr int HPW = dec_heads_per_wave(GQ);  // heads per wave
    constexpr int SPW = 4 / WPS;                 // slots per workgroup
    constexpr int DS = D + 4;                    // workspace record
    using Wave = DecodeWave<T, D, HPW>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = p.n_kv;  // cache capacity (the row stride of K and V)
    const int pos = seq_pos(p.ctx_lens, n - 1, n, b, 0);
    const int cp = pos / p.block;

    const int total = chunk_list(word_of, cp, L.wtot, L.chunks);  // ends with a barrier
    const int upc = (p.block + kDecUnit - 1) / kDecUnit;  // units per chunk
    const int slots = min(dec_slots(total * upc), (int)gridDim.z * SPW);
    if (s * SPW >= slots) return;  // every slot of this workgroup is idle (uniform)

    const int cs = wave / WPS;              // slot within the workgroup
    const int h0 = (wave % WPS) * HPW;      // first head of this wave within the group
    const int li = lane % Wave::LPK;
    const int64_t kv_stride = (int64_t)p.h_kv * D;
    const T* kb = k + (int64_t)b * n * kv_stride + (int64_t)r * D + li * Wave::EPL;
    const T* vb = v + (int64_t)b * n * kv_stride + (int64_t)r * D + li * Wave::EPL;

    uint4 qp[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
        qp[hh] = *reinterpret_cast<const uint4*>(&L.qs[(h0 + hh) * D + li * Wave::EPL]);
    Wave st;
    st.init();
    st.run(kb, vb, kv_stride, qp, L.chunks, total * upc, s * SPW + cs, slots, upc, p.block,
           pos, cp, p.scale * kDecLog2e, bias_of);
    st.store(&L.part[wave][0][0]);
    __syncthreads();
    // merge the workgroup's slots (waves cs * WPS + set, in slot order) per head; an empty slot
    // has max = -inf and sum = 0
    float* grp = ws + ((int64_t)b * p.h_kv + r) * gridDim.z * GQ * DS;  // this group's records
    for (int e = tid; e < GQ * D; e += blockDim.x) {
        const int hg = e / D, d = e % D;
        const int set = hg / HPW, hh = hg % HPW;
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < SPW; ++c) mx = fmaxf(mx, L.part[c * WPS + set][hh][D]);
        const float2 ol = merge_parts([&](int c) { return &L.part[c * WPS + set][hh][0]; }, SPW, D, d);
        float* out = grp + ((int64_t)s * GQ + hg) * DS;
        handoff_store(out + d, ol.x);
        if (d == 0) {
            handoff_store(out + D, mx);
            handoff_store(out + D + 1, ol.y);
        }
    }

    // take a ticket; the last of the group's np working workgroups merges all partials in order
    const int np = slots / SPW;
    __shared__ int last;
    if (!handoff_last(&tickets[(int64_t)b * p.h_kv + r], (unsigned)np, &last)) return;
    // every partial's (max, sum) into LDS (over the chunk list, no longer needed), then each
    // thread merges its outputs in record order, eight records' loads in flight at a time
    float* ml = reinterpret_cast<float*>(L.chunks);  // [np][GQ][2]
    for (int i = tid; i < np * GQ; i += blockDim.x) {
        const float* pr = grp + (int64_t)i * DS;
        ml[2 * i] = handoff_load(pr + D);
        ml[2 * i + 1] = handoff_load(pr + D + 1);
    }
    __syncthreads();
    T* orow = o + ((int64_t)b * p.h_q + r * GQ) * D;
    for (int e = tid; e < GQ * D; e += blockDim.x) {
        const int hg = e / D, d = e % D;
        float mx = -INFINITY;
        for (int c = 0; c < np; ++c) mx = fmaxf(mx, ml[2 * (c * GQ + hg)]);
        float acc = 0.f, l = 0.f;
        for (int c0 = 0; c0 < np; c0 += 8) {
            float ov[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                ov[j] = c0 + j < np ? handoff_load(grp + ((int64_t)(c0 + j) * GQ + hg) * DS + d) : 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c0 + j >= np) break;
                const float mc = ml[2 * ((c0 + j) * GQ + hg)];
                const float f = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - mx);
                acc = f > 0.f ? fmaf(f, ov[j], acc) : acc;
                l = fmaf(f, ml[2 * ((c0 + j) * GQ + hg) + 1], l);
            }
        }
        store_elem(orow + e, acc / l);
    }
}

// the group's queries into LDS (16-byte loads; visible after the next barrier)
template <typename T, int D, int GQ>
__device__ __forceinline__ void decode_load_q(const T* __restrict__ q, int b, int r,
                                              const AttnParams& p, T* qs) {
    for (int e = threadIdx.x; e < GQ * D * (int)sizeof(T) / 16; e += blockDim.x)
        reinterpret_cast<uint4*>(qs)[e] =
            reinterpret_cast<const uint4*>(q + ((int64_t)b * p.h_q + r * GQ) * D)[e];
}

// Stage 2 from a given mask and bias. The slot-set index is the slowest grid dimension: the
// workgroups every (sequence, group) uses (the first 32 slots) are dispatched first, the extra
// ones for long selections last.
template <typename T, int D, int GQ>
__global__ __launch_bounds__(256) void decode_split_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           const T* __restrict__ v,
                                                           const uint32_t* __restrict__ mask,
                                                           const float* __restrict__ bias,
                                                           float* ws, unsigned* tickets,
                                                           T* __restrict__ o, AttnParams p) {
    __shared__ __align__(16) DecodeLds<T, D, GQ> L;
    const int r = blockIdx.x, b = blockIdx.y, s = blockIdx.z;
    const uint32_t* mrow = mask + ((int64_t)b * p.h_kv + r) * p.nw;
    const float* brow = bias + ((int64_t)b * p.h_kv + r) * p.nc;
    decode_load_q<T, D, GQ>(q, b, r, p, L.qs);
    decode_attend_group<T, D, GQ>(k, v, [&](int i) { return mrow[i]; },
                                  [&](int c) { return brow[c]; }, ws, tickets, o, p, b, r, s, L);
}

// one ticket counter per (sequence, group) at the start of the workspace (so that calls of any
// batch size share the same words), padded to 256 bytes, then the partial records
static size_t decode_ticket_bytes(const AttnParams& p) {
    return ((size_t)p.batch * p.h_kv * sizeof(unsigned) + 255) / 256 * 256;
}

size_t decode_workspace_bytes(const AttnParams& p) {
    return decode_ticket_bytes(p) +
           (size_t)p.batch * p.h_kv * dec_workgroups(p.g) * p.g * (p.head_dim + 4) * sizeof(float);
}

template <typename T, int D>
static void launch_decode_t(const void* q, const void* k, const void* v, const uint32_t* mask,
                            const float* bias, void* o, const AttnParams& p, float* ws,
                            hipStream_t st) {
    unsigned* tickets = reinterpret_cast<unsigned*>(ws);
    ws = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + decode_ticket_bytes(p));
#define DASH_DEC(GG)                                                                           \
    hipLaunchKernelGGL((decode_split_kernel<T, D, GG>), dim3(p.h_kv, p.batch, dec_workgroups(GG)), \
                       dim3(256), 0, st, static_cast<const T*>(q), static_cast<const T*>(k),     \
                       static_cast<const T*>(v), mask, bias, ws, tickets, static_cast<T*>(o), p)
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

// The decode step: [tickets | partial records] as dash_sparse_attn_decode's workspace, then the
// scores [B, H_q, Nc] fp32 that Stage 1 of decode works through.
size_t decode_step_workspace_bytes(const RouteParams& rp, const AttnParams& p) {
    return decode_workspace_bytes(p) + route_workspace_bytes(rp, kF32);
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v, int dt,
                              const float* kbar, const RouteParams& rp, const AttnParams& p,
                              uint32_t* mask, float* bias, void* o, void* ws, hipStream_t st) {
    void* route_ws = static_cast<char*>(ws) + decode_workspace_bytes(p);
    const hipError_t e = launch_block_entmax(q, dt, kbar, rp, mask, bias, nullptr, route_ws, st);
    if (e != hipSuccess) return e;
    return launch_attn_decode(q, k, v, dt, mask, bias, o, p, ws, st);
}

}  // namespace dash
