// Per-wave pieces of Stage 2 for one new token per sequence ("DashAttention",
// arXiv 2605.18753v1, §3.4 Prop. 1, §3.5 "split-KV variant"), shared by the split decode kernel
// and the fused decode step.
//
// The keys a (sequence, group) attends to -- those of its selected chunks and of its own chunk,
// in increasing order -- are cut into units of kDecUnit keys. A wave takes units of the list and
// holds their keys and values in registers: a 16-byte load per lane holds a piece of one key
// row, a row of D elements spans D / 8 (bf16) or D / 4 (fp32) lanes, and one load instruction
// covers 64 / (that many) whole rows. Dot products run on packed bf16 pairs (v_dot2) and finish
// with DPP sums inside each row's lanes; the online softmax keeps one running maximum per head
// (log2 domain) and per-lane partial sums until the wave folds its rows at the end.
#pragma once

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dash {

constexpr int kDecUnit = 16;       // keys per unit
constexpr int kDecMaxWords = 256;  // 8192 chunks
constexpr float kDecLog2e = 1.4426950408889634f;

// Sum over aligned groups of LANES consecutive lanes (8, 16 or 32); every lane gets its group's sum.
template <int LANES>
__device__ __forceinline__ float seg_sum(float v) {
    v += dpp_f<0xb1, 0xf>(0.f, v);       // pairs
    v += dpp_f<0x4e, 0xf>(0.f, v);       // quads
    v += dpp_f<0x141, 0xf>(0.f, v);      // half rows (8 lanes)
    if (LANES >= 16) v += dpp_f<0x140, 0xf>(0.f, v);  // rows (16 lanes)
    if (LANES >= 32) v = rowpair_sum(v);
    return v;
}

// Sum / maximum over the lanes l, l + LANES, l + 2 LANES, ... (LANES = 8, 16 or 32): the lanes of a
// wave that hold the same position of different key rows. Every lane gets the result.
template <int LANES>
__device__ __forceinline__ float cross_sum(float v) {
    if (LANES == 8) v += dpp_f<0x128, 0xf>(0.f, v);  // row_ror:8, the other half of the row
    if (LANES <= 16) v = rowpair_sum(v);
    return halves_sum(v);
}
template <int LANES>
__device__ __forceinline__ float cross_max(float v) {
    if (LANES == 8) v = fmaxf(v, dpp_f<0x128, 0xf>(-INFINITY, v));
    if (LANES <= 16) v = rowpair_max(v);
    return halves_max(v);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// <q, k> over one 16-byte piece: q as 8 bf16 (4 packed pairs) or 4 floats.
__device__ __forceinline__ float piece_dot(const uint4& qp, const uint4& kp, bf16_t) {
    float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp.x),
                                              __builtin_bit_cast(bf16x2_t, kp.x), 0.f, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp.y),
                                        __builtin_bit_cast(bf16x2_t, kp.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp.z),
                                        __builtin_bit_cast(bf16x2_t, kp.z), d, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp.w),
                                           __builtin_bit_cast(bf16x2_t, kp.w), d, false);
}
__device__ __forceinline__ float piece_dot(const uint4& qp, const uint4& kp, float) {
    float d = __uint_as_float(qp.x) * __uint_as_float(kp.x);
    d = fmaf(__uint_as_float(qp.y), __uint_as_float(kp.y), d);
    d = fmaf(__uint_as_float(qp.z), __uint_as_float(kp.z), d);
    return fmaf(__uint_as_float(qp.w), __uint_as_float(kp.w), d);
}

// Elements of a 16-byte piece as floats.
__device__ __forceinline__ void unpack(const uint4& u, float (&f)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack(const uint4& u, float (&f)[4]) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
}

__host__ __device__ constexpr int dec_heads_per_wave(int g) { return g > 4 ? 4 : g; }
__host__ __device__ constexpr int dec_waves_per_slot(int g) { return g > 4 ? g / 4 : 1; }

// The chunks with their mask bit set among 0 .. cp, in increasing order, into chunks[]; returns
// their number (the same in every thread). Bits past cp are ignored and cp's own bit counts as
// set. word_of(i) reads mask word i (i <= cp / 32). Uses every thread of the workgroup
// (cp / 32 + 1 <= blockDim.x) and wtot[blockDim.x / 64] of LDS; ends with a barrier.
template <class WORD>
__device__ __forceinline__ int chunk_list(WORD word_of, int cp, int* wtot, uint16_t* chunks) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int nwr = cp / 32 + 1;
    uint32_t word = 0;
    if (tid < nwr) {
        word = word_of(tid);
        const int hi = cp - 32 * tid;
        if (hi < 31) word &= (2u << hi) - 1u;
        if (hi < 32) word |= 1u << hi;
    }
    const int cnt = __popc(word);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int rank = incl - cnt, total = 0;
    for (int i = 0; i < nwaves; ++i) {
        rank += i < wave ? wtot[i] : 0;
        total += wtot[i];
    }
    while (word) {
        const int bit = __builtin_ctz(word);
        word &= word - 1u;
        chunks[rank++] = (uint16_t)(32 * tid + bit);
    }
    __syncthreads();
    return total;
}

// One wave's running softmax state over HPW heads of a group.
template <typename T, int D, int HPW>
struct DecodeWave {
    static constexpr int EPL = 16 / sizeof(T);  // elements per 16-byte piece
    static constexpr int LPK = D / EPL;         // lanes per key row
    static constexpr int KPI = 64 / LPK;        // key rows per load instruction
    static constexpr int NI = kDecUnit / KPI;   // loads per tensor and unit
    static_assert(kDecUnit % KPI == 0 && LPK >= 8 && LPK <= 32, "unsupported head size");

    float acc[HPW][EPL], m_run[HPW], l_run[HPW];

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            m_run[hh] = -INFINITY;
            l_run[hh] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
        }
    }

    // Units u0, u0 + ustep, ... below n_units of the list chunks[] (increasing; the query's own
    // chunk cp last, its keys up to pos). kb / vb: this lane's piece of key row 0 of the
    // (sequence, KV head); rows kv_stride elements apart. bias_of(c): d of chunk c < cp.
    template <class BIAS>
    __device__ __forceinline__ void run(const T* kb, const T* vb, int64_t kv_stride,
                                        const uint4 (&qp)[HPW], const uint16_t* chunks,
                                        int n_units, int u0, int ustep, int upc, int block,
                                        int pos, int cp, float qk_scale, BIAS bias_of) {
        const int seg = (threadIdx.x & 63) / LPK;
        for (int u = u0; u < n_units; u += ustep) {
            const int c = chunks[u / upc];
            const int k0 = c * block + (u % upc) * kDecUnit;
            const bool diag = c == cp;
            const int kend = diag ? pos + 1 : min((c + 1) * block, k0 + kDecUnit);
            if (k0 >= kend) continue;  // a unit of the own chunk past the query
            const float off = diag ? 0.f : bias_of(c) * kDecLog2e;
            uint4 kr[NI], vr[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int key = min(k0 + i * KPI + seg, kend - 1);  // rows past the end: clamped
                kr[i] = *reinterpret_cast<const uint4*>(kb + key * kv_stride);
                vr[i] = *reinterpret_cast<const uint4*>(vb + key * kv_stride);
            }
            float sc[HPW][NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const bool valid = k0 + i * KPI + seg < kend;
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    const float d = seg_sum<LPK>(piece_dot(qp[hh], kr[i], T()));
                    sc[hh][i] = valid ? fmaf(d, qk_scale, off) : -INFINITY;
                }
            }
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                float mx = sc[hh][0];
#pragma unroll
                for (int i = 1; i < NI; ++i) mx = fmaxf(mx, sc[hh][i]);
                mx = cross_max<LPK>(mx);
                const float m_new = fmaxf(m_run[hh], mx);
                const float corr = __builtin_amdgcn_exp2f(m_run[hh] - m_new);
                m_run[hh] = m_new;
                float l = l_run[hh] * corr;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    sc[hh][i] = __builtin_amdgcn_exp2f(sc[hh][i] - m_new);
                    l += sc[hh][i];
                }
                l_run[hh] = l;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[hh][e] *= corr;
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                float vf[EPL];
                unpack(vr[i], vf);
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(sc[hh][i], vf[e], acc[hh][e]);
            }
        }
    }

    // Fold the wave's key rows (lanes l, l + LPK, ... hold the same dimensions) and store the
    // partial (unnormalised output, max, sum) of each head into part + hh * (D + 4).
    __device__ __forceinline__ void store(float* part) {
        const int lane = threadIdx.x & 63;
        const int seg = lane / LPK, li = lane % LPK;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            l_run[hh] = cross_sum<LPK>(l_run[hh]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[hh][e] = cross_sum<LPK>(acc[hh][e]);
        }
        if (seg == 0) {
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                float* pr = part + hh * (D + 4);
#pragma unroll
                for (int e = 0; e < EPL; e += 4)
                    *reinterpret_cast<float4*>(&pr[li * EPL + e]) =
                        make_float4(acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]);
                if (li == 0) {
                    pr[D] = m_run[hh];
                    pr[D + 1] = l_run[hh];
                }
            }
        }
    }
};

// Merge of nparts partial records (unnormalised output, max, sum; max = -inf for an empty one)
// in order: returns (sum_i f_i o_i[d], sum_i f_i l_i) with f_i = 2^(m_i - max m).
template <class REC>
__device__ __forceinline__ float2 merge_parts(REC rec, int nparts, int D, int d) {
    float mx = -INFINITY;
    for (int c = 0; c < nparts; ++c) mx = fmaxf(mx, rec(c)[D]);
    float o = 0.f, l = 0.f;
    for (int c = 0; c < nparts; ++c) {
        const float* pr = rec(c);
        const float f = pr[D] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pr[D] - mx);
        o = f > 0.f ? fmaf(f, pr[d], o) : o;
        l = fmaf(f, pr[D + 1], l);
    }
    return make_float2(o, l);
}

}  // namespace dash
