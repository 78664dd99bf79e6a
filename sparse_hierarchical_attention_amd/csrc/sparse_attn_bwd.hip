// Stage 2 backward for prefill, the selection held fixed ("DashAttention", arXiv 2605.18753v1,
// §3.4 Prop. 1 for the forward; its gradients by the chain rule). With the forward's lse,
//   p_j = exp(scale <q, k_j> + d_c(j) - lse),  dp_j = <dO, v_j>,  ds_j = p_j (dp_j - <dO, O>),
//   dQ = scale sum_j ds_j k_j,  dK_j = scale sum ds_j q,  dV_j = sum p_j dO,
// where <dO, O> = sum_j p_j dp_j is summed from the probabilities in fp32 rather than read from
// the stored O: O's rounding to bf16 (2^-9) would enter every ds, and the routing gradient
// downstream multiplies dL/dd by 1 / w, which is large near the edge of a head's support.
//   dL/dd_c = sum of ds_j over chunk c's keys and the group's heads (the chunks below the query's
//   own whose mask bit is set).
// These VALU kernels serve fp32 inputs; bf16 runs on the matrix cores (sparse_attn_bwd_mfma.hip).
// Two kernels, each output element written by one wave (no atomics, deterministic):
//   attn_bwd_dq_kernel, row-parallel: one wave per (token, KV group, set of four heads) walks the
//     token's selection in units of kDecUnit keys (the decode path's per-lane layout: a 16-byte
//     piece of a key row per lane, dot products on packed pairs with DPP row sums) twice: first
//     for <dO, O>, which it leaves for the second kernel, then for dQ and each chunk's dL/dd;
//   attn_bwd_dkv_kernel, column-parallel: one workgroup per (sequence, KV group, chunk), one wave
//     per unit of kDecUnit keys; the tokens that attend the chunk (its own tokens causally, later
//     ones whose mask bit is set) are listed in LDS in blocks, in order, and every wave adds their
//     contributions to its keys' dK and dV.
#include <math.h>

#include "common.h"
#include "decode_common.h"
#include "kernels.h"

namespace dash {

namespace {

constexpr int kBwdScan = 256;  // tokens listed per block of the column scan

// Mask word wd of a row with the bits past the query's own chunk cp cleared and cp's bit set.
__device__ __forceinline__ uint32_t row_word(const uint32_t* mrow, int wd, int cp) {
    uint32_t word = mrow[wd];
    const int hi = cp - 32 * wd;
    if (hi < 31) word &= (2u << hi) - 1u;
    if (hi < 32) word |= 1u << hi;
    return word;
}

}  // namespace

// One pass of a wave over the keys its row attends (the selected chunks below the own chunk cp,
// then cp up to the query t), in units of kDecUnit keys. For every key j and head hh of the wave:
//   p = exp(scale <q, k_j> + d - lse), dpv = <dout, v_j>.
// FINAL = false: returns per head the sum of p dpv (rowsum(dout * o) without o's rounding).
// FINAL = true: ds = p (dpv - dsum[hh]); accumulates scale ds k_j into acc and, per chunk, the
// sum of ds over its keys and the wave's heads, which it hands to emit(c, wave's sum).
template <bool FINAL, typename T, int D, int HPW, class EMIT>
__device__ __forceinline__ void dq_keys(const T* kb, const T* vb, int64_t kv_stride,
                                        const uint32_t* mrow, const float* brow, int t, int cp,
                                        int block, int n, float qk_scale, float scale,
                                        const uint4 (&qp)[HPW], const uint4 (&dp_)[HPW],
                                        const float (&lse2)[HPW], const float (&dsum)[HPW],
                                        float (&out)[HPW], float (&acc)[HPW][16 / sizeof(T)],
                                        EMIT emit) {
    using W = DecodeWave<T, D, HPW>;
    constexpr int EPL = W::EPL, LPK = W::LPK, KPI = W::KPI, NI = W::NI;
    const int lane = threadIdx.x & 63;
    const int seg = lane / LPK, li = lane % LPK;
    for (int wd = 0; wd <= cp / 32; ++wd) {
        uint32_t word = row_word(mrow, wd, cp);
        while (word) {
            const int c = 32 * wd + __builtin_ctz(word);
            word &= word - 1u;
            const bool diag = c == cp;
            const float off = diag ? 0.f : brow[c] * kDecLog2e;
            const int kend = diag ? t + 1 : min((c + 1) * block, n);
            float db = 0.f;
            for (int k0 = c * block; k0 < kend; k0 += kDecUnit) {
                uint4 kr[NI], vr[NI];
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int key = min(k0 + i * KPI + seg, kend - 1);  // rows past the end: clamped
                    kr[i] = *reinterpret_cast<const uint4*>(kb + key * kv_stride);
                    vr[i] = *reinterpret_cast<const uint4*>(vb + key * kv_stride);
                }
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const bool valid = k0 + i * KPI + seg < kend;
                    float kf[EPL];
                    if (FINAL) unpack(kr[i], kf);
#pragma unroll
                    for (int hh = 0; hh < HPW; ++hh) {
                        const float sc = seg_sum<LPK>(piece_dot(qp[hh], kr[i], T()));
                        const float dpv = seg_sum<LPK>(piece_dot(dp_[hh], vr[i], T()));
                        const float pr = valid ? __builtin_amdgcn_exp2f(fmaf(sc, qk_scale, off) - lse2[hh]) : 0.f;
                        if (!FINAL) {
                            out[hh] = fmaf(pr, dpv, out[hh]);
                        } else {
                            const float ds = pr * (dpv - dsum[hh]);
                            db += ds;
#pragma unroll
                            for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(ds * scale, kf[e], acc[hh][e]);
                        }
                    }
                }
            }
            if (FINAL && !diag) {
                // every lane of a key row's segment holds the same ds: count each row once
                db = li == 0 ? db : 0.f;
#pragma unroll
                for (int o2 = LPK; o2 < 64; o2 <<= 1) db += __shfl_xor(db, o2, 64);
                emit(c, db);
            }
        }
    }
    if (!FINAL) {
        // every lane of a segment holds its segment's sum: adding across the segments leaves
        // the row's total in every lane
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            float v = out[hh];
#pragma unroll
            for (int o2 = LPK; o2 < 64; o2 <<= 1) v += __shfl_xor(v, o2, 64);
            out[hh] = v;
        }
    }
}

template <typename T, int D, int GQ>
__global__ __launch_bounds__(64 * dec_waves_per_slot(GQ)) void attn_bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ lse, const T* __restrict__ dout, const uint32_t* __restrict__ mask,
    const float* __restrict__ bias, float* __restrict__ dq, float* __restrict__ dbias,
    float* __restrict__ drow, AttnParams p) {
    constexpr int HPW = dec_heads_per_wave(GQ);
    using W = DecodeWave<T, D, HPW>;
    constexpr int EPL = W::EPL, LPK = W::LPK;
    __shared__ float dbw[16];
    const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane / LPK, li = lane % LPK;
    const int h0 = wave * HPW;  // first head of this wave within the group
    const int n = p.n_kv;
    const int cp = t / p.block;
    const int64_t row = (int64_t)b * n + t;
    const uint32_t* mrow = mask + (row * p.h_kv + r) * p.nw;
    const float* brow = bias + (row * p.h_kv + r) * p.nc;
    const int64_t kv_stride = (int64_t)p.h_kv * D;
    const T* kb = k + (int64_t)b * n * kv_stride + (int64_t)r * D + li * EPL;
    const T* vb = v + (int64_t)b * n * kv_stride + (int64_t)r * D + li * EPL;
    const float qk_scale = p.scale * kDecLog2e;

    if (dbias) {  // the row's entries that no selected chunk writes below
        for (int c = threadIdx.x; c < p.nc; c += blockDim.x)
            if (c >= cp || !((mrow[c >> 5] >> (c & 31)) & 1u)) dbias[(row * p.h_kv + r) * p.nc + c] = 0.f;
    }

    uint4 qp[HPW], dp_[HPW];
    float dsum[HPW], lse2[HPW];
    float acc[HPW][EPL];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const int64_t qi = (row * p.h_q + r * GQ + h0 + hh) * D + li * EPL;
        qp[hh] = *reinterpret_cast<const uint4*>(q + qi);
        dp_[hh] = *reinterpret_cast<const uint4*>(dout + qi);
        lse2[hh] = lse[row * p.h_q + r * GQ + h0 + hh] * kDecLog2e;
        dsum[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
    }
    auto no_emit = [](int, float) {};
    // pass 1: rowsum(dout * o) = sum_j p_j <dout, v_j>, from the probabilities themselves
    dq_keys<false, T, D, HPW>(kb, vb, kv_stride, mrow, brow, t, cp, p.block, n, qk_scale, p.scale,
                              qp, dp_, lse2, dsum, dsum, acc, no_emit);
    if (seg == 0 && li == 0) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) drow[row * p.h_q + r * GQ + h0 + hh] = dsum[hh];
    }
    // pass 2: ds, dq and dL/dd of the selected chunks
    float unused[HPW];
    auto emit = [&](int c, float db) {
        if (!dbias) return;
        if (GQ > 4) {
            // the group's other head sets are other waves: add them in wave order in LDS
            if (lane == 0) dbw[wave] = db;
            __syncthreads();
            if (threadIdx.x == 0) {
                float s = 0.f;
                for (int w2 = 0; w2 < (int)(blockDim.x >> 6); ++w2) s += dbw[w2];
                dbias[(row * p.h_kv + r) * p.nc + c] = s;
            }
            __syncthreads();
        } else if (lane == 0) {
            dbias[(row * p.h_kv + r) * p.nc + c] = db;
        }
    };
    dq_keys<true, T, D, HPW>(kb, vb, kv_stride, mrow, brow, t, cp, p.block, n, qk_scale, p.scale,
                             qp, dp_, lse2, dsum, unused, acc, emit);
    // fold the wave's key-row segments (lanes l, l + LPK, ... hold the same dimensions)
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
        for (int o2 = LPK; o2 < 64; o2 <<= 1)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], o2, 64);
    if (seg == 0) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            float* out = dq + (row * p.h_q + r * GQ + h0 + hh) * D + li * EPL;
#pragma unroll
            for (int e = 0; e < EPL; e += 4)
                *reinterpret_cast<float4*>(out + e) = make_float4(acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]);
        }
    }
}

template <typename T, int D, int GQ>
__global__ __launch_bounds__(512) void attn_bwd_dkv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ lse, const T* __restrict__ dout, const uint32_t* __restrict__ mask,
    const float* __restrict__ bias, const float* __restrict__ drow, float* __restrict__ dk,
    float* __restrict__ dv, AttnParams p) {
    using W = DecodeWave<T, D, 1>;
    constexpr int EPL = W::EPL, LPK = W::LPK, KPI = W::KPI, NI = W::NI;
    __shared__ int list[kBwdScan];
    __shared__ int wtot[8];
    const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int seg = lane / LPK, li = lane % LPK;
    const int n = p.n_kv;
    const int c0 = c * p.block, cend = min(c0 + p.block, n);
    const int k0 = c0 + wave * kDecUnit;  // this wave's unit
    const int64_t kv_stride = (int64_t)p.h_kv * D;
    const T* kb = k + (int64_t)b * n * kv_stride + (int64_t)r * D + li * EPL;
    const T* vb = v + (int64_t)b * n * kv_stride + (int64_t)r * D + li * EPL;
    const float qk_scale = p.scale * kDecLog2e;

    uint4 kr[NI], vr[NI];
    float kf[NI][EPL], vf[NI][EPL];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int key = min(k0 + i * KPI + seg, cend - 1);
        kr[i] = *reinterpret_cast<const uint4*>(kb + key * kv_stride);
        vr[i] = *reinterpret_cast<const uint4*>(vb + key * kv_stride);
        unpack(kr[i], kf[i]);
        unpack(vr[i], vf[i]);
    }
    float gk[NI][EPL], gv[NI][EPL];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            gk[i][e] = 0.f;
            gv[i][e] = 0.f;
        }

    // the tokens that attend chunk c: its own (t >= c0, causally) and later ones whose bit is set
    for (int t0 = c0; t0 < n; t0 += kBwdScan) {
        int sel = 0;
        const int t = t0 + tid;
        if (tid < kBwdScan && t < n) {
            const int ct = t / p.block;
            const uint32_t* mrow = mask + (((int64_t)b * n + t) * p.h_kv + r) * p.nw;
            sel = ct == c || (ct > c && ((mrow[c >> 5] >> (c & 31)) & 1u));
        }
        // ordered compaction of the block's attending tokens into list[]
        const uint64_t bal = __ballot(sel);
        if (lane == 0) wtot[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
        for (int w2 = 0; w2 < nwaves; ++w2) {
            before += w2 < wave ? wtot[w2] : 0;
            total += wtot[w2];
        }
        if (sel) list[before + __popcll(bal & ((1ull << lane) - 1ull))] = t;
        __syncthreads();
        if (k0 < cend) {
            for (int j = 0; j < total; ++j) {
                const int tt = list[j];
                const int64_t row = (int64_t)b * n + tt;
                const bool diag = tt / p.block == c;
                const float off = diag ? 0.f : bias[(row * p.h_kv + r) * p.nc + c] * kDecLog2e;
#pragma unroll 1
                for (int hh = 0; hh < GQ; ++hh) {
                    const int64_t qi = (row * p.h_q + r * GQ + hh) * D + li * EPL;
                    const uint4 qp = *reinterpret_cast<const uint4*>(q + qi);
                    const uint4 dp_ = *reinterpret_cast<const uint4*>(dout + qi);
                    const float lse2 = lse[row * p.h_q + r * GQ + hh] * kDecLog2e;
                    const float dsum = drow[row * p.h_q + r * GQ + hh];
                    float qf[EPL], df[EPL];
                    unpack(qp, qf);
                    unpack(dp_, df);
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        const int key = k0 + i * KPI + seg;
                        const bool valid = key < cend && key <= tt;
                        const float s = seg_sum<LPK>(piece_dot(qp, kr[i], T()));
                        const float dpv = seg_sum<LPK>(piece_dot(dp_, vr[i], T()));
                        const float pr = valid ? __builtin_amdgcn_exp2f(fmaf(s, qk_scale, off) - lse2) : 0.f;
                        const float ds = pr * (dpv - dsum) * p.scale;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) {
                            gv[i][e] = fmaf(pr, df[e], gv[i][e]);
                            gk[i][e] = fmaf(ds, qf[e], gk[i][e]);
                        }
                    }
                }
            }
        }
        __syncthreads();  // list[] is refilled by the next block
    }
    if (k0 < cend) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = k0 + i * KPI + seg;
            if (key >= cend) continue;
            const int64_t base = (((int64_t)b * n + key) * p.h_kv + r) * D + li * EPL;
#pragma unroll
            for (int e = 0; e < EPL; e += 4) {
                *reinterpret_cast<float4*>(dk + base + e) = make_float4(gk[i][e], gk[i][e + 1], gk[i][e + 2], gk[i][e + 3]);
                *reinterpret_cast<float4*>(dv + base + e) = make_float4(gv[i][e], gv[i][e + 1], gv[i][e + 2], gv[i][e + 3]);
            }
        }
    }
}

size_t attn_backward_workspace_bytes(const AttnParams& p) {
    return (size_t)p.batch * p.n_q * p.h_q * sizeof(float);
}

template <typename T, int D, int GQ>
static void launch_bwd_t(const void* q, const void* k, const void* v,
                         const float* lse, const void* dout, const uint32_t* mask,
                         const float* bias, float* dq, float* dk, float* dv, float* dbias,
                         float* drow, const AttnParams& p, hipStream_t st) {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, GQ>), dim3(p.n_q, p.h_kv, p.batch),
                       dim3(64 * dec_waves_per_slot(GQ)), 0, st, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), lse,
                       static_cast<const T*>(dout), mask, bias, dq, dbias, drow, p);
    const int waves = div_up(p.block, kDecUnit);
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, D, GQ>), dim3(p.nc, p.h_kv, p.batch),
                       dim3(64 * (waves < 4 ? 4 : waves)), 0, st, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), lse,
                       static_cast<const T*>(dout), mask, bias, drow, dk, dv, p);
}

template <typename T, int D>
static void launch_bwd_d(const void* q, const void* k, const void* v,
                         const float* lse, const void* dout, const uint32_t* mask,
                         const float* bias, float* dq, float* dk, float* dv, float* dbias,
                         float* drow, const AttnParams& p, hipStream_t st) {
    switch (p.g) {
        case 1: launch_bwd_t<T, D, 1>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, drow, p, st); break;
        case 2: launch_bwd_t<T, D, 2>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, drow, p, st); break;
        case 4: launch_bwd_t<T, D, 4>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, drow, p, st); break;
        case 8: launch_bwd_t<T, D, 8>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, drow, p, st); break;
        default: launch_bwd_t<T, D, 16>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, drow, p, st); break;
    }
}

hipError_t launch_attn_backward(const void* q, const void* k, const void* v, const float* lse,
                                const void* dout, int dt, const uint32_t* mask,
                                const float* bias, float* dq, float* dk, float* dv, float* dbias,
                                const AttnParams& p, void* ws, hipStream_t st) {
    // bf16 runs on the matrix cores (sparse_attn_bwd_mfma.hip); fp32 here
    if (dt == kBF16) return launch_attn_backward_mfma(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, p, ws, st);
    float* drow = static_cast<float*>(ws);
    if (p.head_dim == 64) launch_bwd_d<float, 64>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, drow, p, st);
    else launch_bwd_d<float, 128>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, drow, p, st);
    return hipGetLastError();
}

}  // namespace dash
