// Stage 2 backward for prefill on bf16 MFMA ("DashAttention", arXiv 2605.18753v1, §3.4 Prop. 1,
// differentiated with the selection held fixed), gfx950. The same gradients as the VALU kernels
// of sparse_attn_bwd.hip:
//   p_j = exp(scale <q, k_j> + d_c(j) - lse), dp_j = <dO, v_j>, ds_j = p_j (dp_j - Delta),
//   Delta = sum_j p_j dp_j (summed in fp32 from the probabilities, not from the stored O),
//   dQ = scale sum_j ds_j k_j, dK_j = scale sum ds_j q, dV_j = sum p_j dO, dL/dd_c = sum of ds_j
//   over chunk c's keys and the group's heads.
// The score and dP products accumulate exact bf16 products in fp32, so p, dp, ds, Delta and
// dL/dd carry fp32 rounding only; the products that take p or ds as an operand (dV, dK, dQ)
// round them to bf16, as attention's forward rounds p for P V.
//
// attn_bwd_dq_mfma_kernel, row-parallel, one workgroup (4 waves) per 128 rows of one (sequence,
// KV group): T = 128 / g consecutive tokens times the g heads, as the forward kernel tiles them.
// It walks the union of its tokens' selected chunks twice, K and V tiles of up to 64 keys staged
// through LDS (double-buffered):
//   pass 1: S^T = K Q^T and dP^T = V dO^T (v_mfma_f32_32x32x16_bf16, Q and dO rows held as B
//           operands), p from the stored lse, Delta += p dp;
//   pass 2: the same products, ds = p (dp - Delta), dL/dd per (token, chunk) summed over the
//           chunk's keys and the token's heads, and dQ^T += K^T dS^T with K^T read through
//           transposing LDS loads (ds_read_b64_tr_b16), dS^T straight from the accumulator.
// Two workgroups share a CU (two waves per SIMD, 256 registers each): K and V fragments are read a
// few k-steps ahead of their products rather than all at once, and K^T right at its product.
// attn_bwd_dkv16_mfma_kernel, column-parallel, one workgroup per (sequence, KV group, chunk), one
// wave per 16 keys holding its keys and values as B operands of v_mfma_f32_16x16x32_bf16 (two
// waves fit each SIMD), the chunks of one (sequence, group) on one XCD: the tokens that attend the
// chunk (its own, causally, and later ones whose mask bit is set) are listed in order, their rows
// (token x head) gathered into LDS 64 at a time, and per tile
//   S = Q K^T, dP = dO V^T, p, ds = p (dp - Delta), dV^T += dO^T P, dK^T += Q^T dS,
// with dO^T and Q^T read through transposing LDS loads and P, dS from the accumulators.
// Probabilities are formed without branches: a pair that does not attend gets exp2(-inf) = 0
// (branches per element, each waiting on its own LDS read, had cost the dK / dV kernel a fifth
// of its time).
// Each output element is written once, by one lane: deterministic, no atomics.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dash {

namespace {

typedef __bf16 bw_bf16x8 __attribute__((ext_vector_type(8)));
typedef short bw_i16x4 __attribute__((ext_vector_type(4)));
typedef float bw_f32x16 __attribute__((ext_vector_type(16)));
typedef float bw_f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bw_i16x4 bw_lds_i16x4;

constexpr int kBwRows = 128;     // rows (token x head) per workgroup of the dq kernel
constexpr int kBwThreads = 256;
constexpr int kBwMaxWords = 256;  // 8192 chunks
constexpr float kBwLog2e = 1.4426950408889634f;

__device__ __forceinline__ bw_i16x4 bw_read_tr16(const bf16_t* ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (bw_lds_i16x4*)(__attribute__((address_space(3))) void*)(ptr));
}

// A operand (32 dims x 16 rows) of X^T += Y^T Z for Y stored row-major in LDS (stride LS): the
// transposing loads give lane l dimension 32 dt + (l % 32) of the rows 16 ks + 4 G + {0..3} and
// + 8, the order in which the accumulator-derived B operand holds its rows.
template <int LS>
__device__ __forceinline__ bw_bf16x8 tr_operand(const bf16_t* base, int ks, int dt, int lane) {
    const int grp = lane >> 4, kl = lane & 15;
    const int r = 4 * (grp >> 1) + (kl >> 2);
    const int d = 16 * (grp & 1) + 4 * (kl & 3);
    const bf16_t* ptr = base + (16 * ks + r) * LS + 32 * dt + d;
    const bw_i16x4 lo = bw_read_tr16(ptr);
    const bw_i16x4 hi = bw_read_tr16(ptr + 8 * LS);
    return __builtin_bit_cast(bw_bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand (16 dims x 32 rows) of X^T += Y^T Z on v_mfma_f32_16x16x32_bf16 for Y stored
// row-major in LDS (stride LS): lane l receives dimension 16 db + (l % 16) of the rows
// 32 kb + 4 (l / 16) + {0..3} and + 16, the order in which the B operand built from two 16-row
// score accumulators holds its rows.
template <int LS>
__device__ __forceinline__ bw_bf16x8 tr_operand16(const bf16_t* base, int kb, int db, int lane) {
    const int grp = lane >> 4, kl = lane & 15;
    const bf16_t* ptr = base + (32 * kb + 4 * grp + (kl >> 2)) * LS + 16 * db + 4 * (kl & 3);
    const bw_i16x4 lo = bw_read_tr16(ptr);
    const bw_i16x4 hi = bw_read_tr16(ptr + 16 * LS);
    return __builtin_bit_cast(bw_bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace

template <int D, int BLK, int GQ>
__global__ __launch_bounds__(kBwThreads, 2) void attn_bwd_dq_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ lse, const bf16_t* __restrict__ dout,
    const uint32_t* __restrict__ mask, const float* __restrict__ bias, float* __restrict__ dq,
    float* __restrict__ dbias, float* __restrict__ delta, AttnParams p, int n_tiles) {
    constexpr int T = kBwRows / GQ;          // tokens per workgroup
    constexpr int KT = BLK < 64 ? BLK : 64;  // keys per LDS tile
    constexpr int NSUB = BLK / KT;
    // K / V row stride in LDS (elements): the LDS has 64 banks and serves a 128-bit read 16 lanes
    // per cycle; at D + 24 the 16 rows a lane group reads fall on distinct banks (at D + 16 two
    // rows shared each bank), and the transposing reads stay two-way as before
    constexpr int LS = D + 24;
    constexpr int MT = KT / 32;              // 32-key M-tiles
    constexpr int DT = D / 32;               // 32-dim M-tiles of dQ^T
    constexpr int LOADS = KT * (D / 8) / kBwThreads;
    static_assert(LOADS >= 1, "tile too small");
    __shared__ __align__(16) bf16_t Ks[2][KT * LS];
    __shared__ __align__(16) bf16_t Vs[2][KT * LS];
    __shared__ uint32_t uni[kBwMaxWords];

    int gr;
    {
        const int bh = p.batch * p.h_kv, x = blockIdx.x;
        gr = bh % 8 == 0 ? (x % 8) + 8 * ((x / 8) % (bh / 8)) : x % bh;
    }
    const int tile = n_tiles - 1 - blockIdx.x / (p.batch * p.h_kv);
    const int b = gr / p.h_kv, r = gr % p.h_kv;
    const int n = p.n_kv;
    const int tile0 = tile * T;
    const int tile_end = min(tile0 + T, n);
    const int c_first = tile0 / BLK, c_last = (tile_end - 1) / BLK;
    const int nwt = c_last / 32 + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, G = lane >> 5;
    const int row = wave * 32 + j;
    const int tok = row / GQ, hl = row % GQ;
    const int pos = tile0 + tok;
    const bool valid = pos < n;
    const int cpos = pos / BLK;
    const int64_t qrow = (int64_t)b * n + pos;
    const int64_t qrow_c = (int64_t)b * n + min(pos, n - 1);  // rows past the end read the last
    const uint32_t* mrow = mask + (qrow_c * p.h_kv + r) * p.nw;
    const float* brow = bias + (qrow_c * p.h_kv + r) * p.nc;
    // this row's mask word and bias for a chunk, loaded without a branch (chunk clamped into
    // range) one tile ahead of their use, so that they have landed by then
    auto row_view = [&](int cc, uint32_t& mw, float& dv) {
        const int cq = valid ? min(cc, cpos) : 0;
        mw = mrow[cq >> 5];
        dv = brow[cq];
    };

    // dL/dd entries no selected chunk writes: chunks at or past each token's own, and unselected
    if (dbias) {
        for (int idx = tid; idx < T * p.nc; idx += kBwThreads) {
            const int t = idx / p.nc, c = idx % p.nc;
            const int ps = tile0 + t;
            if (ps >= n) continue;
            const int64_t rr = ((int64_t)b * n + ps) * p.h_kv + r;
            if (c >= ps / BLK || !((mask[rr * p.nw + (c >> 5)] >> (c & 31)) & 1u)) dbias[rr * p.nc + c] = 0.f;
        }
    }
    // union of the tile tokens' selections (bits past a token's own chunk ignored)
    for (int w = tid; w < nwt; w += kBwThreads) uni[w] = 0u;
    __syncthreads();
    for (int idx = tid; idx < T * nwt; idx += kBwThreads) {
        const int t = idx / nwt, w = idx % nwt;
        const int ps = tile0 + t;
        if (ps >= n) continue;
        const int hi = ps / BLK - 32 * w;
        if (hi < 0) continue;
        uint32_t word = mask[(((int64_t)b * n + ps) * p.h_kv + r) * p.nw + w];
        if (hi < 31) word &= (2u << hi) - 1u;
        if (hi < 32) word |= 1u << hi;
        if (word) atomicOr(&uni[w], word);
    }
    __syncthreads();
    auto next_chunk = [&](int c) -> int {
        int w = (c + 1) >> 5;
        if (w >= nwt) return -1;
        uint32_t word = uni[w] & (~0u << ((c + 1) & 31));
        while (true) {
            if (word) return 32 * w + __builtin_ctz(word);
            if (++w >= nwt) return -1;
            word = uni[w];
        }
    };

    // this wave's Q and dO rows as B operands (k-slot order shared with the K / V row reads)
    bw_bf16x8 qf[D / 16], df[D / 16];
    {
        const int64_t off = (qrow * p.h_q + r * GQ + hl) * D + 8 * G;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const uint4 uq = valid ? *reinterpret_cast<const uint4*>(q + off + 16 * s) : make_uint4(0, 0, 0, 0);
            const uint4 ud = valid ? *reinterpret_cast<const uint4*>(dout + off + 16 * s) : make_uint4(0, 0, 0, 0);
            qf[s] = __builtin_bit_cast(bw_bf16x8, uq);
            df[s] = __builtin_bit_cast(bw_bf16x8, ud);
        }
    }
    const float lse2 = valid ? lse[qrow * p.h_q + r * GQ + hl] * kBwLog2e : 0.f;
    const float qk_scale = p.scale * kBwLog2e;
    const int64_t kv_row_stride = (int64_t)p.h_kv * D;
    const bf16_t* kbase = k + (int64_t)b * n * kv_row_stride + (int64_t)r * D;
    const bf16_t* vbase = v + (int64_t)b * n * kv_row_stride + (int64_t)r * D;

    uint4 pk[LOADS], pv[LOADS];
    auto fetch = [&](int c, int sub) {
        const int key0 = c * BLK + sub * KT;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int e = tid + i * kBwThreads;
            const int kk = e / (D / 8), d8 = e % (D / 8);
            const int key = key0 + kk;
            pk[i] = make_uint4(0, 0, 0, 0);
            pv[i] = make_uint4(0, 0, 0, 0);
            if (key < n) {
                pk[i] = *reinterpret_cast<const uint4*>(kbase + key * kv_row_stride + 8 * d8);
                pv[i] = *reinterpret_cast<const uint4*>(vbase + key * kv_row_stride + 8 * d8);
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int e = tid + i * kBwThreads;
            const int kk = e / (D / 8), d8 = e % (D / 8);
            *reinterpret_cast<uint4*>(&Ks[buf][kk * LS + 8 * d8]) = pk[i];
            *reinterpret_cast<uint4*>(&Vs[buf][kk * LS + 8 * d8]) = pv[i];
        }
    };

    float dsum = 0.f;   // pass 1: this lane's part of Delta
    float Delta = 0.f;  // pass 2: the row's Delta
    float dbpart = 0.f; // pass 2: this lane's part of dL/dd of the current chunk
    bw_f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = bw_f32x16{};

    // the two passes as separate code (PASS is a compile-time constant in each), so that the dQ
    // accumulators live in the second only
    auto walk = [&](auto pass_c) __attribute__((always_inline)) {
        constexpr int pass = decltype(pass_c)::value;
        int c = next_chunk(-1), sub = 0;  // every tile has at least its own chunk
        uint32_t mw;
        float dv;
        row_view(c, mw, dv);
        fetch(c, 0);
        stash(0);
        __syncthreads();
        for (int buf = 0; c >= 0; buf ^= 1) {
            const int key0 = c * BLK + sub * KT;
            const int c_nx = sub + 1 < NSUB ? c : next_chunk(c);
            const int sub_nx = sub + 1 < NSUB ? sub + 1 : 0;
            if (c_nx >= 0) fetch(c_nx, sub_nx);
            uint32_t mw_nx;
            float dv_nx;
            row_view(c_nx >= 0 ? c_nx : c, mw_nx, dv_nx);
            const bool sel = valid && c <= cpos && (c == cpos || ((mw >> (c & 31)) & 1u));
            const float off = sel ? (c == cpos ? 0.f : dv * kBwLog2e) - lse2 : -INFINITY;
            const bool causal = c >= c_first;
            // a wave none of whose rows selected the tile adds nothing (p = 0 on every key)
            if (__any(sel)) {
                // per 32-key M-tile: S^T = K Q^T, dP^T = V dO^T, then p (and in pass 2 ds and the
                // two 16-key k-steps of dQ^T += K^T dS^T that this M-tile feeds); the M-tiles are
                // not unrolled, which leaves fewer registers spilled (17.5 against 18.2 ms for the
                // Stage 2 backward at 32K)
    #pragma unroll 1
                for (int mt = 0; mt < MT; ++mt) {
                    // the M-tile's K and V rows, each k-step's read one step ahead of its products
                    // (two waves share each SIMD, so the other wave covers what latency remains;
                    // a ring of two holds fewer registers than three, 17.2 against 17.4 ms)
                    constexpr int KSN = D / 16;
                    bw_bf16x8 ka[2], va[2];
                    auto kvread = [&](int ks) __attribute__((always_inline)) {
                        ka[ks % 2] = *reinterpret_cast<const bw_bf16x8*>(&Ks[buf][(32 * mt + j) * LS + 16 * ks + 8 * G]);
                        va[ks % 2] = *reinterpret_cast<const bw_bf16x8*>(&Vs[buf][(32 * mt + j) * LS + 16 * ks + 8 * G]);
                    };
                    kvread(0);
                    bw_f32x16 s = bw_f32x16{}, dp = bw_f32x16{};
    #pragma unroll
                    for (int ks = 0; ks < KSN; ++ks) {
                        if (ks + 1 < KSN) kvread(ks + 1);
                        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % 2], qf[ks], s, 0, 0, 0);
                        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks % 2], df[ks], dp, 0, 0, 0);
                    }
                    // p = exp(scale s + d - lse) on the row's selected, causal keys; 0 elsewhere
                    // (only tiles that hold some row's own chunk compare keys with positions)
                    if (causal) {
    #pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            const int key = key0 + 32 * mt + 8 * (rr >> 2) + 4 * G + (rr & 3);
                            s[rr] = __builtin_amdgcn_exp2f(key > pos ? -INFINITY : fmaf(s[rr], qk_scale, off));
                        }
                    } else {
    #pragma unroll
                        for (int rr = 0; rr < 16; ++rr) s[rr] = __builtin_amdgcn_exp2f(fmaf(s[rr], qk_scale, off));
                    }
                    if (pass == 0) {
    #pragma unroll
                        for (int rr = 0; rr < 16; ++rr) dsum = fmaf(s[rr], dp[rr], dsum);
                    } else {
                        bw_bf16x8 dsf[2];
    #pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            const float ds = s[rr] * (dp[rr] - Delta);
                            dbpart += ds;
                            dsf[rr >> 3][rr & 7] = (__bf16)ds;
                        }
                        // dQ^T += K^T dS^T over k-steps 2 mt and 2 mt + 1
    #pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2)
    #pragma unroll
                            for (int dt = 0; dt < DT; ++dt)
                                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    tr_operand<LS>(Ks[buf], 2 * mt + h2, dt, lane), dsf[h2], acc[dt], 0, 0, 0);
                    }
                }
            }
            if (pass == 1) {
                if (sub == NSUB - 1) {
                    // dL/dd of chunk c: the row's keys (both lane halves), then the token's heads
                    float tot = dbpart + __shfl_xor(dbpart, 32, kWave);
#pragma unroll
                    for (int x = 1; x < GQ; x <<= 1) tot += __shfl_xor(tot, x, kWave);
                    if (dbias && sel && c != cpos && G == 0 && hl == 0)
                        dbias[(qrow * p.h_kv + r) * p.nc + c] = tot;
                    dbpart = 0.f;
                }
            }
            if (c_nx >= 0) stash(buf ^ 1);
            __syncthreads();
            c = c_nx;
            sub = sub_nx;
            mw = mw_nx;
            dv = dv_nx;
        }
        if (pass == 0) Delta = dsum + __shfl_xor(dsum, 32, kWave);
    };
    walk(std::integral_constant<int, 0>{});
    walk(std::integral_constant<int, 1>{});

    if (!valid) return;
    if (G == 0) delta[qrow * p.h_q + r * GQ + hl] = Delta;
    float* orow = dq + (qrow * p.h_q + r * GQ + hl) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int d0 = 32 * dt + 8 * qd + 4 * G;
            *reinterpret_cast<float4*>(orow + d0) =
                make_float4(acc[dt][4 * qd] * p.scale, acc[dt][4 * qd + 1] * p.scale,
                            acc[dt][4 * qd + 2] * p.scale, acc[dt][4 * qd + 3] * p.scale);
        }
}

// dK and dV with one wave per 16 keys on v_mfma_f32_16x16x32_bf16: a wave holds its keys and
// values as B operands (D / 32 registers of 8 bf16 each) and dK^T, dV^T as D / 16 accumulators of
// 16 dims x 16 keys, so that two waves fit each SIMD (one wave per 32 keys on the 32 x 32 product
// needed twice the registers and ran alone on its SIMD). One workgroup per (sequence, KV group,
// chunk), BLK / 16 waves; the attending rows are listed in order and gathered 64 (32 for chunks
// of 32) at a time, and per 32-row k-step kb of a tile
//   S = Q K^T and dP = dO V^T on the two 16-row blocks 2 kb, 2 kb + 1 (A = the rows from LDS),
//   p and ds per element (lane l: key l % 16, rows 4 (l / 16) + {0..3} of each block),
//   dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read through transposing LDS loads and P,
//   dS from the accumulators (rows 4 (l / 16) + {0..3} of both blocks, the order the transposing
//   loads give).
template <int D, int BLK, int GQ>
__global__ __launch_bounds__(4 * BLK, 2) void attn_bwd_dkv16_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ lse, const bf16_t* __restrict__ dout,
    const uint32_t* __restrict__ mask, const float* __restrict__ bias,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv,
    AttnParams p) {
    constexpr int NTH = 4 * BLK;             // one wave per 16 keys
    constexpr int NWV = NTH / 64;
    constexpr int LS = D + 24;               // row stride of the gathered Q / dO rows
    constexpr int RT = BLK >= 64 ? 64 : 32;  // rows (token x head) per tile
    constexpr int KB = RT / 32;              // 32-row k-steps per tile
    constexpr int TPT = RT / GQ;             // tokens per tile
    constexpr int KS = D / 32;               // 32-dim k-steps of S and dP
    constexpr int DB = D / 16;               // 16-dim blocks of dK^T and dV^T
    constexpr int PIECES = RT * (D / 8);     // 16-byte pieces per tensor and tile
    constexpr int NP = PIECES / NTH;         // of them per thread
    static_assert(PIECES % NTH == 0 && NTH >= RT, "tile does not split over the threads");
    __shared__ __align__(16) bf16_t Qs[RT * LS];
    __shared__ __align__(16) bf16_t Ds[RT * LS];
    __shared__ float4 meta[RT];               // per row: lse log2(e) - d log2(e), Delta, token, valid
    __shared__ int list[NTH];
    __shared__ int wtot[NWV];

    // XCD-aware order: workgroups are dealt to the eight XCDs round-robin, so index x runs on
    // XCD x % 8; all chunks of one (sequence, KV group) are given to one XCD, in increasing
    // order, so the workgroups streaming the same query rows share that XCD's L2
    int c, gr;
    {
        const int bh = p.batch * p.h_kv, x = blockIdx.x;
        if (bh % 8 == 0) {
            gr = (x % 8) + 8 * ((x / 8) / p.nc);
            c = (x / 8) % p.nc;
        } else {
            gr = x / p.nc;
            c = x % p.nc;
        }
    }
    const int b = gr / p.h_kv, r = gr % p.h_kv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kl = lane & 15, grp = lane >> 4;
    const int n = p.n_kv;
    const int key = c * BLK + 16 * wave + kl;  // this lane's key (B operand column)
    const bool key_ok = key < n;
    const int64_t kv_row_stride = (int64_t)p.h_kv * D;

    // the wave's keys and values as B operands: lane (kl, grp) holds dims 32 ks + 8 grp .. + 7
    bw_bf16x8 kf[KS], vf[KS];
    {
        const int64_t off = ((int64_t)b * n + (key_ok ? key : 0)) * kv_row_stride + (int64_t)r * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 uk = key_ok ? *reinterpret_cast<const uint4*>(k + off + 32 * s) : make_uint4(0, 0, 0, 0);
            const uint4 uv = key_ok ? *reinterpret_cast<const uint4*>(v + off + 32 * s) : make_uint4(0, 0, 0, 0);
            kf[s] = __builtin_bit_cast(bw_bf16x8, uk);
            vf[s] = __builtin_bit_cast(bw_bf16x8, uv);
        }
    }
    bw_f32x4 acck[DB], accv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        acck[db] = bw_f32x4{};
        accv[db] = bw_f32x4{};
    }
    const float qk_scale = p.scale * kBwLog2e;

    // the tokens from chunk c on, in blocks of NTH taken from the last block down: workgroups of
    // the same (sequence, group) start together at the end of the sequence and walk down in step,
    // so the query rows they gather are read from HBM once and shared through the L2
    const int nblk = div_up(n - c * BLK, NTH);
    for (int bi = nblk - 1; bi >= 0; --bi) {
        const int t0 = c * BLK + bi * NTH;
        const int t = t0 + tid;
        bool att = false;
        if (t < n) {
            const int ct = t / BLK;
            att = ct == c || (ct > c && ((mask[(((int64_t)b * n + t) * p.h_kv + r) * p.nw + (c >> 5)] >> (c & 31)) & 1u));
        }
        const uint64_t bal = __ballot(att);
        if (lane == 0) wtot[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
        for (int w2 = 0; w2 < NWV; ++w2) {
            before += w2 < wave ? wtot[w2] : 0;
            total += wtot[w2];
        }
        if (att) list[before + __popcll(bal & ((1ull << lane) - 1ull))] = t;
        __syncthreads();

        // the rows of a tile (row m = token tl0 + m / g, head m % g) go global -> registers ->
        // LDS, the next tile's loads issued before the current tile's products; rows past the
        // list read its first token and are zeroed after (no branches, so every load is issued
        // back to back), and their record carries token -1, which no key pairs with
        uint4 gq[NP], gd[NP];
        float g_base = 0.f, g_dl = 0.f, g_tok = -1.f, g_ok = 0.f;
        auto gather = [&](int tl0) {
            int tok[NP];
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int tl = tl0 + (tid + i * NTH) / (D / 8) / GQ;
                tok[i] = list[tl < total ? tl : 0];
            }
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int e = tid + i * NTH;
                const int m = e / (D / 8), d8 = e % (D / 8);
                const int64_t off = ((((int64_t)b * n + tok[i]) * p.h_q) + r * GQ + m % GQ) * D + 8 * d8;
                gq[i] = *reinterpret_cast<const uint4*>(q + off);
                gd[i] = *reinterpret_cast<const uint4*>(dout + off);
            }
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                if (tl0 + (tid + i * NTH) / (D / 8) / GQ >= total) {
                    gq[i] = make_uint4(0, 0, 0, 0);
                    gd[i] = make_uint4(0, 0, 0, 0);
                }
            }
            if (tid < RT) {
                const int m = tid, tl = tl0 + m / GQ;
                g_base = 0.f, g_dl = 0.f, g_tok = -1.f, g_ok = 0.f;
                if (tl < total) {
                    const int tt = list[tl];
                    const int64_t qr = (int64_t)b * n + tt;
                    const int h = r * GQ + m % GQ;
                    const float dd = tt / BLK == c ? 0.f : bias[(qr * p.h_kv + r) * p.nc + c];
                    g_base = (lse[qr * p.h_q + h] - dd) * kBwLog2e;
                    g_dl = delta[qr * p.h_q + h];
                    g_tok = (float)tt;
                    g_ok = 1.f;
                }
            }
        };
        auto put = [&]() {
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int e = tid + i * NTH;
                const int m = e / (D / 8), d8 = e % (D / 8);
                *reinterpret_cast<uint4*>(&Qs[m * LS + 8 * d8]) = gq[i];
                *reinterpret_cast<uint4*>(&Ds[m * LS + 8 * d8]) = gd[i];
            }
            if (tid < RT) meta[tid] = make_float4(g_base, g_dl, g_tok, g_ok);
        };
        if (total > 0) gather(0);
        for (int tl0 = 0; tl0 < total; tl0 += TPT) {
            put();
            __syncthreads();
            if (tl0 + TPT < total) gather(tl0 + TPT);

#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                bw_f32x4 s[2], dp[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int rb = 2 * kb + h;
                    bw_bf16x8 aq[KS], ad[KS];
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        aq[ks] = *reinterpret_cast<const bw_bf16x8*>(&Qs[(16 * rb + kl) * LS + 32 * ks + 8 * grp]);
                        ad[ks] = *reinterpret_cast<const bw_bf16x8*>(&Ds[(16 * rb + kl) * LS + 32 * ks + 8 * grp]);
                    }
                    s[h] = bw_f32x4{};
                    dp[h] = bw_f32x4{};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[ks], kf[ks], s[h], 0, 0, 0);
                        dp[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad[ks], vf[ks], dp[h], 0, 0, 0);
                    }
                }
                // the eight rows' (base, Delta, token, valid) records read together, and p formed
                // without a branch (exp2(-inf) = 0 on rows and keys that do not pair)
                float4 mr[8];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) mr[4 * h + e] = meta[32 * kb + 16 * h + 4 * grp + e];
                bw_bf16x8 pf, dsf;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // rows past the list carry token -1, and every listed token is below n,
                        // so the one comparison also masks keys past the sequence
                        const float4 m4 = mr[4 * h + e];
                        const float x = fmaf(s[h][e], qk_scale, -m4.x);
                        const float pe = __builtin_amdgcn_exp2f((float)key <= m4.z ? x : -INFINITY);
                        const float ds = pe * (dp[h][e] - m4.y);
                        pf[4 * h + e] = (__bf16)pe;
                        dsf[4 * h + e] = (__bf16)ds;
                    }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bw_bf16x8 trd = tr_operand16<LS>(Ds, kb, db, lane);
                    const bw_bf16x8 trq = tr_operand16<LS>(Qs, kb, db, lane);
                    accv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(trd, pf, accv[db], 0, 0, 0);
                    acck[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(trq, dsf, acck[db], 0, 0, 0);
                }
            }
            __syncthreads();  // Qs, Ds and meta are refilled by the next tile
        }
    }
    if (!key_ok) return;
    // lane (kl, grp) holds dims 16 db + 4 grp + {0..3} of key kl
    const int64_t obase = (((int64_t)b * n + key) * p.h_kv + r) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d0 = 16 * db + 4 * grp;
        *reinterpret_cast<float4*>(dk + obase + d0) =
            make_float4(acck[db][0] * p.scale, acck[db][1] * p.scale, acck[db][2] * p.scale, acck[db][3] * p.scale);
        *reinterpret_cast<float4*>(dv + obase + d0) = make_float4(accv[db][0], accv[db][1], accv[db][2], accv[db][3]);
    }
}

template <int D, int BLK, int GQ>
static void launch_bwd_mfma_g(const void* q, const void* k, const void* v, const float* lse,
                              const void* dout, const uint32_t* mask, const float* bias,
                              float* dq, float* dk, float* dv, float* dbias, float* delta,
                              const AttnParams& p, hipStream_t st) {
    const int T = kBwRows / GQ;
    const int n_tiles = div_up(p.n_kv, T);
    hipLaunchKernelGGL((attn_bwd_dq_mfma_kernel<D, BLK, GQ>), dim3(p.batch * p.h_kv * n_tiles),
                       dim3(kBwThreads), 0, st, static_cast<const bf16_t*>(q),
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), lse,
                       static_cast<const bf16_t*>(dout), mask, bias, dq, dbias, delta, p, n_tiles);
    hipLaunchKernelGGL((attn_bwd_dkv16_mfma_kernel<D, BLK, GQ>), dim3(p.nc * p.h_kv * p.batch),
                       dim3(4 * BLK), 0, st, static_cast<const bf16_t*>(q),
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), lse,
                       static_cast<const bf16_t*>(dout), mask, bias, delta, dk, dv, p);
}

template <int D, int BLK>
static void launch_bwd_mfma_b(const void* q, const void* k, const void* v, const float* lse,
                              const void* dout, const uint32_t* mask, const float* bias,
                              float* dq, float* dk, float* dv, float* dbias, float* delta,
                              const AttnParams& p, hipStream_t st) {
    switch (p.g) {
        case 1: launch_bwd_mfma_g<D, BLK, 1>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st); break;
        case 2: launch_bwd_mfma_g<D, BLK, 2>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st); break;
        case 4: launch_bwd_mfma_g<D, BLK, 4>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st); break;
        case 8: launch_bwd_mfma_g<D, BLK, 8>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st); break;
        default: launch_bwd_mfma_g<D, BLK, 16>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st); break;
    }
}

template <int D>
static void launch_bwd_mfma_d(const void* q, const void* k, const void* v, const float* lse,
                              const void* dout, const uint32_t* mask, const float* bias,
                              float* dq, float* dk, float* dv, float* dbias, float* delta,
                              const AttnParams& p, hipStream_t st) {
    if (p.block == 32) launch_bwd_mfma_b<D, 32>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st);
    else if (p.block == 64) launch_bwd_mfma_b<D, 64>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st);
    else launch_bwd_mfma_b<D, 128>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st);
}

hipError_t launch_attn_backward_mfma(const void* q, const void* k, const void* v,
                                     const float* lse, const void* dout, const uint32_t* mask,
                                     const float* bias, float* dq, float* dk, float* dv,
                                     float* dbias, const AttnParams& p, void* ws,
                                     hipStream_t st) {
    float* delta = static_cast<float*>(ws);
    if (p.head_dim == 64) launch_bwd_mfma_d<64>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st);
    else launch_bwd_mfma_d<128>(q, k, v, lse, dout, mask, bias, dq, dk, dv, dbias, delta, p, st);
    return hipGetLastError();
}

}  // namespace dash
