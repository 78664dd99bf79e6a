// Stage 2 prefill on bf16 MFMA ("DashAttention", arXiv 2605.18753v1, §3.3-3.4 Prop. 1;
// App. G Alg. 3), gfx950.
//
// A workgroup (4 waves) owns 128 query rows of one (sequence b, KV group r): T = 128 / g
// consecutive tokens times the g heads of the group, row = token * g + head. All rows share the
// group's chunk selection per token, so the workgroup walks the union of its tokens' selected
// chunks (their own diagonal chunks included) and masks, per row, the chunks its token did not
// select. Each chunk is staged through LDS in sub-tiles of up to 64 keys: K as stored, V
// transposed, both read by all four waves.
//
// Per wave (32 rows) and sub-tile, with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   A = K rows from LDS, B = the wave's Q rows held in registers for the whole
//                 kernel; the accumulator gives lane l the column l % 32 (its query row) and
//                 16 keys, so a row's maximum and sum need one exchange with lane l ^ 32.
//   O^T += V^T P^T  B = P straight from the S accumulator registers (converted to bf16): the
//                 k-slots of a lane are its own 8 keys, and A = V^T is read from LDS in the
//                 same key order, so P never moves between lanes.
// Logits live in the log2 domain: x = s * scale * log2(e) + d * log2(e), online softmax with
// exp2. A row whose token did not select the chunk gets x = -inf; the query's own chunk is
// causally masked.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaRows = 128;
constexpr int kMfmaThreads = 256;
constexpr int kMaxMaskWords = 256;  // 8192 chunks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int xcd_remap(int x, int bh, int* gr) {
    // Workgroups are dispatched round-robin over the 8 XCDs (x % 8). When the (sequence, group)
    // pairs split evenly over them, keep every tile of a pair on one XCD so its K/V chunks stay
    // in that XCD's L2; tile ranks count up, so the longest (last) tiles start first.
    if (bh % 8 == 0) {
        *gr = (x % 8) + 8 * ((x / 8) % (bh / 8));
    } else {
        *gr = x % bh;
    }
    return x / bh;
}

template <int D, int BLK, int GQ>
__global__ __launch_bounds__(kMfmaThreads, 2) void attn_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const uint32_t* __restrict__ mask, const float* __restrict__ bias, bf16_t* __restrict__ o,
    float* __restrict__ lse, AttnParams p, int n_tiles) {
    constexpr int T = kMfmaRows / GQ;        // tokens per tile
    constexpr int KT = BLK < 64 ? BLK : 64;  // keys per LDS sub-tile
    constexpr int NSUB = BLK / KT;
    constexpr int KS = D + 8;                // K row stride in LDS (elements)
    constexpr int VS = KT + 4;               // V^T row stride in LDS (elements)
    constexpr int MT = KT / 32;              // 32-key M-tiles of S^T
    constexpr int KSTEP = KT / 16;           // 16-key k-steps of P V
    constexpr int DT = D / 32;               // 32-dim M-tiles of O^T
    __shared__ __align__(16) bf16_t Ks[KT * KS];
    __shared__ __align__(16) bf16_t Vt[D * VS];
    __shared__ uint32_t uni[kMaxMaskWords];

    int gr;
    const int tile = n_tiles - 1 - xcd_remap(blockIdx.x, p.batch * p.h_kv, &gr);
    const int b = gr / p.h_kv, r = gr % p.h_kv;
    const int n = p.n_kv;
    const int tile0 = tile * T;
    const int tile_end = min(tile0 + T, n);
    const int c_last = (tile_end - 1) / BLK;
    const int nwt = c_last / 32 + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, G = lane >> 5;
    const int row = wave * 32 + j;
    const int tok = row / GQ, hl = row % GQ;
    const int pos = tile0 + tok;
    const bool valid = pos < n;
    const int cpos = pos / BLK;
    const int64_t qrow = (int64_t)b * p.n_q + pos;
    const uint32_t* mrow = mask + (qrow * p.h_kv + r) * p.nw;
    const float* brow = bias + (qrow * p.h_kv + r) * p.nc;

    // union of the tile tokens' selections (bits past a token's own chunk ignored)
    for (int w = tid; w < nwt; w += kMfmaThreads) uni[w] = 0u;
    __syncthreads();
    for (int idx = tid; idx < T * nwt; idx += kMfmaThreads) {
        const int t = idx / nwt, w = idx % nwt;
        const int ps = tile0 + t;
        if (ps >= n) continue;
        const int hi = ps / BLK - 32 * w;
        if (hi < 0) continue;
        uint32_t word = mask[(((int64_t)b * p.n_q + ps) * p.h_kv + r) * p.nw + w];
        if (hi < 31) word &= (2u << hi) - 1u;
        if (hi < 32) word |= 1u << hi;
        if (word) atomicOr(&uni[w], word);
    }

    // this wave's Q rows as the B operand of S^T = K Q^T (k-slot order shared with K's reads)
    bf16x8 qf[D / 16];
    {
        const bf16_t* qp = q + (qrow * p.h_q + r * GQ + hl) * D + 8 * G;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            uint4 u = valid ? *reinterpret_cast<const uint4*>(qp + 16 * s) : make_uint4(0, 0, 0, 0);
            qf[s] = __builtin_bit_cast(bf16x8, u);
        }
    }
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const float qk_scale = p.scale * kLog2e;
    const int64_t kv_row_stride = (int64_t)p.h_kv * D;
    const bf16_t* kbase = k + (int64_t)b * n * kv_row_stride + (int64_t)r * D;
    const bf16_t* vbase = v + (int64_t)b * n * kv_row_stride + (int64_t)r * D;
    __syncthreads();

    for (int w = 0; w < nwt; ++w) {
        uint32_t word = uni[w];
        uint32_t myword = 0u;
        if (valid && 32 * w <= cpos) {
            const int hi = cpos - 32 * w;
            myword = mrow[w];
            if (hi < 31) myword &= (2u << hi) - 1u;
            if (hi < 32) myword |= 1u << hi;
        }
        while (word) {
            const int bit = __builtin_ctz(word);
            word &= word - 1u;
            const int c = 32 * w + bit;
            const bool sel = (myword >> bit) & 1u;
            const bool diag = c == cpos;
            float off = -INFINITY, sc = 0.f;
            if (sel) {
                sc = qk_scale;
                off = diag ? 0.f : brow[c] * kLog2e;
            }
            const bool causal = diag;  // only the query's own chunk holds keys after it
#pragma unroll 1
            for (int sub = 0; sub < NSUB; ++sub) {
                const int key0 = c * BLK + sub * KT;
                __syncthreads();  // the previous sub-tile has been consumed
                // K sub-tile, rows as stored
                for (int e = tid; e < KT * (D / 8); e += kMfmaThreads) {
                    const int kk = e / (D / 8), d8 = e % (D / 8);
                    const int key = key0 + kk;
                    uint4 u = make_uint4(0, 0, 0, 0);
                    if (key < n) u = *reinterpret_cast<const uint4*>(kbase + key * kv_row_stride + 8 * d8);
                    *reinterpret_cast<uint4*>(&Ks[kk * KS + 8 * d8]) = u;
                }
                // V sub-tile, transposed: 4 keys x 8 dims per item, written as 8 runs of 4 keys
                for (int e = tid; e < (KT / 4) * (D / 8); e += kMfmaThreads) {
                    const int d8 = e % (D / 8), kq = e / (D / 8);
                    uint4 u[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = key0 + 4 * kq + i;
                        u[i] = key < n ? *reinterpret_cast<const uint4*>(vbase + key * kv_row_stride + 8 * d8)
                                       : make_uint4(0, 0, 0, 0);
                    }
                    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&u[0]);
                    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&u[1]);
                    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&u[2]);
                    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&u[3]);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        // dims 2jj (low halves) and 2jj + 1 (high halves) of the four keys
                        const uint32_t lo01 = (w0[jj] & 0xffffu) | (w1[jj] << 16);
                        const uint32_t lo23 = (w2[jj] & 0xffffu) | (w3[jj] << 16);
                        const uint32_t hi01 = (w0[jj] >> 16) | (w1[jj] & 0xffff0000u);
                        const uint32_t hi23 = (w2[jj] >> 16) | (w3[jj] & 0xffff0000u);
                        *reinterpret_cast<uint2*>(&Vt[(8 * d8 + 2 * jj) * VS + 4 * kq]) = make_uint2(lo01, lo23);
                        *reinterpret_cast<uint2*>(&Vt[(8 * d8 + 2 * jj + 1) * VS + 4 * kq]) = make_uint2(hi01, hi23);
                    }
                }
                __syncthreads();

                // S^T = K Q^T
                f32x16 s[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    s[mt] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(32 * mt + j) * KS + 16 * ks + 8 * G]);
                        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mt], 0, 0, 0);
                    }
                }
                // logits, masking, row maximum
                float rmax = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        float x = s[mt][rr] * sc + off;
                        if (causal) {
                            const int key = key0 + 32 * mt + 8 * (rr >> 2) + 4 * G + (rr & 3);
                            if (key > pos) x = -INFINITY;
                        }
                        s[mt][rr] = x;
                        rmax = fmaxf(rmax, x);
                    }
                rmax = fmaxf(rmax, __shfl_xor(rmax, 32, kWave));
                const float m_new = fmaxf(m_run, rmax);
                const float m_ref = m_new == -INFINITY ? 0.f : m_new;
                const float corr = __builtin_amdgcn_exp2f(m_run - m_ref);
                float rsum = 0.f;
                bf16x8 pf[KSTEP];
#pragma unroll
                for (int ks = 0; ks < KSTEP; ++ks)
#pragma unroll
                    for (int vv = 0; vv < 8; ++vv) {
                        const float pv = __builtin_amdgcn_exp2f(s[ks >> 1][8 * (ks & 1) + vv] - m_ref);
                        rsum += pv;
                        pf[ks][vv] = (__bf16)pv;
                    }
                rsum += __shfl_xor(rsum, 32, kWave);
                l_run = l_run * corr + rsum;
                m_run = m_new;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= corr;
                // O^T += V^T P^T
#pragma unroll
                for (int ks = 0; ks < KSTEP; ++ks)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const bf16_t* vp = &Vt[(32 * dt + j) * VS + 16 * ks + 4 * G];
                        const bf16x4 a0 = *reinterpret_cast<const bf16x4*>(vp);
                        const bf16x4 a1 = *reinterpret_cast<const bf16x4*>(vp + 8);
                        const bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], acc[dt], 0, 0, 0);
                    }
            }
        }
    }

    if (!valid) return;
    const float inv_l = 1.0f / l_run;
    bf16_t* orow = o + (qrow * p.h_q + r * GQ + hl) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int d0 = 32 * dt + 8 * qd + 4 * G;
            bf16x4 ov;
#pragma unroll
            for (int u = 0; u < 4; ++u) ov[u] = (__bf16)(acc[dt][4 * qd + u] * inv_l);
            *reinterpret_cast<bf16x4*>(orow + d0) = ov;
        }
    if (lse && G == 0) lse[qrow * p.h_q + r * GQ + hl] = (m_run + __log2f(l_run)) * kLn2;
}

template <int D, int BLK>
static void launch_mfma_blk(const void* q, const void* k, const void* v, const uint32_t* mask,
                            const float* bias, void* o, float* lse, const AttnParams& p,
                            hipStream_t st) {
    const int T = kMfmaRows / p.g;
    const int n_tiles = div_up(p.n_kv, T);
    dim3 grid(p.batch * p.h_kv * n_tiles);
#define DASH_MFMA(GG)                                                                       \
    hipLaunchKernelGGL((attn_mfma_kernel<D, BLK, GG>), grid, dim3(kMfmaThreads), 0, st,     \
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),        \
                       static_cast<const bf16_t*>(v), mask, bias, static_cast<bf16_t*>(o), \
                       lse, p, n_tiles)
    switch (p.g) {
        case 1: DASH_MFMA(1); break;
        case 2: DASH_MFMA(2); break;
        case 4: DASH_MFMA(4); break;
        case 8: DASH_MFMA(8); break;
        default: DASH_MFMA(16); break;
    }
#undef DASH_MFMA
}

template <int D>
static void launch_mfma_d(const void* q, const void* k, const void* v, const uint32_t* mask,
                          const float* bias, void* o, float* lse, const AttnParams& p,
                          hipStream_t st) {
    if (p.block == 32) launch_mfma_blk<D, 32>(q, k, v, mask, bias, o, lse, p, st);
    else if (p.block == 64) launch_mfma_blk<D, 64>(q, k, v, mask, bias, o, lse, p, st);
    else launch_mfma_blk<D, 128>(q, k, v, mask, bias, o, lse, p, st);
}

hipError_t launch_attn_prefill_mfma(const void* q, const void* k, const void* v,
                                   const uint32_t* mask, const float* bias, void* o, float* lse,
                                   const AttnParams& p, hipStream_t st) {
    if (p.head_dim == 64) launch_mfma_d<64>(q, k, v, mask, bias, o, lse, p, st);
    else launch_mfma_d<128>(q, k, v, mask, bias, o, lse, p, st);
    return hipGetLastError();
}

}  // namespace dash
