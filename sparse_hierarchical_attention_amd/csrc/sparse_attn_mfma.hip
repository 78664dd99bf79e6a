// Stage 2 prefill on bf16 MFMA ("DashAttention", arXiv 2605.18753v1, §3.3-3.4 Prop. 1;
// App. G Alg. 3), gfx950.
//
// A workgroup (4 waves) owns 128 query rows of one (sequence b, KV group r): T = 128 / g
// consecutive tokens times the g heads of the group, row = token * g + head. All rows share the
// group's chunk selection per token, so the workgroup walks the union of its tokens' selected
// chunks (their own diagonal chunks included) and masks, per row, the chunks its token did not
// select. Chunks are cut into tiles of up to 64 keys; K and V tiles are staged through LDS in
// their stored layout, double-buffered: the next tile's global loads are in flight while the
// current one is multiplied, and one barrier per tile hands the buffers over.
//
// Per wave (32 rows) and tile, with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   A = K rows (ds_read_b128), B = the wave's Q rows held in registers for the
//                 whole kernel; lane l of the accumulator holds query row l % 32 and 16 keys.
//   O^T += V^T P^T  B = P straight from the S accumulator (converted to bf16), A = V^T read with
//                 ds_read_b64_tr_b16: inside each 16-lane group the four 64-bit loads of lanes
//                 4v .. 4v + 3 form key v, and lane i receives dimension i of keys 0..3, which
//                 is the run of four keys the lane's P slots refer to.
// Softmax in the log2 domain: x = s * scale * log2(e) + d * log2(e). The running maximum m is
// only raised when a tile's maximum exceeds it by more than 8 (so exp2(x - m) <= 256 and the
// output, normalised by the sum taken against the same m, is unchanged); p = exp2(x - m) is a
// single FMA and exp2 per score. A row whose token did not select the chunk has x = -inf; the
// query's own chunk is causally masked on the raw scores, so every tile takes the same code.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaRows = 128;
constexpr int kMfmaThreads = 256;
constexpr int kMaxMaskWords = 256;  // 8192 chunks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;    // log2 headroom before the running maximum is raised

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 ds_read_tr16(const bf16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(__attribute__((address_space(3))) void*)(p));
}

template <int D, int BLK, int GQ>
__global__ __launch_bounds__(kMfmaThreads, 2) void attn_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const uint32_t* __restrict__ mask, const float* __restrict__ bias, bf16_t* __restrict__ o,
    float* __restrict__ lse, AttnParams p, int n_tiles) {
    constexpr int T = kMfmaRows / GQ;        // tokens per tile
    constexpr int KT = BLK < 64 ? BLK : 64;  // keys per LDS tile
    constexpr int NSUB = BLK / KT;
    constexpr int KS = D + 8;                // K row stride in LDS (elements)
    constexpr int VS = D + 16;               // V row stride in LDS (elements)
    constexpr int MT = KT / 32;              // 32-key M-tiles of S^T
    constexpr int KSTEP = KT / 16;           // 16-key k-steps of P V
    constexpr int DT = D / 32;               // 32-dim M-tiles of O^T
    constexpr int LOADS = KT * (D / 8) / kMfmaThreads;  // 16-byte loads per thread and tensor
    static_assert(LOADS >= 1, "tile too small");
    __shared__ __align__(16) bf16_t Ks[2][KT * KS];
    __shared__ __align__(16) bf16_t Vs[2][KT * VS];
    __shared__ uint32_t uni[kMaxMaskWords];

    int gr;
    {
        const int bh = p.batch * p.h_kv, x = blockIdx.x;
        gr = bh % 8 == 0 ? (x % 8) + 8 * ((x / 8) % (bh / 8)) : x % bh;
    }
    const int tile = n_tiles - 1 - blockIdx.x / (p.batch * p.h_kv);
    const int b = gr / p.h_kv, r = gr % p.h_kv;
    const int n = p.n_kv;
    const int tile0 = tile * T;                        // first row of the tile among the n_q rows
    const int tile_end = min(tile0 + T, p.n_q);
    const int c_first = (p.q_pos0 + tile0) / BLK, c_last = (p.q_pos0 + tile_end - 1) / BLK;
    const int nwt = c_last / 32 + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, G = lane >> 5;
    const int row = wave * 32 + j;
    const int tok = row / GQ, hl = row % GQ;
    const int rowi = tile0 + tok;                       // the row among the n_q rows
    const int pos = p.q_pos0 + rowi;                    // its token position
    const bool valid = rowi < p.n_q;
    const int cpos = pos / BLK;
    const int64_t qrow = (int64_t)b * p.n_q + rowi;
    const uint32_t* mrow = mask + (qrow * p.h_kv + r) * p.nw;
    const float* brow = bias + (qrow * p.h_kv + r) * p.nc;

    // union of the tile tokens' selections (bits past a token's own chunk ignored)
    for (int w = tid; w < nwt; w += kMfmaThreads) uni[w] = 0u;
    __syncthreads();
    for (int idx = tid; idx < T * nwt; idx += kMfmaThreads) {
        const int t = idx / nwt, w = idx % nwt;
        const int ps = tile0 + t;
        if (ps >= p.n_q) continue;
        const int hi = (p.q_pos0 + ps) / BLK - 32 * w;
        if (hi < 0) continue;
        uint32_t word = mask[(((int64_t)b * p.n_q + ps) * p.h_kv + r) * p.nw + w];
        if (hi < 31) word &= (2u << hi) - 1u;
        if (hi < 32) word |= 1u << hi;
        if (word) atomicOr(&uni[w], word);
    }
    __syncthreads();
    // the union's next chunk after c (-1 when none): the same walk in every thread
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
    float m_used = -INFINITY, l_run = 0.f;
    const float qk_scale = p.scale * kLog2e;
    const int64_t kv_row_stride = (int64_t)p.h_kv * D;
    const bf16_t* kbase = k + (int64_t)b * n * kv_row_stride + (int64_t)r * D;
    const bf16_t* vbase = v + (int64_t)b * n * kv_row_stride + (int64_t)r * D;

    // global -> registers -> LDS for one tile (chunk c, 64-key part sub); thread tid moves the
    // 16-byte pieces tid + 256 i
    uint4 pk[LOADS], pv[LOADS];
    auto fetch = [&](int c, int sub) {
        const int key0 = c * BLK + sub * KT;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int e = tid + i * kMfmaThreads;
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
            const int e = tid + i * kMfmaThreads;
            const int kk = e / (D / 8), d8 = e % (D / 8);
            *reinterpret_cast<uint4*>(&Ks[buf][kk * KS + 8 * d8]) = pk[i];
            *reinterpret_cast<uint4*>(&Vs[buf][kk * VS + 8 * d8]) = pv[i];
        }
    };
    int c = next_chunk(-1), sub = 0;  // every tile has at least its own chunk
    fetch(c, 0);
    stash(0);
    __syncthreads();

    // transposed V reads: lane kl of 16-lane group grp reads key (kl / 4) of its 4-key run at
    // dimensions d0 + 4 (kl % 4)
    const int grp = lane >> 4, kl = lane & 15;
    const int v_key = 4 * (grp >> 1) + (kl >> 2);           // + 16 ks (+ 8 for the second run)
    const int v_dim = 16 * (grp & 1) + 4 * (kl & 3);        // + 32 dt

    for (int buf = 0; c >= 0; buf ^= 1) {
        const int key0 = c * BLK + sub * KT;
        // the tile after this one: the chunk's next 64 keys, or the union's next chunk
        const int c_nx = sub + 1 < NSUB ? c : next_chunk(c);
        const int sub_nx = sub + 1 < NSUB ? sub + 1 : 0;
        if (c_nx >= 0) fetch(c_nx, sub_nx);
        // this row's view of the chunk
        bool sel = false;
        if (valid && c <= cpos) sel = c == cpos || ((mrow[c >> 5] >> (c & 31)) & 1u);
        const float off = sel ? (c == cpos ? 0.f : brow[c] * kLog2e) : -INFINITY;
        const bool causal = c >= c_first;  // some row's own chunk: mask keys past each row

        // S^T = K Q^T
        f32x16 s[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            s[mt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[buf][(32 * mt + j) * KS + 16 * ks + 8 * G]);
                s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mt], 0, 0, 0);
            }
        }
        // keys past the row's own position score -inf; x = s * scale log2(e) + off is then -inf
        // too (scale > 0), as it is for every key of a row that did not select the chunk
        if (causal) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int key = key0 + 32 * mt + 8 * (rr >> 2) + 4 * G + (rr & 3);
                    if (key > pos) s[mt][rr] = -INFINITY;
                }
        }
        float smax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) smax = fmaxf(smax, s[mt][rr]);
        const float xmax = fmaf(halves_max(smax), qk_scale, off);
        // raise the running maximum only when needed (rare once a row has seen its peak)
        const bool raise = xmax > m_used + kLazyMax;
        if (__any(raise)) {
            const float m_new = raise ? xmax : m_used;
            const float corr = m_used == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_used - m_new);
            l_run *= corr;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= corr;
            m_used = m_new;
        }
        // p = exp2(x - m) as one FMA and exp2; the row sum stays per lane (this half's keys) until
        // the end, since both halves scale it by the same factors
        const float off_m = off - (m_used == -INFINITY ? 0.f : m_used);
        bf16x8 pf[KSTEP];
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks)
#pragma unroll
            for (int vv = 0; vv < 8; ++vv) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][8 * (ks & 1) + vv], qk_scale, off_m));
                l_run += pe;
                pf[ks][vv] = (__bf16)pe;
            }

        // O^T += V^T P^T, V^T from the stored rows through transposing reads
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16_t* vp = &Vs[buf][(16 * ks + v_key) * VS + 32 * dt + v_dim];
                const i16x4 lo = ds_read_tr16(vp);
                const i16x4 hi = ds_read_tr16(vp + 8 * VS);
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], acc[dt], 0, 0, 0);
            }
        if (c_nx >= 0) stash(buf ^ 1);
        __syncthreads();
        c = c_nx;
        sub = sub_nx;
    }

    l_run = halves_sum(l_run);
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
    if (lse && G == 0) lse[qrow * p.h_q + r * GQ + hl] = (m_used + __log2f(l_run)) * kLn2;
}

template <int D, int BLK>
static void launch_mfma_blk(const void* q, const void* k, const void* v, const uint32_t* mask,
                            const float* bias, void* o, float* lse, const AttnParams& p,
                            hipStream_t st) {
    const int T = kMfmaRows / p.g;
    const int n_tiles = div_up(p.n_q, T);
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

// head dim 64 here; head dim 128 streams its tiles with direct LDS loads (sparse_attn_dma.hip)
hipError_t launch_attn_prefill_mfma(const void* q, const void* k, const void* v,
                                   const uint32_t* mask, const float* bias, void* o, float* lse,
                                   const AttnParams& p, hipStream_t st) {
    if (p.head_dim != 64) return launch_attn_prefill_dma(q, k, v, mask, bias, o, lse, p, st);
    launch_mfma_d<64>(q, k, v, mask, bias, o, lse, p, st);
    return hipGetLastError();
}

}  // namespace dash
