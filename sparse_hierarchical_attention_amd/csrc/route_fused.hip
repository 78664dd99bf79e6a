// Stage 1 for many queries in one pass, without a score workspace ("DashAttention",
// arXiv 2605.18753v1, §3.2 Eq. 4, §3.4 Prop. 1; App. G Alg. 2 with the score rows kept on chip).
//
// A workgroup of NW waves owns 32 NR query rows of one (sequence b, KV group r): T = 32 NR / g
// consecutive tokens times the g heads of the group (row = token * g + head).
// Phase 1, scores: X^T = Kbar Q^T on v_mfma_f32_32x32x16_bf16. The fp32 summaries are split once
// per call (split_kbar_kernel, into the workspace) as kbar = hi + mid + lo, each a bf16
// (hi = bf16(kbar), mid = bf16(kbar - hi), lo = bf16 of the rest), so three bf16 products carry
// about 24 mantissa bits of the summary (Q is bf16 already) with fp32 accumulation. Wave w
// computes the 32-chunk tiles w, w + NW, ... of all rows.
// The score rows then go through LDS (row-major, odd stride) so that one wave can own a token.
// Phase 2: per token, the same register-resident threshold solver and row writer as the
// workspace path (entmax.h, route_common.h): the g heads in turn, the GQA mean, mask and bias.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "entmax.h"
#include "kernels.h"
#include "route_common.h"

namespace dash {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLongRows = 16;   // query rows per workgroup of route_long_kernel
constexpr int kLongMax = 2048;  // chunks route_long_kernel holds per row
constexpr int kLongCand = 256;  // packed candidates of a long row's threshold solve

// The fp32 summaries as three bf16 terms, hi = bf16(kbar), mid = bf16(kbar - hi),
// lo = bf16(kbar - hi - mid), each rounded to nearest even (together about 24 mantissa bits),
// stored in the order phase 1 loads them as MFMA A fragments:
//   [B][H_kv][ct = c / 32][ks = d / 16][term][lane = c % 32 + 32 ((d / 8) % 2)][8 bf16]
// so that one fragment load of a wave reads 1 KiB contiguous. Chunks of the last tile past Tc
// are zero. One thread per (b, r, ct, ks, lane): 8 elements.
__global__ __launch_bounds__(256) void split_kbar_kernel(const float* __restrict__ kbar,
                                                         bf16_t* __restrict__ planes, int batch,
                                                         int tc, int h_kv, int D) {
    const int ks_n = D / 16, ct_n = div_up(tc, 32);
    const int64_t n = (int64_t)batch * h_kv * ct_n * ks_n * 64;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int lane = (int)(i % 64);
    int64_t rest = i / 64;
    const int ks = (int)(rest % ks_n);
    rest /= ks_n;
    const int ct = (int)(rest % ct_n);
    rest /= ct_n;
    const int r = (int)(rest % h_kv);
    const int b = (int)(rest / h_kv);
    const int c = 32 * ct + (lane & 31);
    float kv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < tc) {
        const float4* src = reinterpret_cast<const float4*>(
            kbar + (((int64_t)b * tc + c) * h_kv + r) * D + 16 * ks + 8 * (lane >> 5));
        const float4 x0 = src[0], x1 = src[1];
        kv[0] = x0.x; kv[1] = x0.y; kv[2] = x0.z; kv[3] = x0.w;
        kv[4] = x1.x; kv[5] = x1.y; kv[6] = x1.z; kv[7] = x1.w;
    }
    bf16x8_t hi, mid, lo;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const __bf16 h = (__bf16)kv[u];
        const float r1 = kv[u] - (float)h;
        const __bf16 md = (__bf16)r1;
        hi[u] = h;
        mid[u] = md;
        lo[u] = (__bf16)(r1 - (float)md);
    }
    uint4* out = reinterpret_cast<uint4*>(planes) + (((int64_t)(b * h_kv + r) * ct_n + ct) * ks_n + ks) * 3 * 64 + lane;
    out[0] = __builtin_bit_cast(uint4, hi);
    out[64] = __builtin_bit_cast(uint4, mid);
    out[128] = __builtin_bit_cast(uint4, lo);
}

// The mask words and bias of one token's row from its group-summed probabilities wsum (entry c
// in lane c % 16 of a 16-lane group, slot c / 16; every group holds the same row when g >= 4,
// the rows of 4 / g tokens otherwise): w = wsum / g, mu = mean log w over R = {w > 0},
// d = (log w - mu) / sigma on R, the window's chunks (the query's own chunk cp and the win
// before it) always set with d = 0.
template <int NSS, int GQ>
__device__ __forceinline__ void route_write_token(float (&wsum)[NSS], int tok, int b, int r,
                                                  uint32_t* __restrict__ mask,
                                                  float* __restrict__ bias, const RouteParams& p) {
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, li = lane & 15;
    const bool tvalid = tok < p.n_q;
    const int pos = route_pos(p, b, tok);
    const int cp = pos / p.block;
    const int m = route_cands(p, pos);  // chunks m .. cp: the window, always attended with d = 0
    const float inv_g = 1.0f / (float)GQ;
    // the groups that write: one per token
    const bool writer = tvalid && (GQ >= 4 ? grp == 0 : (GQ == 2 ? (grp & 1) == 0 : true));
    const int64_t qrow = (int64_t)b * p.n_q + tok;
    uint32_t* mrow = mask + (qrow * p.h_kv + r) * p.nw;
    float* brow = bias + (qrow * p.h_kv + r) * p.nc;
#pragma unroll
    for (int sl = 0; sl < NSS; ++sl) wsum[sl] *= inv_g;
    if (GQ >= 4) {
        // every group holds the token's row: group k takes the log of slots k, k + 4, ... once, for
        // mu and for its own bias stores; the four groups' sums meet across the wave's rows
        constexpr int NQ = (NSS + 3) / 4;
        float lq[NQ];
        float lsum = 0.f, lcnt = 0.f;
#pragma unroll
        for (int s0 = 0; s0 < NSS; s0 += 4) {
            float w = wsum[s0];
#pragma unroll
            for (int j = 1; j < 4; ++j)
                if (s0 + j < NSS && grp == j) w = wsum[s0 + j];
            const bool in = s0 + grp < NSS && w > 0.f;
            const float l = in ? __logf(w) : 0.f;
            lq[s0 / 4] = l;
            lsum += l;
            lcnt += in ? 1.f : 0.f;
        }
        lsum = halves_sum(rowpair_sum(row16_sum(lsum)));
        lcnt = halves_sum(rowpair_sum(row16_sum(lcnt)));
        const float mu = lcnt > 0.f ? lsum / lcnt : 0.f;
#pragma unroll
        for (int s0 = 0; s0 < NSS; s0 += 4) {
            float w = wsum[s0];
#pragma unroll
            for (int j = 1; j < 4; ++j)
                if (s0 + j < NSS && grp == j) w = wsum[s0 + j];
            if (tvalid && s0 + grp < NSS && w > 0.f) brow[16 * (s0 + grp) + li] = (lq[s0 / 4] - mu) * p.inv_sigma;
        }
    } else {
        // log w on R (0 elsewhere), kept for the bias when the row is short enough to hold it in
        // registers, else computed again there
        constexpr bool kKeepLog = NSS <= 16;
        float lw[kKeepLog ? NSS : 1];
        auto logw = [&](int sl) { return wsum[sl] > 0.f ? __logf(wsum[sl]) : 0.f; };
        float lsum = 0.f, lcnt = 0.f;
#pragma unroll
        for (int sl = 0; sl < NSS; ++sl) {
            const float l = logw(sl);
            if (kKeepLog) lw[kKeepLog ? sl : 0] = l;
            lsum += l;
            lcnt += wsum[sl] > 0.f ? 1.f : 0.f;
        }
        lsum = row16_sum(lsum);
        lcnt = row16_sum(lcnt);
        const float mu = lcnt > 0.f ? lsum / lcnt : 0.f;
#pragma unroll
        for (int sl = 0; sl < NSS; ++sl)
            if (writer && wsum[sl] > 0.f)
                brow[16 * sl + li] = ((kKeepLog ? lw[kKeepLog ? sl : 0] : logw(sl)) - mu) * p.inv_sigma;
    }
    // mask words of the bucket, gathered so that lane li of a group holds words li and li + 16
    uint32_t wlo = 0u, whi = 0u;
#pragma unroll
    for (int wd = 0; wd < NSS / 2; ++wd) {
        const uint64_t b0 = __ballot(wsum[2 * wd] > 0.f);
        const uint64_t b1 = __ballot(wsum[2 * wd + 1] > 0.f);
        const uint32_t word = (uint32_t)((b0 >> (16 * grp)) & 0xffffu) |
                              ((uint32_t)((b1 >> (16 * grp)) & 0xffffu) << 16);
        if (li == (wd & 15)) {
            if (wd < 16) wlo = word;
            else whi = word;
        }
    }
    if (writer && li < NSS / 2 && li < p.nw) mrow[li] = wlo | span_bits(li, m, cp);
    if (NSS / 2 > 16 && writer && li + 16 < NSS / 2 && li + 16 < p.nw)
        mrow[li + 16] = whi | span_bits(li + 16, m, cp);
    // words past the bucket: only the window's chunks can be set there
    for (int wd = NSS / 2 + li; wd < p.nw; wd += 16)
        if (writer) mrow[wd] = span_bits(wd, m, cp);
    for (int c = m + li; c <= cp; c += 16)
        if (writer) brow[c] = 0.f;
}

// One pass of the fused route's phase 2 (see route_fused_kernel): the four rows xr0 + k xstride,
// k = 0..3, one per 16-lane group, rows row0 .. row0 + 3 of the tile. Solves each row's threshold
// and returns its probabilities, summed over the heads of the pass that share a token, in wsum.
template <int NSS, int KIND, int GQ>
__device__ __forceinline__ void route_pass(const float* __restrict__ xr0, int xstride, int row0,
                                           int tile0, int b, int r, float* __restrict__ tau_out,
                                           const RouteParams& p, float (&wsum)[NSS]) {
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, li = lane & 15;
    const float e = 1.0f / (p.alpha - 1.0f);
    const int row = row0 + grp;
    const int tok = tile0 + row / GQ;
    const bool tvalid = tok < p.n_q;
    const int m = tvalid ? route_cands(p, route_pos(p, b, tok)) : 0;
    const float* xr = xr0 + grp * xstride;
    float xv[NSS];
#pragma unroll
    for (int sl = 0; sl < NSS; ++sl) {
        const int c = 16 * sl + li;
        const float v = xr[c];
        xv[sl] = c < m ? v : -INFINITY;
    }
    const float tau = solve_tau_exact<NSS, KIND, 16>(xv, NSS, m, p.alpha);
    if (tau_out && tvalid && li == 0)
        tau_out[((int64_t)b * p.n_q + tok) * p.h_q + r * GQ + row % GQ] = tau;
#pragma unroll
    for (int sl = 0; sl < NSS; ++sl) {
        float pv = pow_e<KIND>(xv[sl] - tau, e);
        if (GQ >= 2) pv = pair16_sum(pv);   // heads in groups 0+1 and 2+3
        if (GQ >= 4) pv = pair32_sum(pv);   // all four groups
        wsum[sl] = pv;
    }
}

// A whole unit of phase 2 for g <= 4: 4 / g tokens (g < 4) or one token (g = 4) in one pass.
template <int NSS, int KIND, int GQ>
__device__ __forceinline__ void route_unit(const float* __restrict__ xr0, int xstride, int row0,
                                           int tile0, int b, int r, uint32_t* __restrict__ mask,
                                           float* __restrict__ bias, float* __restrict__ tau_out,
                                           const RouteParams& p) {
    static_assert(GQ <= 4, "groups of more than four heads take one pass per unit");
    const int grp = (threadIdx.x & 63) >> 4;
    float wsum[NSS];
    route_pass<NSS, KIND, GQ>(xr0, xstride, row0, tile0, b, r, tau_out, p, wsum);
    route_write_token<NSS, GQ>(wsum, tile0 + (GQ >= 4 ? row0 : row0 + grp) / GQ, b, r, mask, bias, p);
}

// One pass of a token's heads for g > 4: its probabilities, summed over the pass's four heads,
// replace the first of the pass's score rows in LDS (this wave has read all four).
template <int NSS, int KIND, int GQ>
__device__ __forceinline__ void route_head_pass(float* __restrict__ xr0, int xstride, int row0,
                                                int tile0, int b, int r,
                                                float* __restrict__ tau_out, const RouteParams& p) {
    const int lane = threadIdx.x & 63;
    float wsum[NSS];
    route_pass<NSS, KIND, GQ>(xr0, xstride, row0, tile0, b, r, tau_out, p, wsum);
    if (lane < 16) {
#pragma unroll
        for (int sl = 0; sl < NSS; ++sl) xr0[16 * sl + lane] = wsum[sl];
    }
}

// The token's rows for g > 4 once every pass has left its partial sum in LDS: the partials
// (rows 0, 4, 8, ... of the token) added in pass order, then the token's mask and bias.
template <int NSS, int GQ>
__device__ __forceinline__ void route_finish_token(const float* __restrict__ xt, int xstride,
                                                   int tok, int b, int r,
                                                   uint32_t* __restrict__ mask,
                                                   float* __restrict__ bias, const RouteParams& p) {
    const int li = threadIdx.x & 15;
    float wsum[NSS];
#pragma unroll
    for (int sl = 0; sl < NSS; ++sl) wsum[sl] = 0.f;
#pragma unroll
    for (int ps = 0; ps < GQ / 4; ++ps)
#pragma unroll
        for (int sl = 0; sl < NSS; ++sl) wsum[sl] += xt[4 * ps * xstride + 16 * sl + li];
    route_write_token<NSS, GQ>(wsum, tok, b, r, mask, bias, p);
}

// NW waves per workgroup, at least 16 / NW waves per SIMD (the register budget follows). NR MFMA
// N-tiles of 32 query rows share every summary fragment a wave loads.
template <int D, int GQ, int MT, int NW, int NR, int KIND>
__global__ __launch_bounds__(NW * 64, 16 / NW) void route_fused_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ planes, uint32_t* __restrict__ mask,
    float* __restrict__ bias, float* __restrict__ tau_out, RouteParams p, int n_tiles,
    float coef) {
    constexpr int ROWS = 32 * NR;            // NR MFMA N-tiles of query rows
    constexpr int T = ROWS / GQ;             // tokens per workgroup
    constexpr int CMAX = 32 * NW * MT;       // chunks the workgroup can hold
    constexpr int NPL = CMAX / 64;           // row slots per lane when a wave owns a row
    constexpr int XS = CMAX + 17;            // LDS row stride of the scores (bank spread for the
                                             // MFMA-layout writes and the 16-lane-group reads)
    constexpr int QS = D + 8;                // LDS row stride of Q (elements)
    static_assert(NPL >= 1, "at least one slot");
    // Q (phase 1) and the score rows (phase 2) share the LDS
    __shared__ __align__(16) float lds[ROWS * XS > (ROWS * QS) / 2 ? ROWS * XS : (ROWS * QS) / 2];
    bf16_t* qs = reinterpret_cast<bf16_t*>(lds);
    float* xs = lds;

    const int bh = p.batch * p.h_kv;
    const int x = blockIdx.x;
    const int gr = bh % 8 == 0 ? (x % 8) + 8 * ((x / 8) % (bh / 8)) : x % bh;
    const int tile = n_tiles - 1 - x / bh;
    const int b = gr / p.h_kv, r = gr % p.h_kv;
    const int tile0 = tile * T;
    const int tile_end = min(tile0 + T, p.n_q);
    const int m_max = route_cands(p, route_pos(p, b, tile_end - 1));
    const int n_ct = div_up(m_max, 32);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, G = lane >> 5;

    // ---- phase 1: scores X^T = kbar Q^T on MFMA, kbar = hi + mid + lo in bf16
    for (int idx = tid; idx < ROWS * (D / 8); idx += NW * 64) {
        const int row = idx / (D / 8), d8 = idx % (D / 8);
        const int t = tile0 + row / GQ;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (t < p.n_q)
            u = *reinterpret_cast<const uint4*>(
                q + (((int64_t)b * p.n_q + t) * p.h_q + r * GQ + row % GQ) * D + 8 * d8);
        *reinterpret_cast<uint4*>(&qs[row * QS + 8 * d8]) = u;
    }
    __syncthreads();
    f32x16_t X[MT][NR];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nr = 0; nr < NR; ++nr) X[mt][nr] = f32x16_t{};
    // A fragments of this wave's chunk tiles (hi, mid, lo of each 16-d slice, 1 KiB per wave and
    // term); the slice ks + 1 is in flight while slice ks is multiplied
    const int ct_n = div_up(p.tc, 32);
    const uint4* src[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int ct = min(wave + NW * mt, ct_n - 1);
        src[mt] = reinterpret_cast<const uint4*>(planes) +
                  ((int64_t)(b * p.h_kv + r) * ct_n + ct) * (D / 16) * 3 * 64 + lane;
    }
    uint4 cur[MT][3], nxt[MT][3];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        if (wave + NW * mt < n_ct) {
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) cur[mt][pl] = src[mt][pl * 64];
        }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        if (ks + 1 < D / 16) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                if (wave + NW * mt < n_ct) {
#pragma unroll
                    for (int pl = 0; pl < 3; ++pl) nxt[mt][pl] = src[mt][((ks + 1) * 3 + pl) * 64];
                }
        }
        bf16x8_t qf[NR];
#pragma unroll
        for (int nr = 0; nr < NR; ++nr)
            qf[nr] = *reinterpret_cast<const bf16x8_t*>(&qs[(32 * nr + j) * QS + 16 * ks + 8 * G]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (wave + NW * mt >= n_ct) break;
#pragma unroll
            for (int nr = 0; nr < NR; ++nr) {
#pragma unroll
                for (int pl = 2; pl >= 0; --pl)  // lo, mid, hi: the small terms first
                    X[mt][nr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, cur[mt][pl]), qf[nr], X[mt][nr], 0, 0, 0);
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) cur[mt][pl] = nxt[mt][pl];
    }
    __syncthreads();  // Q is dead; its LDS now takes the score rows
    // lane (j, G) holds row 32 nr + j, chunks 32 ct + 8 (rr / 4) + 4 G + rr % 4
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int ct = wave + NW * mt;
        if (ct >= n_ct) break;
#pragma unroll
        for (int nr = 0; nr < NR; ++nr)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                xs[(32 * nr + j) * XS + 32 * ct + 8 * (rr >> 2) + 4 * G + (rr & 3)] = coef * X[mt][nr][rr];
    }
    __syncthreads();

    // ---- phase 2: a wave takes 4 rows at a time, one per 16-lane DPP row (lane group); entry c
    // of a row sits in lane c % 16 of its group, slot c / 16. For g <= 4 a unit is one pass over
    // 4 / g tokens or one token; for g > 4 it is one pass over four heads of a token, and the
    // token's passes, spread over the waves, leave partial sums in LDS that one wave then adds.
    // The slot count is a compile-time bucket (the unit's longest row, rounded up to a multiple of
    // 4 slots up to 32, of 8 up to 64) so that every slot loop unrolls and a row pays for at most
    // a few slots it does not have; slots past a row hold -inf.
#define DASH_BUCKETS(NS_, CALL)                                                                 \
    if ((NS_) <= 4) CALL(4);                                                                    \
    else if ((NS_) <= 8) CALL(8);                                                               \
    else if ((NS_) <= 12) CALL(12);                                                             \
    else if ((NS_) <= 16) CALL(16);                                                             \
    else if (CMAX >= 512 && (NS_) <= 20) CALL(CMAX >= 512 ? 20 : 16);                           \
    else if (CMAX >= 512 && (NS_) <= 24) CALL(CMAX >= 512 ? 24 : 16);                           \
    else if (CMAX >= 512 && (NS_) <= 28) CALL(CMAX >= 512 ? 28 : 16);                           \
    else if (CMAX >= 512 && (NS_) <= 32) CALL(CMAX >= 512 ? 32 : 16);                           \
    else if (CMAX >= 1024 && (NS_) <= 40) CALL(CMAX >= 1024 ? 40 : 16);                         \
    else if (CMAX >= 1024 && (NS_) <= 48) CALL(CMAX >= 1024 ? 48 : 16);                         \
    else if (CMAX >= 1024 && (NS_) <= 56) CALL(CMAX >= 1024 ? 56 : 16);                         \
    else if (CMAX >= 1024) CALL(CMAX >= 1024 ? 64 : 16)
    auto slots_of = [&](int tok) {  // 16-lane slots of a token's row
        return div_up(route_cands(p, route_pos(p, b, min(tok, p.n_q - 1))), 16);
    };
    if constexpr (GQ <= 4) {
        for (int u = wave; u < ROWS / 4; u += NW) {
            const int row0 = u * 4;
            const int ns = slots_of(tile0 + (row0 + 3) / GQ);
#define DASH_UNIT(NS) route_unit<NS, KIND, GQ>(xs + row0 * XS, XS, row0, tile0, b, r, mask, bias, tau_out, p)
            DASH_BUCKETS(ns, DASH_UNIT);
#undef DASH_UNIT
        }
    } else {
        for (int u = wave; u < ROWS / 4; u += NW) {
            const int row0 = u * 4;
            const int ns = slots_of(tile0 + row0 / GQ);
#define DASH_PASS(NS) route_head_pass<NS, KIND, GQ>(xs + row0 * XS, XS, row0, tile0, b, r, tau_out, p)
            DASH_BUCKETS(ns, DASH_PASS);
#undef DASH_PASS
        }
        __syncthreads();
        for (int t = wave; t < T; t += NW) {
            const int ns = slots_of(tile0 + t);
#define DASH_FINISH(NS) route_finish_token<NS, GQ>(xs + t * GQ * XS, XS, tile0 + t, b, r, mask, bias, p)
            DASH_BUCKETS(ns, DASH_FINISH);
#undef DASH_FINISH
        }
    }
#undef DASH_BUCKETS
}

// (MT, NW) with NW * MT * 32 >= tc chunks: up to 1024 chunks (8 waves of 4 tiles); 1025 to 2048
// chunks in route_long_kernel
bool route_fused_supported(const RouteParams& p, int dt) {
    if (dt != kBF16 || p.n_q <= 1) return false;
    return p.tc <= 1024 ? p.nw <= 32 : p.tc <= kLongMax;
}

template <int D, int GQ, int MT, int NW, int NR>
static void launch_fused_shape(const void* q, const bf16_t* kbar, uint32_t* mask, float* bias,
                               float* tau, const RouteParams& p, float coef, hipStream_t st) {
    constexpr int T = 32 * NR / GQ;
    const int n_tiles = div_up(p.n_q, T);
    dim3 grid(p.batch * p.h_kv * n_tiles), block(NW * 64);
    const int kind = pow_kind(p.alpha);
#define DASH_FUSED(K)                                                                        \
    hipLaunchKernelGGL((route_fused_kernel<D, GQ, MT, NW, NR, K>), grid, block, 0, st,      \
                       static_cast<const bf16_t*>(q), kbar, mask, bias, tau, p, n_tiles, coef)
    if (kind == kPowOne) DASH_FUSED(kPowOne);
    else if (kind == kPowTwo) DASH_FUSED(kPowTwo);
    else DASH_FUSED(kPowGeneral);
#undef DASH_FUSED
}

// (MT, NW, NR) per row length: 32 query rows per workgroup (the LDS of their score rows), 4 to 8
// waves. Past 512 chunks eight waves of four tiles each: 32 rows give phase 2 no more than 8
// units, and eight waves leave each one 256 registers for the 64-slot rows.
template <int D, int GQ>
static void launch_fused_g(const void* q, const bf16_t* kbar, uint32_t* mask, float* bias,
                           float* tau, const RouteParams& p, float coef, hipStream_t st) {
    if (p.tc <= 256) launch_fused_shape<D, GQ, 2, 4, 1>(q, kbar, mask, bias, tau, p, coef, st);
    else if (p.tc <= 512) launch_fused_shape<D, GQ, 2, 8, 1>(q, kbar, mask, bias, tau, p, coef, st);
    else launch_fused_shape<D, GQ, 4, 8, 1>(q, kbar, mask, bias, tau, p, coef, st);
}

// Rows of 1025 to 2048 chunks. 32 score rows of that length do not fit the LDS, so a workgroup
// of 16 waves owns 16 query rows (16 / g tokens times the g heads) of one (sequence b, KV group r)
// and their score rows take 132 KiB:
//   phase 1: X^T = Kbar Q^T from the same three bf16 terms as route_fused_kernel, on
//            v_mfma_f32_16x16x32_bf16 (16 chunks x 16 rows per product); wave w takes the
//            chunk tiles w, w + 16, ..., two at a time, and writes their scores to LDS;
//   phase 2: wave w solves row w's threshold with the row over the whole wave (entry c in lane
//            c % 64, slot c / 64) and leaves the row's probabilities in its LDS row;
//   phase 3: per token the waves split the chunks, 128 each: the GQA mean, mu (summed over the
//            waves in order), the mask words and the bias.
template <int D, int GQ, int KIND>
__global__ __launch_bounds__(1024) void route_long_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ planes, uint32_t* __restrict__ mask,
    float* __restrict__ bias, float* __restrict__ tau_out, RouteParams p, int n_tiles,
    float coef) {
    constexpr int NW = 16;
    constexpr int T = kLongRows / GQ;     // tokens per workgroup
    constexpr int XS = kLongMax + 17;     // LDS row stride of the scores
    constexpr int QS = D + 8;             // LDS row stride of Q (elements)
    __shared__ __align__(16) float xs[kLongRows * XS];
    __shared__ __align__(16) bf16_t qs[kLongRows * QS];
    __shared__ float st_s[NW];
    __shared__ float st_n[NW];

    const int bh = p.batch * p.h_kv;
    const int x = blockIdx.x;
    const int gr = bh % 8 == 0 ? (x % 8) + 8 * ((x / 8) % (bh / 8)) : x % bh;
    const int tile = n_tiles - 1 - x / bh;
    const int b = gr / p.h_kv, r = gr % p.h_kv;
    const int tile0 = tile * T;
    const int tile_end = min(tile0 + T, p.n_q);
    const int m_max = route_cands(p, route_pos(p, b, tile_end - 1));
    const int n_ct = div_up(m_max, 32);
    const int ct_n = div_up(p.tc, 32);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---- phase 1
    for (int idx = tid; idx < kLongRows * (D / 8); idx += NW * 64) {
        const int row = idx / (D / 8), d8 = idx % (D / 8);
        const int t = tile0 + row / GQ;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (t < p.n_q)
            u = *reinterpret_cast<const uint4*>(
                q + (((int64_t)b * p.n_q + t) * p.h_q + r * GQ + row % GQ) * D + 8 * d8);
        *reinterpret_cast<uint4*>(&qs[row * QS + 8 * d8]) = u;
    }
    __syncthreads();
    // 16 x 16 x 32 products: A = 16 chunks x 32 dims of a summary term (lane l: chunk l % 16,
    // dims 8 (l / 16) .. + 7, one 16-byte piece of the fragment-ordered terms), B = the 16 rows'
    // Q (lane l: row l % 16, the same dims), C = 16 chunks x 16 rows. Wave w takes the chunk tiles
    // w, w + 16, ..., two at a time, each as two halves of 16 chunks.
    const int ci = lane & 15, jg = lane >> 4;
    bf16x8_t qb[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        qb[kk] = *reinterpret_cast<const bf16x8_t*>(&qs[ci * QS + 32 * kk + 8 * jg]);
    for (int c0 = wave; c0 < n_ct; c0 += 2 * NW) {
        const bool two = c0 + NW < n_ct;
        f32x4_t X[2][2] = {{f32x4_t{}, f32x4_t{}}, {f32x4_t{}, f32x4_t{}}};
        const uint4* base[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            base[i] = reinterpret_cast<const uint4*>(planes) +
                      ((int64_t)(b * p.h_kv + r) * ct_n + min(c0 + NW * i, ct_n - 1)) * (D / 16) * 3 * 64;
        // step s: k-step kk = s / 3 of 32 dims, term lo, mid, hi (the small terms first); the
        // 16-dim slice ks = 2 kk + jg / 2 of the fragment order holds dims 8 (jg % 2) .. + 7 in
        // lanes 32 .. 63 of its 64
        constexpr int NSTEP = 3 * (D / 32);
        auto load = [&](int st, uint4 (&dst)[2][2]) __attribute__((always_inline)) {
            const int kk = st / 3, pl = 2 - st % 3;
            const int ks = 2 * kk + (jg >> 1);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    dst[i][h] = base[i][(ks * 3 + pl) * 64 + 16 * h + ci + 32 * (jg & 1)];
        };
        uint4 cur[2][2], nxt[2][2];
        load(0, cur);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            if (st + 1 < NSTEP) load(st + 1, nxt);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (i == 1 && !two) break;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    X[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, cur[i][h]), qb[st / 3], X[i][h], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h) cur[i][h] = nxt[i][h];
        }
        // lane l holds row l % 16, chunks 32 ct + 16 h + 4 (l / 16) + {0..3}
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i == 1 && !two) break;
            const int ct = c0 + NW * i;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2)
                    xs[ci * XS + 32 * ct + 16 * h + 4 * jg + e2] = coef * X[i][h][e2];
        }
    }
    __syncthreads();

    // ---- phase 2: wave w owns row w
    {
        const int row = wave;
        const int tok = tile0 + row / GQ;
        const bool tvalid = tok < p.n_q;
        const int m = tvalid ? route_cands(p, route_pos(p, b, tok)) : 0;
        const int ns = div_up(m, 64);
        float* xr = xs + row * XS;
        const float e = 1.0f / (p.alpha - 1.0f);
        auto solve = [&](auto nsc) __attribute__((always_inline)) {
            constexpr int NS = decltype(nsc)::value;
            float xv[NS];
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int c = 64 * i + lane;
                xv[i] = c < m ? xr[c] : -INFINITY;
            }
            // Long rows: the threshold restricted to a subset of the row is a lower bound on the
            // row's threshold, since dropping entries only lowers the sum of Eq. 2. The subset is
            // the 16 maxima of lanes l, l + 16, l + 32, l + 48 (solved within each 16-lane row,
            // all four rows alike). Entries at or below that bound (less a margin) are outside the
            // support; one pass packs those above it into the wave's own LDS row (its scores are
            // in xv) and counts them, and when at most kLongCand remain the threshold is solved on
            // that list, which has the same root. Otherwise the whole row is solved.
            float tau;
            bool packed = false;
            if (NS >= 16 && m > kLongCand) {
                float lm = -INFINITY;
#pragma unroll
                for (int i = 0; i < NS; ++i) lm = fmaxf(lm, xv[i]);
                lm = halves_max(rowpair_max(lm));  // lanes l, l ^ 16, l ^ 32, l ^ 48
                const float lmv[1] = {lm};
                const float tl = solve_tau_exact<1, KIND, 16>(lmv, 1, 16, p.alpha);
                const float lo = tl - 1e-3f * fmaxf(1.0f, fabsf(tl));
                const uint64_t below = (1ull << lane) - 1ull;
                int cnt = 0;
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const bool in = xv[i] > lo;
                    const uint64_t bal = __ballot(in);
                    const int at = cnt + __popcll(bal & below);
                    if (in && at < kLongCand) xr[at] = xv[i];
                    cnt += __popcll(bal);
                }
                if (cnt <= kLongCand) {
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    float cv[kLongCand / 64];
#pragma unroll
                    for (int i = 0; i < kLongCand / 64; ++i)
                        cv[i] = 64 * i + lane < cnt ? xr[64 * i + lane] : -INFINITY;
                    tau = solve_tau_exact<kLongCand / 64, KIND, 64>(cv, (cnt + 63) / 64, cnt, p.alpha);
                    packed = true;
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            if (!packed) tau = solve_tau_exact<NS, KIND, 64>(xv, ns, m, p.alpha);
            if (tau_out && tvalid && lane == 0)
                tau_out[((int64_t)b * p.n_q + tok) * p.h_q + r * GQ + row % GQ] = tau;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int c = 64 * i + lane;
                if (c < m) xr[c] = pow_e<KIND>(xv[i] - tau, e);
            }
        };
        if (ns <= 8) solve(std::integral_constant<int, 8>{});
        else if (ns <= 16) solve(std::integral_constant<int, 16>{});
        else solve(std::integral_constant<int, 32>{});
    }
    __syncthreads();

    // ---- phase 3: per token, chunks 128 w .. 128 w + 127 in wave w
    const float inv_g = 1.0f / (float)GQ;
    for (int t = 0; t < T; ++t) {
        const int tok = tile0 + t;
        const bool tvalid = tok < p.n_q;
        const int pos = route_pos(p, b, min(tok, p.n_q - 1));
        const int cp = pos / p.block;
        const int m = route_cands(p, pos);
        float w[2], lw[2];
        float lsum = 0.f, lcnt = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = 128 * wave + 64 * i + lane;
            float sum = 0.f;
            if (c < m) {
#pragma unroll
                for (int h = 0; h < GQ; ++h) sum += xs[(t * GQ + h) * XS + c];
            }
            w[i] = sum * inv_g;
            lw[i] = w[i] > 0.f ? __logf(w[i]) : 0.f;
            lsum += lw[i];
            lcnt += w[i] > 0.f ? 1.f : 0.f;
        }
        lsum = wave_sum(lsum);
        lcnt = wave_sum(lcnt);
        if (lane == 0) {
            st_s[wave] = lsum;
            st_n[wave] = lcnt;
        }
        __syncthreads();
        float tot = 0.f, cnt = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            tot += st_s[i];
            cnt += st_n[i];
        }
        const float mu = cnt > 0.f ? tot / cnt : 0.f;
        const int64_t qrow = (int64_t)b * p.n_q + tok;
        uint32_t* mrow = mask + (qrow * p.h_kv + r) * p.nw;
        float* brow = bias + (qrow * p.h_kv + r) * p.nc;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = 128 * wave + 64 * i + lane;
            const bool sel = c < m && w[i] > 0.f;
            if (tvalid && sel) brow[c] = (lw[i] - mu) * p.inv_sigma;
            const uint64_t bal = __ballot(sel || (c >= m && c <= cp));
            const int wd = (128 * wave + 64 * i) / 32;
            if (tvalid && lane == 0 && wd < p.nw) {
                mrow[wd] = (uint32_t)bal;
                if (wd + 1 < p.nw) mrow[wd + 1] = (uint32_t)(bal >> 32);
            }
        }
        // a word past the 2048 chunks holds the window's bits only
        for (int wd = kLongMax / 32 + tid; wd < p.nw; wd += NW * 64)
            if (tvalid) mrow[wd] = span_bits(wd, m, cp);
        for (int c = m + tid; c <= cp; c += NW * 64)
            if (tvalid) brow[c] = 0.f;
        __syncthreads();  // st_s / st_n are read again for the next token
    }
}

template <int D, int GQ>
static void launch_long_g(const void* q, const bf16_t* kbar, uint32_t* mask, float* bias,
                          float* tau, const RouteParams& p, float coef, hipStream_t st) {
    constexpr int T = kLongRows / GQ;
    const int n_tiles = div_up(p.n_q, T);
    dim3 grid(p.batch * p.h_kv * n_tiles), block(1024);
    const int kind = pow_kind(p.alpha);
#define DASH_LONG(K)                                                                        \
    hipLaunchKernelGGL((route_long_kernel<D, GQ, K>), grid, block, 0, st,                  \
                       static_cast<const bf16_t*>(q), kbar, mask, bias, tau, p, n_tiles, coef)
    if (kind == kPowOne) DASH_LONG(kPowOne);
    else if (kind == kPowTwo) DASH_LONG(kPowTwo);
    else DASH_LONG(kPowGeneral);
#undef DASH_LONG
}

template <int D>
static void launch_fused_d(const void* q, const bf16_t* kbar, uint32_t* mask, float* bias,
                           float* tau, const RouteParams& p, float coef, hipStream_t st) {
    if (p.tc > 1024) {
        switch (p.g) {
            case 1: launch_long_g<D, 1>(q, kbar, mask, bias, tau, p, coef, st); break;
            case 2: launch_long_g<D, 2>(q, kbar, mask, bias, tau, p, coef, st); break;
            case 4: launch_long_g<D, 4>(q, kbar, mask, bias, tau, p, coef, st); break;
            case 8: launch_long_g<D, 8>(q, kbar, mask, bias, tau, p, coef, st); break;
            default: launch_long_g<D, 16>(q, kbar, mask, bias, tau, p, coef, st); break;
        }
        return;
    }
    switch (p.g) {
        case 1: launch_fused_g<D, 1>(q, kbar, mask, bias, tau, p, coef, st); break;
        case 2: launch_fused_g<D, 2>(q, kbar, mask, bias, tau, p, coef, st); break;
        case 4: launch_fused_g<D, 4>(q, kbar, mask, bias, tau, p, coef, st); break;
        case 8: launch_fused_g<D, 8>(q, kbar, mask, bias, tau, p, coef, st); break;
        default: launch_fused_g<D, 16>(q, kbar, mask, bias, tau, p, coef, st); break;
    }
}

size_t route_fused_workspace_bytes(const RouteParams& p) {
    return (size_t)p.batch * p.h_kv * div_up(p.tc, 32) * 32 * 3 * p.head_dim * sizeof(bf16_t);
}

hipError_t launch_route_fused(const void* q, const float* kbar, uint32_t* mask, float* bias,
                              float* tau, const RouteParams& p, void* ws, hipStream_t st) {
    const float coef = (p.alpha - 1.0f) * p.gamma / sqrtf((float)p.head_dim);
    bf16_t* planes = static_cast<bf16_t*>(ws);
    if (p.tc > 0) {
        const int64_t n = (int64_t)p.batch * p.h_kv * div_up(p.tc, 32) * (p.head_dim / 16) * 64;
        hipLaunchKernelGGL(split_kbar_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           kbar, planes, p.batch, p.tc, p.h_kv, p.head_dim);
    }
    if (p.head_dim == 64) launch_fused_d<64>(q, planes, mask, bias, tau, p, coef, st);
    else launch_fused_d<128>(q, planes, mask, bias, tau, p, coef, st);
    return hipGetLastError();
}

}  // namespace dash
