// Per-row helpers shared by the Stage 1 route kernels ("DashAttention", arXiv 2605.18753v1,
// §3.2 and §3.4 Prop. 1; App. G Alg. 2).
#pragma once

#include <math.h>

#include "common.h"
#include "entmax.h"
#include "kernels.h"

namespace dash {

// Row c < m of a score row (workspace or LDS) into registers (lane c % 64, slot c / 64), -inf past m.
// The loads are unconditional (indices clamped into the row) so that all of them are in flight
// together; the row is never read when m = 0.
template <int NPL>
__device__ __forceinline__ void load_row(const float* __restrict__ xr, int m, int lane,
                                         float (&xv)[NPL]) {
    const int last = m > 0 ? m - 1 : 0;
    if (m == 0) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) xv[i] = -INFINITY;
        return;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) xv[i] = xr[min(64 * i + lane, last)];
#pragma unroll
    for (int i = 0; i < NPL; ++i)
        if (64 * i + lane >= m) xv[i] = -INFINITY;
}

// Mask words and bias of one (query, group) row from the group-averaged probabilities w held in
// registers (chunk c in lane c % 64, slot c / 64): mu = mean log w over R = {c < m : w_c > 0},
// d_c = (log w_c - mu) / sigma on R; the window's chunks m .. cp (the query's own chunk and the
// blocks before it that are always attended) get their bits and d = 0.
template <int NPL>
__device__ __forceinline__ void write_route_row(const float (&w)[NPL], int m, int cp, int lane,
                                                uint32_t* mrow, float* brow, const RouteParams& p) {
    float sl = 0.f;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
        if (w[i] > 0.f) { sl += __logf(w[i]); ++cnt; }
    sl = wave_sum(sl);
    cnt = wave_sum_int(cnt);
    const float mu = cnt > 0 ? sl / (float)cnt : 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        if (2 * i >= p.nw) break;
        const int c = 64 * i + lane;
        const bool sel = c < m && w[i] > 0.f;
        if (sel) brow[c] = (__logf(w[i]) - mu) * p.inv_sigma;
        const uint64_t bal = __ballot(sel || (c >= m && c <= cp));
        if (lane == 0) {
            mrow[2 * i] = (uint32_t)bal;
            if (2 * i + 1 < p.nw) mrow[2 * i + 1] = (uint32_t)(bal >> 32);
        }
    }
    for (int c = m + lane; c <= cp; c += 64) brow[c] = 0.f;
}

// Reductions of the threshold solver over the WPH waves that hold one row, for a workgroup
// whose waves all run the solver together (each reduction is one barrier). red: LDS scratch of
// 2 x 16 x 6 floats, double-buffered so that one barrier per pass suffices. The loop of the
// solver ends for the whole workgroup once every wave reported done at the start of a pass.
template <int WPH>
struct WaveSetReduce {
    float* red;
    int wave, lane, w0, nwaves;
    int buf;
    bool all_done;
    __device__ float max(float v) {
        v = wave_max(v);
        if (lane == 0) red[wave * 6] = v;
        __syncthreads();
        float m = red[w0 * 6];
#pragma unroll
        for (int i = 1; i < WPH; ++i) m = fmaxf(m, red[(w0 + i) * 6]);
        buf = 1;
        all_done = false;
        return m;
    }
    __device__ bool all(bool) { return all_done; }
    __device__ void gather(float& k, float& p1, float& p2, float& tmin, float& tout, bool done) {
        k = wave_sum(k);
        p1 = wave_sum(p1);
        p2 = wave_sum(p2);
        tmin = wave_min(tmin);
        tout = wave_max(tout);
        float* rb = red + buf * 96;
        if (lane == 0) {
            rb[wave * 6 + 0] = k;
            rb[wave * 6 + 1] = p1;
            rb[wave * 6 + 2] = p2;
            rb[wave * 6 + 3] = tmin;
            rb[wave * 6 + 4] = tout;
            rb[wave * 6 + 5] = done ? 1.f : 0.f;
        }
        __syncthreads();
        k = rb[w0 * 6];
        p1 = rb[w0 * 6 + 1];
        p2 = rb[w0 * 6 + 2];
        tmin = rb[w0 * 6 + 3];
        tout = rb[w0 * 6 + 4];
#pragma unroll
        for (int i = 1; i < WPH; ++i) {
            k += rb[(w0 + i) * 6];
            p1 += rb[(w0 + i) * 6 + 1];
            p2 += rb[(w0 + i) * 6 + 2];
            tmin = fminf(tmin, rb[(w0 + i) * 6 + 3]);
            tout = fmaxf(tout, rb[(w0 + i) * 6 + 4]);
        }
        bool ad = true;
        for (int i = 0; i < nwaves; ++i) ad = ad && rb[i * 6 + 5] != 0.f;
        all_done = ad;
        buf ^= 1;
    }
};

constexpr int kDecCand = 256;  // packed candidates per head row

// LDS that the routing of one (sequence, group) uses, in the calling workgroup.
struct DecodeRouteLds {
    float* red;     // 2 * 16 * 6
    float* stat_s;  // 16
    int* stat_n;    // 16
    int* cand_n;    // 16
    float* tau_h;   // 16
    float* cand;    // 16 * kDecCand
    float* wsum;    // one per chunk of the row
};

// Stage 1 of one query and KV group by a whole workgroup (64 WPH g threads): the g heads' rows
// are each spread over WPH waves (entry c in lane c % 64 of the head's wave (c / 64) % WPH, slot
// c / (64 WPH)), which solve the head's threshold together; the heads' probabilities are added
// in head order in LDS; then every wave takes part in writing the mask words and the bias.
// xat(hh, c): score c of head hh of the group (m entries, c < m the routing candidates; cp
// the query's own chunk, chunks m .. cp its window). Outputs, each optional (null): the global
// mask row mrow and bias row brow (routed entries and the window), tau_out[hh], the mask words
// mw and, for every chunk whose bit is set, its bias bl[c] (both in LDS, for a fused Stage 2).
template <int NS, int KIND, int WPH, class XAT>
__device__ __forceinline__ void decode_route_group(XAT xat, int m, int cp, const RouteParams& p,
                                                   const DecodeRouteLds& s, uint32_t* mrow,
                                                   float* brow, float* tau_out, uint32_t* mw,
                                                   float* bl) {
    constexpr int L = 64 * WPH;  // lanes per row
    float* red = s.red;
    float* stat_s = s.stat_s;
    int* stat_n = s.stat_n;
    int* cand_n = s.cand_n;
    float* tau_h = s.tau_h;
    float* cand = s.cand;
    float* wsum = s.wsum;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int hh = wave / WPH, wq = wave % WPH;
    const int ns = (m + L - 1) / L;
    const float e = 1.0f / (p.alpha - 1.0f);

    // the row, loads unconditional (clamped into the row) so that all are in flight together
    const int last = m > 0 ? m - 1 : 0;
    float xv[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) xv[i] = xat(hh, min(i * L + wq * 64 + lane, last));
#pragma unroll
    for (int i = 0; i < NS; ++i)
        if (i * L + wq * 64 + lane >= m) xv[i] = -INFINITY;

    // tau never falls below max x - 1, so only entries above it can enter the support. When no
    // head has more than kDecCand of them, they are packed into LDS and each head's first wave
    // solves on its packed list alone; otherwise the head's waves solve on the whole row.
    WaveSetReduce<WPH> rd{red, wave, lane, hh * WPH, nwaves, 0, false};
    float xm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NS; ++i) xm = fmaxf(xm, xv[i]);
    const float lo = rd.max(xm) - 1.0f;
    int ncand = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) ncand += __popcll(__ballot(xv[i] > lo));
    if (lane == 0) cand_n[wave] = ncand;
    __syncthreads();
    int before = 0, head_n = 0, most = 0;
    for (int w = 0; w < nwaves; ++w) {
        const int cw = cand_n[w];
        if (w / WPH == hh) {
            head_n += cw;
            before += w < wave ? cw : 0;
        }
        if (w % WPH == WPH - 1) {
            int hn = 0;
            for (int v = w - WPH + 1; v <= w; ++v) hn += cand_n[v];
            most = max(most, hn);
        }
    }
    float tau;
    if (most <= kDecCand) {
        const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const bool in = xv[i] > lo;
            const uint64_t bal = __ballot(in);
            if (in) cand[hh * kDecCand + before + __popcll(bal & below)] = xv[i];
            before += __popcll(bal);
        }
        __syncthreads();
        if (wq == 0) {
            float cv[kDecCand / 64];
#pragma unroll
            for (int i = 0; i < kDecCand / 64; ++i)
                cv[i] = 64 * i + lane < head_n ? cand[hh * kDecCand + 64 * i + lane] : -INFINITY;
            const float t = solve_tau_exact<kDecCand / 64, KIND, 64>(cv, (head_n + 63) / 64, head_n, p.alpha);
            if (lane == 0) tau_h[hh] = t;
        }
        __syncthreads();
        tau = tau_h[hh];
    } else {
        tau = solve_tau_core<NS, KIND>(xv, ns, m, p.alpha, rd);
    }
    if (tau_out && wq == 0 && lane == 0) tau_out[hh] = tau;

    for (int g0 = 0; g0 < p.g; ++g0) {
        if (hh == g0) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int c = i * L + wq * 64 + lane;
                if (c < m) {
                    const float pv = pow_e<KIND>(xv[i] - tau, e);
                    wsum[c] = g0 == 0 ? pv : wsum[c] + pv;
                }
            }
        }
        __syncthreads();
    }

    // mu = mean of log w over R, in a fixed order (waves, then lanes by DPP)
    const float inv_g = 1.0f / (float)p.g;
    float sl = 0.f;
    int cnt = 0;
    for (int c = tid; c < m; c += blockDim.x) {
        const float w = wsum[c] * inv_g;
        if (w > 0.f) {
            sl += __logf(w);
            ++cnt;
        }
    }
    sl = wave_sum(sl);
    cnt = wave_sum_int(cnt);
    if (lane == 0) {
        stat_s[wave] = sl;
        stat_n[wave] = cnt;
    }
    __syncthreads();
    float tot = 0.f;
    int n_r = 0;
    for (int i = 0; i < nwaves; ++i) {
        tot += stat_s[i];
        n_r += stat_n[i];
    }
    const float mu = n_r > 0 ? tot / (float)n_r : 0.f;
    for (int base = wave * 64; base < p.nw * 32; base += nwaves * 64) {
        const int c = base + lane;
        const float w = c < m ? wsum[c] * inv_g : 0.f;
        const bool sel = c < m && w > 0.f;
        const bool win = c >= m && c <= cp;  // the window: always attended, d = 0
        const float d = sel ? (__logf(w) - mu) * p.inv_sigma : 0.f;
        if (sel && brow) brow[c] = d;
        if (bl && (sel || win)) bl[c] = d;
        const uint64_t bal = __ballot(sel || win);
        if (lane == 0) {
            const uint32_t w0 = (uint32_t)bal, w1 = (uint32_t)(bal >> 32);
            if (mrow) {
                mrow[base / 32] = w0;
                if (base / 32 + 1 < p.nw) mrow[base / 32 + 1] = w1;
            }
            if (mw) {
                mw[base / 32] = w0;
                if (base / 32 + 1 < p.nw) mw[base / 32 + 1] = w1;
            }
        }
    }
    if (brow)
        for (int c = m + tid; c <= cp; c += blockDim.x) brow[c] = 0.f;
}


}  // namespace dash
