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

}  // namespace dash
