// Stage 1: alpha-entmax chunk routing ("DashAttention", arXiv 2605.18753v1, §3.2 Eq. 4,
// §3.4 Prop. 1; App. G Alg. 2).
//
// Two kernels. A score kernel computes the entmax arguments
//     x[b, t, h, c] = (alpha - 1) * gamma * <q_t^(h), kbar_c^(h / g)> / sqrt(D),   c < c_t
// into a workspace; a route kernel then solves each head's threshold tau on the row held in
// LDS, averages the group's probabilities and writes the bit-packed mask and the bias.
// Many queries with bf16 inputs and up to 2048 chunks run in one pass instead (route_fused.hip).
// Other many-query cases: score_kernel (64 x 64 tiles) and route_kernel (one wave per query and
// group).
// One query per sequence (decode): score_one_kernel (a coalesced stream over the summaries) and
// route_decode_kernel (one workgroup per group, several waves per head; route_group_kernel, one
// wave per head, for rows too long for it).
#include <math.h>

#include "common.h"
#include "entmax.h"
#include "kernels.h"
#include "route_common.h"

namespace dash {

// ----------------------------------------------------------------------------- scores

constexpr int kScoreTile = 64;  // rows (query, head) x chunks per workgroup

template <typename T, int D>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ q,
                                                    const float* __restrict__ kbar,
                                                    float* __restrict__ x, RouteParams p,
                                                    float coef) {
    const int b = blockIdx.z / p.h_kv, r = blockIdx.z % p.h_kv;
    const int row0 = blockIdx.y * kScoreTile, c0 = blockIdx.x * kScoreTile;
    const int rows_total = p.n_q * p.g;
    const int row_last = min(row0 + kScoreTile, rows_total) - 1;
    const int m_last = route_cands(p, route_pos(p, b, row_last / p.g));
    if (c0 >= m_last) return;  // every row of this tile sees fewer chunks (uniform exit)

    // D is consumed in slices of 32: 64 x 32 tiles of Q and kbar in LDS (one 8-element load
    // per thread and tile), 4 x 4 outputs per thread at rows ty + 16 i and chunks tx + 16 j.
    __shared__ float qs[kScoreTile][33];
    __shared__ float ks[kScoreTile][33];
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int lr = tid / 4, le = (tid % 4) * 8;
    const int lrow = row0 + lr, lc = c0 + lr;
    const T* qsrc = nullptr;
    if (lrow < rows_total) {
        const int t = lrow / p.g, gg = lrow % p.g;
        qsrc = q + (((int64_t)b * p.n_q + t) * p.h_q + r * p.g + gg) * D;
    }
    const float* ksrc = lc < p.tc ? kbar + (((int64_t)b * p.tc + lc) * p.h_kv + r) * D : nullptr;
    float acc[4][4] = {};
    for (int e0 = 0; e0 < D; e0 += 32) {
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float w[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (qsrc) load8(qsrc + e0 + le, v);
        if (ksrc) load8(ksrc + e0 + le, w);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            qs[lr][le + j] = v[j];
            ks[lr][le + j] = w[j];
        }
        __syncthreads();
#pragma unroll 8
        for (int e = 0; e < 32; ++e) {
            float a[4], bb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = qs[ty + 16 * i][e];
#pragma unroll
            for (int j = 0; j < 4; ++j) bb[j] = ks[tx + 16 * j][e];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = row0 + ty + 16 * i;
        if (row >= rows_total) continue;
        const int t = row / p.g, gg = row % p.g;
        const int m = route_cands(p, route_pos(p, b, t));
        float* xr = x + (((int64_t)b * p.n_q + t) * p.h_q + r * p.g + gg) * p.nc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = c0 + tx + 16 * j;
            if (c < m) xr[c] = coef * acc[i][j];
        }
    }
}

// ----------------------------------------------------------------------------- one query per row

// Scores of a single query per sequence (decode): a bandwidth-bound stream over the cached
// summaries. A quad of lanes owns one chunk summary: lane k of the quad loads 16-byte pieces
// k, k + 4, ... of the row (all of its loads in flight at once), forms partial dot products
// with every head of the group (the group's queries sit in LDS and are read as broadcasts), and
// two DPP steps sum the quad; lane k then writes heads k, k + 4, ....
// One workgroup of nthreads threads scores chunks c0 .. c0 + nthreads / 4 - 1 of (b, r); qs holds
// g * D floats of LDS. Ends without a barrier after its stores.
// Decode scores: each workgroup takes kScoreOneIter groups of 64 consecutive chunks of one
// (sequence, group), a quad of lanes per summary (16-byte loads, 128 or 64 bytes per lane and
// summary); the loads of all its groups are issued before any is used. The quad's partial dot
// products meet by two DPP swaps. One group per workgroup is the fastest on the 16 x 128K step
// (60.9 us; two groups 62.1, four 65.1): more workgroups in flight beat more loads per lane.
constexpr int kScoreOneIter = 1;

template <typename T, int D>
__global__ __launch_bounds__(256) void score_one_kernel(const T* __restrict__ q,
                                                        const float* __restrict__ kbar,
                                                        float* __restrict__ x, RouteParams p,
                                                        float coef) {
    constexpr int NV = D / 16;  // float4 pieces per lane and summary
    constexpr int IT = kScoreOneIter;
    __shared__ __align__(16) float qs[16 * D];
    const int b = blockIdx.y / p.h_kv, r = blockIdx.y % p.h_kv;
    const int m = route_cands(p, route_pos(p, b, 0));  // complete chunks before the window
    const int c_wg = blockIdx.x * 64 * IT;
    if (c_wg >= m) return;  // no chunk of this workgroup is a candidate (uniform)
    const int tid = threadIdx.x;
    const int k = tid & 3;
    float4 kv[IT][NV];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int c = c_wg + 64 * it + tid / 4;
        const float4* src = reinterpret_cast<const float4*>(kbar + (((int64_t)b * p.tc + min(c, p.tc - 1)) * p.h_kv + r) * D);
#pragma unroll
        for (int i = 0; i < NV; ++i) kv[it][i] = src[k + 4 * i];
    }
    for (int e = tid; e < p.g * D; e += blockDim.x) {
        const int gg = e / D, d = e % D;
        qs[gg * D + d] = to_f32(q[(((int64_t)b * p.n_q) * p.h_q + r * p.g + gg) * D + d]);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int c = c_wg + 64 * it + tid / 4;
        for (int g0 = 0; g0 < p.g; g0 += 4) {
            float part[4];
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                const int gg = g0 + hh;
                float a = 0.f;
                if (gg < p.g) {
                    const float4* qv = reinterpret_cast<const float4*>(&qs[gg * D]);
#pragma unroll
                    for (int i = 0; i < NV; ++i) {
                        const float4 qq = qv[k + 4 * i];
                        a = fmaf(kv[it][i].x, qq.x, a);
                        a = fmaf(kv[it][i].y, qq.y, a);
                        a = fmaf(kv[it][i].z, qq.z, a);
                        a = fmaf(kv[it][i].w, qq.w, a);
                    }
                }
                // sum over the quad: swap pairs, then halves
                a += dpp_f<0xb1, 0xf>(0.f, a);
                a += dpp_f<0x4e, 0xf>(0.f, a);
                part[hh] = a;
            }
            const int gg = g0 + k;
            if (c < m && gg < p.g)
                x[(((int64_t)b * p.n_q) * p.h_q + r * p.g + gg) * p.nc + c] = coef * part[k];
        }
    }
}

// ----------------------------------------------------------------------------- routing

// Many queries: one wave per (query t, group r, sequence b); the g heads in turn, each row read
// once from the score workspace into registers, probabilities summed in registers.
template <int NPL, int KIND>
__global__ __launch_bounds__(64) void route_kernel(const float* __restrict__ x,
                                                   uint32_t* __restrict__ mask,
                                                   float* __restrict__ bias,
                                                   float* __restrict__ tau_out, RouteParams p) {
    const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int pos = route_pos(p, b, t);
    const int cp = pos / p.block;
    const int m = route_cands(p, pos);
    const int64_t qrow = (int64_t)b * p.n_q + t;
    const float e = 1.0f / (p.alpha - 1.0f);
    float w[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) w[i] = 0.f;
    for (int gg = 0; gg < p.g; ++gg) {
        const int h = r * p.g + gg;
        float xv[NPL];
        load_row<NPL>(x + (qrow * p.h_q + h) * p.nc, m, lane, xv);
        float tau = INFINITY;
        if (m > 0) {
            tau = solve_tau_reg<NPL, KIND>(xv, m, p.alpha);
#pragma unroll
            for (int i = 0; i < NPL; ++i) w[i] += pow_e<KIND>(xv[i] - tau, e);
        }
        if (tau_out && lane == 0) tau_out[qrow * p.h_q + h] = tau;
    }
    const float inv_g = 1.0f / (float)p.g;
#pragma unroll
    for (int i = 0; i < NPL; ++i) w[i] *= inv_g;
    write_route_row<NPL>(w, m, cp, lane, mask + (qrow * p.h_kv + r) * p.nw,
                         bias + (qrow * p.h_kv + r) * p.nc, p);
}

// One query per sequence (decode): one wave per head solves its threshold; the probabilities
// meet in LDS (g x 64 NPL floats) and wave 0 writes the row. Heads are added in order.
template <int NPL, int KIND>
__global__ __launch_bounds__(NPL >= 64 ? 256 : 1024) void route_group_kernel(const float* __restrict__ x,
                                                           uint32_t* __restrict__ mask,
                                                           float* __restrict__ bias,
                                                           float* __restrict__ tau_out,
                                                           RouteParams p) {
    const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    extern __shared__ float ps[];
    const int pos = route_pos(p, b, t);
    const int cp = pos / p.block;
    const int m = route_cands(p, pos);
    const int64_t qrow = (int64_t)b * p.n_q + t;
    const float e = 1.0f / (p.alpha - 1.0f);
    if (wave < p.g) {
        const int h = r * p.g + wave;
        const float* xr = x + (qrow * p.h_q + h) * p.nc;
        float xv[NPL];
        load_row<NPL>(xr, m, lane, xv);
        float tau = INFINITY;
        if (m > 0) tau = solve_tau_reg<NPL, KIND>(xv, m, p.alpha);
#pragma unroll
        for (int i = 0; i < NPL; ++i) ps[(wave * NPL + i) * 64 + lane] = m > 0 ? pow_e<KIND>(xv[i] - tau, e) : 0.f;
        if (tau_out && lane == 0) tau_out[qrow * p.h_q + h] = tau;
    }
    __syncthreads();
    if (wave != 0) return;
    const float inv_g = 1.0f / (float)p.g;
    float w[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        float s = 0.f;
        for (int gg = 0; gg < p.g; ++gg) s += ps[(gg * NPL + i) * 64 + lane];
        w[i] = s * inv_g;
    }
    write_route_row<NPL>(w, m, cp, lane, mask + (qrow * p.h_kv + r) * p.nw,
                         bias + (qrow * p.h_kv + r) * p.nc, p);
}

// One query per sequence (decode): one workgroup per (sequence, group), scores from the
// workspace (see decode_route_group).
template <int NS, int KIND, int WPH>
__global__ __launch_bounds__(1024) void route_decode_kernel(const float* __restrict__ x,
                                                            uint32_t* __restrict__ mask,
                                                            float* __restrict__ bias,
                                                            float* __restrict__ tau_out,
                                                            RouteParams p) {
    __shared__ float red[2 * 16 * 6];
    __shared__ float stat_s[16];
    __shared__ int stat_n[16];
    __shared__ int cand_n[16];
    __shared__ float tau_h[16];
    __shared__ float cand[16 * kDecCand];
    extern __shared__ float wsum[];  // group sum of probabilities, one per chunk
    const int r = blockIdx.x, b = blockIdx.y;
    const int pos = route_pos(p, b, 0);
    const DecodeRouteLds lds{red, stat_s, stat_n, cand_n, tau_h, cand, wsum};
    const float* xg = x + ((int64_t)b * p.h_q + (int64_t)r * p.g) * p.nc;
    decode_route_group<NS, KIND, WPH>([&](int hh, int c) { return xg[(int64_t)hh * p.nc + c]; },
                                      route_cands(p, pos), pos / p.block, p, lds,
                                      mask + ((int64_t)b * p.h_kv + r) * p.nw,
                                      bias + ((int64_t)b * p.h_kv + r) * p.nc,
                                      tau_out ? tau_out + (int64_t)b * p.h_q + r * p.g : nullptr,
                                      nullptr, nullptr);
}

// waves per head row of route_decode_kernel (16 waves at most), and its slots per lane
__host__ inline int route_decode_wph(int g) { return g <= 4 ? 4 : 16 / g; }
__host__ inline int route_decode_slots(const RouteParams& p) {
    int ns = 1;
    while (ns * 64 * route_decode_wph(p.g) < p.tc) ns *= 2;
    return ns;
}

template <int NS, int WPH>
static void launch_route_decode_ns(const float* x, uint32_t* mask, float* bias, float* tau,
                                   const RouteParams& p, hipStream_t st) {
    const int kind = pow_kind(p.alpha);
    const size_t lds = (size_t)(p.tc > 0 ? p.tc : 1) * sizeof(float);
    dim3 grid(p.h_kv, p.batch), block(64 * WPH * p.g);
#define DASH_RD(K) hipLaunchKernelGGL((route_decode_kernel<NS, K, WPH>), grid, block, lds, st, \
                                      x, mask, bias, tau, p)
    if (kind == kPowOne) DASH_RD(kPowOne); else if (kind == kPowTwo) DASH_RD(kPowTwo); else DASH_RD(kPowGeneral);
#undef DASH_RD
}

template <int WPH>
static void launch_route_decode_wph(const float* x, uint32_t* mask, float* bias, float* tau,
                                    const RouteParams& p, hipStream_t st) {
    switch (route_decode_slots(p)) {
        case 1: launch_route_decode_ns<1, WPH>(x, mask, bias, tau, p, st); break;
        case 2: launch_route_decode_ns<2, WPH>(x, mask, bias, tau, p, st); break;
        case 4: launch_route_decode_ns<4, WPH>(x, mask, bias, tau, p, st); break;
        case 8: launch_route_decode_ns<8, WPH>(x, mask, bias, tau, p, st); break;
        case 16: launch_route_decode_ns<16, WPH>(x, mask, bias, tau, p, st); break;
        default: launch_route_decode_ns<32, WPH>(x, mask, bias, tau, p, st); break;
    }
}

static void launch_route_decode(const float* x, uint32_t* mask, float* bias, float* tau,
                                const RouteParams& p, hipStream_t st) {
    switch (route_decode_wph(p.g)) {
        case 4: launch_route_decode_wph<4>(x, mask, bias, tau, p, st); break;
        case 2: launch_route_decode_wph<2>(x, mask, bias, tau, p, st); break;
        default: launch_route_decode_wph<1>(x, mask, bias, tau, p, st); break;
    }
}

// Many queries off the fused path score through the workspace in slabs of query rows, so that it
// never holds more than kRouteSlabBytes (a 256K-token prefill would otherwise need 64 GiB).
constexpr size_t kRouteSlabBytes = (size_t)512 << 20;

static size_t score_row_bytes(const RouteParams& p) { return (size_t)p.h_q * p.nc * sizeof(float); }

// query rows per slab (of one sequence), or 0 when the whole call fits one workspace
static int route_slab_rows(const RouteParams& p) {
    if (p.n_q == 1 || (size_t)p.batch * p.n_q * score_row_bytes(p) <= kRouteSlabBytes) return 0;
    const size_t rows = kRouteSlabBytes / score_row_bytes(p);
    return (int)(rows < 1 ? 1 : (rows < (size_t)p.n_q ? rows : (size_t)p.n_q));
}

size_t route_workspace_bytes(const RouteParams& p, int dt) {
    if (route_fused_supported(p, dt)) return route_fused_workspace_bytes(p);  // scores stay on chip
    const int slab = route_slab_rows(p);
    if (slab > 0) return (size_t)slab * score_row_bytes(p);
    return (size_t)p.batch * p.n_q * score_row_bytes(p);
}

template <int NPL>
static void launch_route_npl(bool group, const float* x, uint32_t* mask, float* bias, float* tau,
                             const RouteParams& p, hipStream_t st) {
    const int kind = pow_kind(p.alpha);
    if (group) {
        const int threads = (p.g < 4 ? 4 : p.g) * kWave;
        const size_t lds = (size_t)p.g * NPL * 64 * sizeof(float);
        dim3 grid(p.n_q, p.h_kv, p.batch);
#define DASH_RG(K) hipLaunchKernelGGL((route_group_kernel<NPL, K>), grid, dim3(threads), lds, st, \
                                      x, mask, bias, tau, p)
        if (kind == kPowOne) DASH_RG(kPowOne); else if (kind == kPowTwo) DASH_RG(kPowTwo); else DASH_RG(kPowGeneral);
#undef DASH_RG
    } else {
        dim3 grid(p.n_q, p.h_kv, p.batch);
#define DASH_RR(K) hipLaunchKernelGGL((route_kernel<NPL, K>), grid, dim3(64), 0, st, x, mask, bias, tau, p)
        if (kind == kPowOne) DASH_RR(kPowOne); else if (kind == kPowTwo) DASH_RR(kPowTwo); else DASH_RR(kPowGeneral);
#undef DASH_RR
    }
}

static void launch_route(bool group, const float* x, uint32_t* mask, float* bias, float* tau,
                         const RouteParams& p, hipStream_t st) {
    switch (slots_for(p.nc)) {
        case 1: launch_route_npl<1>(group, x, mask, bias, tau, p, st); break;
        case 2: launch_route_npl<2>(group, x, mask, bias, tau, p, st); break;
        case 4: launch_route_npl<4>(group, x, mask, bias, tau, p, st); break;
        case 8: launch_route_npl<8>(group, x, mask, bias, tau, p, st); break;
        case 16: launch_route_npl<16>(group, x, mask, bias, tau, p, st); break;
        case 32: launch_route_npl<32>(group, x, mask, bias, tau, p, st); break;
        case 64: launch_route_npl<64>(group, x, mask, bias, tau, p, st); break;
        default: launch_route_npl<128>(group, x, mask, bias, tau, p, st); break;
    }
}

// one query per sequence: a coalesced stream over the summaries into x [B, H_q, Nc]
hipError_t launch_score_one(const void* q, int dt, const float* kbar, float* x,
                            const RouteParams& p, hipStream_t st) {
    const float coef = (p.alpha - 1.0f) * p.gamma / sqrtf((float)p.head_dim);
    dim3 grid(div_up(p.tc, 64 * kScoreOneIter), p.batch * p.h_kv);
#define DASH_SCORE1(T, DD)                                                                 \
    hipLaunchKernelGGL((score_one_kernel<T, DD>), grid, dim3(256), 0, st,                  \
                       static_cast<const T*>(q), kbar, x, p, coef)
    if (dt == kBF16) {
        if (p.head_dim == 64) DASH_SCORE1(bf16_t, 64); else DASH_SCORE1(bf16_t, 128);
    } else {
        if (p.head_dim == 64) DASH_SCORE1(float, 64); else DASH_SCORE1(float, 128);
    }
#undef DASH_SCORE1
    return hipGetLastError();
}

hipError_t launch_block_entmax(const void* q, int dt, const float* kbar, const RouteParams& p,
                               uint32_t* mask, float* bias, float* tau, void* ws,
                               hipStream_t st) {
    if (route_fused_supported(p, dt)) return launch_route_fused(q, kbar, mask, bias, tau, p, ws, st);
    const int slab = route_slab_rows(p);
    if (slab > 0) {
        // one sequence and up to `slab` query rows at a time through the workspace
        const size_t qe = dt == kBF16 ? sizeof(bf16_t) : sizeof(float);
        for (int b = 0; b < p.batch; ++b)
            for (int t0 = 0; t0 < p.n_q; t0 += slab) {
                RouteParams ps = p;
                ps.batch = 1;
                ps.n_q = p.n_q - t0 < slab ? p.n_q - t0 : slab;
                ps.q_pos0 = p.q_pos0 + t0;
                const int64_t row = (int64_t)b * p.n_q + t0;
                const hipError_t e = launch_block_entmax(
                    static_cast<const char*>(q) + row * p.h_q * p.head_dim * qe, dt,
                    kbar + (int64_t)b * p.tc * p.h_kv * p.head_dim, ps, mask + row * p.h_kv * p.nw,
                    bias + row * p.h_kv * p.nc, tau ? tau + row * p.h_q : nullptr, ws, st);
                if (e != hipSuccess) return e;
            }
        return hipSuccess;
    }
    float* x = static_cast<float*>(ws);
    const float coef = (p.alpha - 1.0f) * p.gamma / sqrtf((float)p.head_dim);
    const size_t group_lds = (size_t)p.g * slots_for(p.nc) * 64 * sizeof(float);
    const bool one = p.n_q == 1;
    if (p.tc > 0) {
        if (one) {
            const hipError_t e = launch_score_one(q, dt, kbar, x, p, st);
            if (e != hipSuccess) return e;
        } else {
            dim3 grid(div_up(p.tc, kScoreTile), div_up(p.n_q * p.g, kScoreTile), p.batch * p.h_kv);
#define DASH_SCORE(T, DD)                                                                    \
            hipLaunchKernelGGL((score_kernel<T, DD>), grid, dim3(256), 0, st,                    \
                               static_cast<const T*>(q), kbar, x, p, coef)
            if (dt == kBF16) {
                if (p.head_dim == 64) DASH_SCORE(bf16_t, 64); else DASH_SCORE(bf16_t, 128);
            } else {
                if (p.head_dim == 64) DASH_SCORE(float, 64); else DASH_SCORE(float, 128);
            }
#undef DASH_SCORE
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (one && route_decode_slots(p) <= 32) {
        launch_route_decode(x, mask, bias, tau, p, st);
        return hipGetLastError();
    }
    // the per-head kernel runs up to 16 waves (64 slots and more: up to 4, for its registers)
    const bool group = one && group_lds <= 128 * 1024 && (slots_for(p.nc) < 64 || p.g <= 4);
    launch_route(group, x, mask, bias, tau, p, st);
    return hipGetLastError();
}

}  // namespace dash
