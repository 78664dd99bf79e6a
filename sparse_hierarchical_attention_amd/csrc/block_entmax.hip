// Stage 1: alpha-entmax chunk routing ("DashAttention", arXiv 2605.18753v1, §3.2 Eq. 4,
// §3.4 Prop. 1; App. G Alg. 2).
//
// Two kernels. score_kernel computes the entmax arguments
//     x[b, t, h, c] = (alpha - 1) * gamma * <q_t^(h), kbar_c^(h / g)> / sqrt(D),   c < c_t
// into a workspace; route_kernel then takes one (sequence, query, KV group) per wave, solves
// each head's threshold tau on the row held in LDS, averages the group's probabilities and
// writes the bit-packed mask and the bias.
#include <math.h>

#include "common.h"
#include "kernels.h"

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
    const int m_last = min((p.q_pos0 + row_last / p.g) / p.block, p.tc);
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
        const int m = min((p.q_pos0 + t) / p.block, p.tc);
        float* xr = x + (((int64_t)b * p.n_q + t) * p.h_q + r * p.g + gg) * p.nc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = c0 + tx + 16 * j;
            if (c < m) xr[c] = coef * acc[i][j];
        }
    }
}

// ----------------------------------------------------------------------------- tau

// Exponent kinds of [x - tau]_+^(1/(alpha-1)): alpha = 2 -> 1, alpha = 1.5 -> 2, else general.
enum { kPowGeneral = 0, kPowOne = 1, kPowTwo = 2 };

struct PowE {
    int kind;
    float e;  // 1 / (alpha - 1)
    __device__ __forceinline__ float val(float t) const {  // t^e, t > 0
        if (kind == kPowOne) return t;
        if (kind == kPowTwo) return t * t;
        return exp2f(e * __log2f(t));
    }
    __device__ __forceinline__ float der(float t) const {  // t^(e - 1), t > 0
        if (kind == kPowOne) return 1.0f;
        if (kind == kPowTwo) return t;
        return exp2f((e - 1.0f) * __log2f(t));
    }
};

// Threshold of one row x[0..m-1] (m >= 1) held in LDS, solved by the whole wave.
// f(tau) = sum_c [x_c - tau]_+^e - 1 is decreasing and convex on tau < max x, with the root in
// [max x - 1, max x - m^(1-alpha)]. Newton steps from the left end increase monotonically to
// the root; a bisection step replaces any step that leaves the current bracket (rounding).
// For alpha in {1.5, 2} the result is then polished with the closed form on its support.
__device__ float solve_tau(const float* xs, int m, float alpha, const PowE& pw, int lane) {
    float xmax = -INFINITY;
    for (int c = lane; c < m; c += kWave) xmax = fmaxf(xmax, xs[c]);
    xmax = wave_max(xmax);
    if (m == 1) return xmax - 1.0f;
    float lo = xmax - 1.0f;
    float hi = xmax - exp2f((1.0f - alpha) * __log2f((float)m));
    float tau = lo;
    for (int it = 0; it < 64; ++it) {
        float s = 0.f, ds = 0.f;
        for (int c = lane; c < m; c += kWave) {
            const float t = xs[c] - tau;
            if (t > 0.f) {
                s += pw.val(t);
                ds += pw.der(t);
            }
        }
        s = wave_sum(s);
        ds = wave_sum(ds);
        const float f = s - 1.0f;
        if (f >= 0.f) lo = fmaxf(lo, tau); else hi = fminf(hi, tau);
        float tn = ds > 0.f ? tau + f / (pw.e * ds) : 0.5f * (lo + hi);
        if (!(tn >= lo && tn <= hi)) tn = 0.5f * (lo + hi);
        const bool done = fabsf(tn - tau) <= 1e-7f * fmaxf(1.0f, fabsf(tau));
        tau = tn;
        if (done) break;
    }
    if (pw.kind == kPowGeneral) return tau;
    // closed form on the support S = {x > tau}: sum_S (x - tau)^e = 1 with e in {1, 2}
    for (int rep = 0; rep < 3; ++rep) {
        float s1 = 0.f;
        int k = 0;
        for (int c = lane; c < m; c += kWave)
            if (xs[c] > tau) { s1 += xs[c]; ++k; }
        s1 = wave_sum(s1);
        k = wave_sum_int(k);
        if (k == 0) break;
        float tn;
        if (pw.kind == kPowOne) {
            tn = (s1 - 1.0f) / (float)k;
        } else {
            const float mean = s1 / (float)k;
            float v = 0.f;
            for (int c = lane; c < m; c += kWave)
                if (xs[c] > tau) { const float dx = xs[c] - mean; v += dx * dx; }
            v = wave_sum(v);
            const float delta = (1.0f - v) / (float)k;  // (1 - k * variance) / k
            if (delta < 0.f) break;
            tn = mean - sqrtf(delta);
        }
        int k2 = 0;
        for (int c = lane; c < m; c += kWave) k2 += xs[c] > tn;
        k2 = wave_sum_int(k2);
        if (!(tn >= lo - 1e-6f && tn <= hi + 1e-6f)) break;
        tau = tn;
        if (k2 == k) break;
    }
    return tau;
}

// One wave per (query t, KV group r, sequence b). Dynamic LDS: 2 * tc floats.
__global__ __launch_bounds__(64) void route_kernel(const float* __restrict__ x,
                                                   uint32_t* __restrict__ mask,
                                                   float* __restrict__ bias,
                                                   float* __restrict__ tau_out, RouteParams p) {
    const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    extern __shared__ float lds[];
    float* xs = lds;
    float* ws = lds + p.tc;
    const int pos = p.q_pos0 + t;
    const int cp = pos / p.block;
    const int m = min(cp, p.tc);
    const int64_t qrow = (int64_t)b * p.n_q + t;

    PowE pw;
    pw.e = 1.0f / (p.alpha - 1.0f);
    pw.kind = p.alpha == 2.0f ? kPowOne : (p.alpha == 1.5f ? kPowTwo : kPowGeneral);

    for (int c = lane; c < m; c += kWave) ws[c] = 0.f;
    for (int gg = 0; gg < p.g; ++gg) {
        const int h = r * p.g + gg;
        const float* xr = x + (qrow * p.h_q + h) * p.nc;
        for (int c = lane; c < m; c += kWave) xs[c] = xr[c];
        __syncthreads();
        float tau = INFINITY;
        if (m > 0) {
            tau = solve_tau(xs, m, p.alpha, pw, lane);
            for (int c = lane; c < m; c += kWave) {
                const float d = xs[c] - tau;
                if (d > 0.f) ws[c] += pw.val(d);
            }
        }
        if (tau_out && lane == 0) tau_out[qrow * p.h_q + h] = tau;
        __syncthreads();
    }
    // GQA mean, routed set, mu = mean log w over it
    const float inv_g = 1.0f / (float)p.g;
    float sl = 0.f;
    int cnt = 0;
    for (int c = lane; c < m; c += kWave) {
        const float w = ws[c] * inv_g;
        ws[c] = w;
        if (w > 0.f) { sl += __logf(w); ++cnt; }
    }
    sl = wave_sum(sl);
    cnt = wave_sum_int(cnt);
    const float mu = cnt > 0 ? sl / (float)cnt : 0.f;

    uint32_t* mrow = mask + (qrow * p.h_kv + r) * p.nw;
    float* brow = bias + (qrow * p.h_kv + r) * p.nc;
    for (int base = 0; base < p.nw * 32; base += kWave) {
        const int c = base + lane;
        const bool sel = c < m && ws[c] > 0.f;
        if (sel) brow[c] = (__logf(ws[c]) - mu) * p.inv_sigma;
        const uint64_t bal = __ballot(sel || c == cp);
        if (lane == 0) {
            mrow[base / 32] = (uint32_t)bal;
            if (base / 32 + 1 < p.nw) mrow[base / 32 + 1] = (uint32_t)(bal >> 32);
        }
    }
    if (lane == 0) brow[cp] = 0.f;
}

size_t route_workspace_bytes(const RouteParams& p) {
    return (size_t)p.batch * p.n_q * p.h_q * p.nc * sizeof(float);
}

hipError_t launch_block_entmax(const void* q, int dt, const float* kbar, const RouteParams& p,
                               uint32_t* mask, float* bias, float* tau, void* ws,
                               hipStream_t st) {
    float* x = static_cast<float*>(ws);
    const float coef = (p.alpha - 1.0f) * p.gamma / sqrtf((float)p.head_dim);
    if (p.tc > 0) {
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
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t lds = 2 * (size_t)(p.tc > 0 ? p.tc : 1) * sizeof(float);
    hipLaunchKernelGGL(route_kernel, dim3(p.n_q, p.h_kv, p.batch), dim3(64), lds, st, x, mask,
                       bias, tau, p);
    return hipGetLastError();
}

}  // namespace dash
