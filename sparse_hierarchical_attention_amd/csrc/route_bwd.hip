// Backward of Stage 1 and Stage 0 for prefill ("DashAttention", arXiv 2605.18753v1: the routing
// of §3.2 Eq. 4 with the GQA mean, the bias d of Prop. 1, and the mean pooling of §3.1 Eq. 3,
// differentiated by the chain rule). The selection (each head's entmax support and the routed set
// R) is held fixed: it is piecewise constant in the inputs. Given dd = dL/dd from the Stage 2
// backward, for one (query row, KV group):
//   mu = mean of log w over R, d_c = (log w_c - mu) / sigma  =>  dlogw_c = (dd_c - mean_R dd) / sigma,
//   w_c = mean over the group's heads of p_h,c             =>  dp_h,c = dlogw_c / (g w_c),
//   p_h = [x_h - tau_h]_+^e, e = 1 / (alpha - 1)            =>  dx_h,c = e u_h,c (dp_h,c - rho_h),
//     u = [x - tau]_+^(e - 1), rho_h = sum_c u_h,c dp_h,c / sum_c u_h,c (the entmax Jacobian,
//     App. A: tau moves so that the probabilities keep summing to one),
//   x_h,c = coef <q_h, kbar_c>, coef = (alpha - 1) gamma / sqrt(D)  =>  dq_h += coef sum_c dx_h,c kbar_c,
//     dkbar_c += coef sum over rows and heads of dx_h,c q_h,
//   kbar_c = the mean of chunk c's keys                     =>  dk_j += dkbar_c / Bc for j in c,
//   or, with a learned summary query qbar_c (Eq. 3's local attention over the chunk's keys),
//   kbar_c = sum_j a_j k_j, a = softmax_j(<qbar_c, k_j> / sqrt(D)), g_j = <dkbar_c, k_j>:
//     dk_j += a_j dkbar_c + a_j (g_j - sum_i a_i g_i) qbar_c / sqrt(D),
//     dqbar_c = sum_j a_j (g_j - sum_i a_i g_i) k_j / sqrt(D)  (the softmax Jacobian).
// Two kernels, each output element written by one thread in a fixed order (deterministic, no
// atomics); both recompute x with the same lane layout and summation order, so they agree bit
// for bit on p, w and the support:
//   route_bwd_row_kernel, one workgroup per (row, group): three passes over R (the mean of dd,
//     then rho per head, then dx) add the routing part of dq and leave mean_R dd and rho per row;
//   route_bwd_col_kernel, one workgroup per (sequence, group, complete chunk): lists in order the
//     rows whose R holds the chunk, recomputes their dx for it, and adds the pooling gradient to
//     the dk of the chunk's keys (and writes the chunk's dqbar);
//   pool_qbar_reduce_kernel sums the per-chunk dqbar over the chunks and sequences that share one
//     summary query, in a fixed order.
#include <math.h>

#include "common.h"
#include "entmax.h"
#include "kernels.h"

namespace dash {

namespace {

constexpr int kRbThreads = 256;  // threads per workgroup (four waves)
constexpr int kRbWaves = kRbThreads / 64;
constexpr int kColThreads = 512;  // threads per workgroup of the column kernel (eight waves)
constexpr int kColWaves = kColThreads / 64;
constexpr int kMaxPoolBlock = 128;  // longest chunk the column kernel pools over
constexpr int kRbCache = 2048;      // floats of the row kernel's pass-2 cache

// bytes of the row kernel's routed list for tc complete chunks (16-byte multiple)
__host__ __device__ constexpr size_t rb_list_bytes(int tc) {
    return ((size_t)(tc > 0 ? tc : 1) * 2 + 15) / 16 * 16;
}

// [t]_+^(e - 1) = p^(2 - alpha) on the support (t = x - tau > 0), 0 off it.
template <int KIND>
__device__ __forceinline__ float u_of(float t, float eu) {
    if (t <= 0.f) return 0.f;
    if (KIND == kPowOne) return 1.f;  // alpha = 2: e - 1 = 0
    if (KIND == kPowTwo) return t;    // alpha = 1.5: e - 1 = 1
    return exp2f(eu * __log2f(t));
}

// Four consecutive elements of a row as floats (8 bytes of bf16 or 16 of fp32).
__device__ __forceinline__ void load4(const bf16_t* s, float (&f)[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(s);
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* s, float (&f)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(s);
    f[0] = u.x;
    f[1] = u.y;
    f[2] = u.z;
    f[3] = u.w;
}

// Sum over aligned groups of LANES (16 or 32) lanes, the same value in each lane of a group.
template <int LANES>
__device__ __forceinline__ float grp4_sum(float v) {
    v += dpp_f<0xb1, 0xf>(0.f, v);
    v += dpp_f<0x4e, 0xf>(0.f, v);
    v += dpp_f<0x141, 0xf>(0.f, v);
    v += dpp_f<0x140, 0xf>(0.f, v);
    if (LANES >= 32) v += __shfl_xor(v, 16, 64);
    return v;
}

// x = coef <q, kbar_c> for one head: q and kbar pieces of 4 elements per lane, LPK lanes per row.
template <int LPK>
__device__ __forceinline__ float score4(const float (&qf)[4], const float (&kf)[4], float coef) {
    float d = qf[0] * kf[0];
    d = fmaf(qf[1], kf[1], d);
    d = fmaf(qf[2], kf[2], d);
    d = fmaf(qf[3], kf[3], d);
    return coef * grp4_sum<LPK>(d);
}

// Ordered list of the chunks c < m whose bit is set in the mask row mrow, into list[]; returns
// their number (the same in every thread). Needs ceil(m / 32) <= blockDim.x; ends with a barrier.
__device__ __forceinline__ int routed_list(const uint32_t* mrow, int m, int* wtot, uint16_t* list) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    uint32_t word = 0;
    if (32 * tid < m) {
        word = mrow[tid];
        const int hi = m - 32 * tid;  // bits 0 .. hi - 1 of this word lie below m
        if (hi < 32) word &= (1u << hi) - 1u;
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
        list[rank++] = (uint16_t)(32 * tid + bit);
    }
    __syncthreads();
    return total;
}

// Sum of a per-wave value over the workgroup's waves, in wave order (the same in every thread).
// Uses red[kRbWaves]; starts and ends with a barrier.
__device__ __forceinline__ float block_sum(float v, float* red) {
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kRbWaves; ++i) s += red[i];
    __syncthreads();
    return s;
}

}  // namespace

template <typename T, int D, int GQ, int KIND>
__global__ __launch_bounds__(kRbThreads) void route_bwd_row_kernel(
    const T* __restrict__ q, const float* __restrict__ kbar, const float* __restrict__ tau,
    const uint32_t* __restrict__ mask, const float* __restrict__ dbias, float* __restrict__ dq,
    float* __restrict__ mean_ws, float* __restrict__ rho_ws, RouteParams p) {
    constexpr int LPK = D / 4;       // lanes per row of D elements
    constexpr int RPW = 64 / LPK;    // chunks per wave step
    // dynamic LDS: the routed list (2 bytes per complete chunk, rounded to 16 bytes), then the
    // per-chunk cache of pass 2 (u of each head and dp, kRbCache floats)
    extern __shared__ __align__(16) unsigned char rb_dyn[];
    uint16_t* list = reinterpret_cast<uint16_t*>(rb_dyn);
    float* cache = reinterpret_cast<float*>(rb_dyn + rb_list_bytes(p.tc));
    __shared__ int wtot[kRbWaves];
    __shared__ float red[kRbWaves];
    __shared__ float hred[kRbWaves][2 * GQ];
    __shared__ float dqred[kRbWaves][GQ * D];
    const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPK, li = lane % LPK;
    const int pos = p.q_pos0 + t;
    const int m = route_cands(p, pos);
    const int64_t row = (int64_t)b * p.n_q + t;
    const float coef = (p.alpha - 1.0f) * p.gamma / sqrtf((float)D);
    const float e = 1.0f / (p.alpha - 1.0f), eu = e - 1.0f;
    const float inv_g = 1.0f / (float)GQ;

    const int nl = routed_list(mask + (row * p.h_kv + r) * p.nw, m, wtot, list);
    // pass 2 leaves u and dp of every routed chunk in LDS when they fit, so that pass 3 does not
    // score the chunks again (the values are the same bits either way)
    const bool cached = nl * (GQ + 1) <= kRbCache;

    float qf[GQ][4], th[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        load4(q + (row * p.h_q + r * GQ + h) * D + 4 * li, qf[h]);
        th[h] = tau[row * p.h_q + r * GQ + h];
    }
    const float* kb = kbar + ((int64_t)b * p.tc * p.h_kv + r) * D + 4 * li;
    const int64_t kstride = (int64_t)p.h_kv * D;
    const float* ddrow = dbias + (row * p.h_kv + r) * p.nc;

    // pass 1: the mean of dd over R
    float sdd = 0.f;
    for (int j0 = wave * RPW; j0 < nl; j0 += kRbWaves * RPW) {
        const int j = j0 + seg;
        if (j < nl && li == 0) sdd += ddrow[list[j]];
    }
    const float mean = nl > 0 ? block_sum(wave_sum(sdd), red) / (float)nl : 0.f;

    // pass 2: rho_h = sum u dp / sum u over R
    float A[GQ], B[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) A[h] = B[h] = 0.f;
    for (int j0 = wave * RPW; j0 < nl; j0 += kRbWaves * RPW) {
        const int j = j0 + seg;
        const bool valid = j < nl;
        const int c = list[valid ? j : 0];
        float kf[4];
        load4(kb + c * kstride, kf);
        float x[GQ], w = 0.f;
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            x[h] = score4<LPK>(qf[h], kf, coef);
            w += pow_e<KIND>(x[h] - th[h], e);
        }
        w *= inv_g;
        const float dlogw = (ddrow[c] - mean) * p.inv_sigma;
        const float dp = w > 0.f ? dlogw / (w * (float)GQ) : 0.f;
        if (valid && li == 0) {
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float u = u_of<KIND>(x[h] - th[h], eu);
                A[h] = fmaf(u, dp, A[h]);
                B[h] += u;
                if (cached) cache[j * (GQ + 1) + h] = u;
            }
            if (cached) cache[j * (GQ + 1) + GQ] = dp;
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        const float a = wave_sum(A[h]), bb = wave_sum(B[h]);
        if (lane == 0) {
            hred[wave][2 * h] = a;
            hred[wave][2 * h + 1] = bb;
        }
    }
    __syncthreads();
    float rho[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        float a = 0.f, bb = 0.f;
#pragma unroll
        for (int i = 0; i < kRbWaves; ++i) {
            a += hred[i][2 * h];
            bb += hred[i][2 * h + 1];
        }
        rho[h] = bb > 0.f ? a / bb : 0.f;
    }

    // pass 3: dx, and dq_h += coef sum_c dx_h,c kbar_c
    float acc[GQ][4];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][i] = 0.f;
    for (int j0 = wave * RPW; j0 < nl; j0 += kRbWaves * RPW) {
        const int j = j0 + seg;
        const bool valid = j < nl;
        const int c = list[valid ? j : 0];
        float kf[4];
        load4(kb + c * kstride, kf);
        float u[GQ], dp;
        if (cached) {
            const int jc = valid ? j : 0;
#pragma unroll
            for (int h = 0; h < GQ; ++h) u[h] = cache[jc * (GQ + 1) + h];
            dp = cache[jc * (GQ + 1) + GQ];
        } else {
            float x[GQ], w = 0.f;
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                x[h] = score4<LPK>(qf[h], kf, coef);
                w += pow_e<KIND>(x[h] - th[h], e);
            }
            w *= inv_g;
            const float dlogw = (ddrow[c] - mean) * p.inv_sigma;
            dp = w > 0.f ? dlogw / (w * (float)GQ) : 0.f;
#pragma unroll
            for (int h = 0; h < GQ; ++h) u[h] = u_of<KIND>(x[h] - th[h], eu);
        }
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float dx = valid ? e * u[h] * (dp - rho[h]) : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[h][i] = fmaf(dx, kf[i], acc[h][i]);
        }
    }
    // fold the wave's chunk segments, then the waves in order
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int o = LPK; o < 64; o <<= 1)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[h][i] += __shfl_xor(acc[h][i], o, 64);
    if (seg == 0) {
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) dqred[wave][h * D + 4 * li + i] = acc[h][i];
    }
    __syncthreads();
    if (nl > 0) {
        for (int idx = tid; idx < GQ * D; idx += kRbThreads) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < kRbWaves; ++i) s += dqred[i][idx];
            const int h = idx / D, d = idx % D;
            dq[(row * p.h_q + r * GQ + h) * D + d] += coef * s;
        }
    }
    if (tid == 0) {
        mean_ws[row * p.h_kv + r] = mean;
#pragma unroll
        for (int h = 0; h < GQ; ++h) rho_ws[row * p.h_q + r * GQ + h] = rho[h];
    }
}

template <typename T, int D, int GQ, int KIND>
__global__ __launch_bounds__(kColThreads) void route_bwd_col_kernel(
    const T* __restrict__ q, const float* __restrict__ kbar, const float* __restrict__ tau,
    const uint32_t* __restrict__ mask, const float* __restrict__ dbias,
    const float* __restrict__ mean_ws, const float* __restrict__ rho_ws, float* __restrict__ dk,
    PoolGrad pg, int64_t fsb, int64_t fsc, RouteParams p) {
    constexpr int LPK = D / 4;
    constexpr int RPW = 64 / LPK;
    constexpr int kScan = kColThreads;  // rows examined per block of the scan
    __shared__ int list[kScan];
    __shared__ int wtot[kColWaves];
    __shared__ float dkred[kColWaves][D];
    // XCD-aware order (index x runs on XCD x % 8): all chunks of one (sequence, group) on one
    // XCD, so that the workgroups gathering the same query rows share its L2
    int c, gr;
    {
        const int bh = p.batch * p.h_kv, x = blockIdx.x;
        if (bh % 8 == 0) {
            gr = (x % 8) + 8 * ((x / 8) / p.tc);
            c = (x / 8) % p.tc;
        } else {
            gr = x / p.tc;
            c = x % p.tc;
        }
    }
    const int b = gr / p.h_kv, r = gr % p.h_kv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPK, li = lane % LPK;
    const float coef = (p.alpha - 1.0f) * p.gamma / sqrtf((float)D);
    const float e = 1.0f / (p.alpha - 1.0f), eu = e - 1.0f;
    const float inv_g = 1.0f / (float)GQ;
    float kf[4];
    load4(kbar + (((int64_t)b * p.tc + c) * p.h_kv + r) * D + 4 * li, kf);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};

    // rows whose routing candidates reach chunk c: c < route_cands(pos), i.e. pos / Bc > c + win
    // the rows from t_first on, in blocks taken from the last one down: the workgroups of one
    // (sequence, group) start together at the end of the sequence and walk down in step
    const int t_first = max(0, (c + p.win + 1) * p.block - p.q_pos0);
    const int nblk = t_first < p.n_q ? div_up(p.n_q - t_first, kScan) : 0;
    for (int bi = nblk - 1; bi >= 0; --bi) {
        const int t0 = t_first + bi * kScan;
        const int t = t0 + tid;
        bool sel = false;
        if (t < p.n_q) {
            const int64_t row = (int64_t)b * p.n_q + t;
            const uint32_t* mrow = mask + (row * p.h_kv + r) * p.nw;
            sel = c < route_cands(p, p.q_pos0 + t) && ((mrow[c >> 5] >> (c & 31)) & 1u);
        }
        const uint64_t bal = __ballot(sel);
        if (lane == 0) wtot[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int i = 0; i < kColWaves; ++i) {
            before += i < wave ? wtot[i] : 0;
            total += wtot[i];
        }
        if (sel) list[before + __popcll(bal & ((1ull << lane) - 1ull))] = t;
        __syncthreads();
        for (int j0 = wave * RPW; j0 < total; j0 += kColWaves * RPW) {
            const int j = j0 + seg;
            const bool valid = j < total;
            const int tt = list[valid ? j : 0];
            const int64_t row = (int64_t)b * p.n_q + tt;
            float qf[GQ][4], x[GQ], w = 0.f;
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                load4(q + (row * p.h_q + r * GQ + h) * D + 4 * li, qf[h]);
                x[h] = score4<LPK>(qf[h], kf, coef) - tau[row * p.h_q + r * GQ + h];
                w += pow_e<KIND>(x[h], e);
            }
            w *= inv_g;
            const float dlogw = (dbias[(row * p.h_kv + r) * p.nc + c] - mean_ws[row * p.h_kv + r]) * p.inv_sigma;
            const float dp = w > 0.f ? dlogw / (w * (float)GQ) : 0.f;
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float rho = rho_ws[row * p.h_q + r * GQ + h];
                const float dx = valid ? e * u_of<KIND>(x[h], eu) * (dp - rho) : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(dx, qf[h][i], acc[i]);
            }
        }
        __syncthreads();  // list[] is refilled by the next block
    }
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], o, 64);
    if (seg == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dkred[wave][4 * li + i] = acc[i];
    }
    __syncthreads();
    if (!pg.qbar) {
        // dk_j += coef dkbar_c / Bc for the chunk's keys (complete chunk: Bc keys)
        const float f = coef / (float)p.block;
        for (int idx = tid; idx < p.block * D; idx += kColThreads) {
            const int j = idx / D, d = idx % D;
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < kColWaves; ++i) s += dkred[i][d];
            dk[(((int64_t)b * p.n_kv + (int64_t)c * p.block + j) * p.h_kv + r) * D + d] += f * s;
        }
        return;
    }

    // learned summary query: back through the chunk's local attention
    __shared__ float dkb[D], qs[D], sl[kMaxPoolBlock], gl[kMaxPoolBlock];
    const float isd = 1.0f / sqrtf((float)D);
    for (int d = tid; d < D; d += kColThreads) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < kColWaves; ++i) s += dkred[i][d];
        dkb[d] = coef * s;
        qs[d] = pg.qbar[b * pg.sb + c * pg.sc + (int64_t)r * D + d];
    }
    __syncthreads();  // dkred is free again from here
    const T* kc = static_cast<const T*>(pg.k) + (((int64_t)b * p.n_kv + (int64_t)c * p.block) * p.h_kv + r) * D + 4 * li;
    float* dkc = dk + (((int64_t)b * p.n_kv + (int64_t)c * p.block) * p.h_kv + r) * D + 4 * li;
    const int64_t kstep = (int64_t)p.h_kv * D;
    float qf4[4], df4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qf4[i] = qs[4 * li + i];
        df4[i] = dkb[4 * li + i];
    }
    // logits s_j = <qbar, k_j> / sqrt(D) and g_j = <dkbar, k_j>; RPW keys per wave and pass (the
    // chunk length is a multiple of kColWaves * RPW, so every lane group holds a key)
    for (int j = wave * RPW + seg; j < p.block; j += kColWaves * RPW) {
        float kf[4], s = 0.f, g = 0.f;
        load4(kc + j * kstep, kf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = fmaf(qf4[i], kf[i], s);
            g = fmaf(df4[i], kf[i], g);
        }
        s = grp4_sum<LPK>(s);
        g = grp4_sum<LPK>(g);
        if (li == 0) {
            sl[j] = s * isd;
            gl[j] = g;
        }
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int j = 0; j < p.block; ++j) mx = fmaxf(mx, sl[j]);
    float z = 0.f, zg = 0.f;
    for (int j = 0; j < p.block; ++j) {
        const float a = __expf(sl[j] - mx);
        z += a;
        zg = fmaf(a, gl[j], zg);
    }
    const float iz = 1.0f / z, gbar = zg * iz;
    float dqa[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = wave * RPW + seg; j < p.block; j += kColWaves * RPW) {
        float kf[4];
        load4(kc + j * kstep, kf);
        const float a = __expf(sl[j] - mx) * iz, ds = a * (gl[j] - gbar);
        float4* dst = reinterpret_cast<float4*>(dkc + j * kstep);
        float4 cur = *dst;
        cur.x += a * df4[0] + ds * qf4[0] * isd;
        cur.y += a * df4[1] + ds * qf4[1] * isd;
        cur.z += a * df4[2] + ds * qf4[2] * isd;
        cur.w += a * df4[3] + ds * qf4[3] * isd;
        *dst = cur;
#pragma unroll
        for (int i = 0; i < 4; ++i) dqa[i] = fmaf(ds, kf[i], dqa[i]);
    }
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) dqa[i] += __shfl_xor(dqa[i], o, 64);
    if (seg == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dkred[wave][4 * li + i] = dqa[i];
    }
    __syncthreads();
    for (int d = tid; d < D; d += kColThreads) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < kColWaves; ++i) s += dkred[i][d];
        pg.dqbar[b * fsb + c * fsc + (int64_t)r * D + d] = s * isd;
    }
}

// dL/dqbar of a summary query shared by several (sequence, chunk) pairs: the sum of their
// per-chunk gradients part [B, Tc, Hkv, D], sequence-major then chunk, in a fixed order. One
// workgroup per output row (b', c', r): b' runs over the sequences when sb != 0 (else 0), c' over
// the chunks when sc != 0 (else 0); each of the SL slices of lanes sums every SL-th term.
template <int D>
__global__ __launch_bounds__(256) void pool_qbar_reduce_kernel(
    const float* __restrict__ part, float* __restrict__ dqbar, int batch, int tc, int h_kv,
    int64_t sb, int64_t sc) {
    constexpr int LPR = D / 4;
    constexpr int SL = 256 / LPR;
    __shared__ float4 red[SL][LPR];
    const int ncc = sc ? tc : 1;
    const int r = blockIdx.x % h_kv, cc = (blockIdx.x / h_kv) % ncc, bb = blockIdx.x / (h_kv * ncc);
    const int nb_sum = sb ? 1 : batch, nc_sum = sc ? 1 : tc;
    const int li = threadIdx.x % LPR, sl = threadIdx.x / LPR;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int u = sl; u < nb_sum * nc_sum; u += SL) {
        const int b = sb ? bb : u / nc_sum, c = sc ? cc : u % nc_sum;
        const float4 x = *reinterpret_cast<const float4*>(part + (((int64_t)b * tc + c) * h_kv + r) * D + 4 * li);
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
    }
    red[sl][li] = acc;
    __syncthreads();
    if (sl == 0) {
        for (int i = 1; i < SL; ++i) {
            acc.x += red[i][li].x;
            acc.y += red[i][li].y;
            acc.z += red[i][li].z;
            acc.w += red[i][li].w;
        }
        *reinterpret_cast<float4*>(dqbar + bb * sb + cc * sc + (int64_t)r * D + 4 * li) = acc;
    }
}

// mean_R dd per (row, group) and rho per (row, head); then, for learned summary queries, each
// chunk's dqbar [B, Tc, Hkv, D] from a 256-byte boundary
size_t route_backward_rows_bytes(const RouteParams& p) {
    return ((size_t)p.batch * p.n_q * (p.h_q + p.h_kv) * sizeof(float) + 255) & ~(size_t)255;
}
size_t route_backward_workspace_bytes(const RouteParams& p, bool with_query) {
    if (!with_query) return (size_t)p.batch * p.n_q * (p.h_q + p.h_kv) * sizeof(float);
    return route_backward_rows_bytes(p) + (size_t)p.batch * p.tc * p.h_kv * p.head_dim * sizeof(float);
}

template <typename T, int D, int GQ, int KIND>
static void launch_rb_k(const void* q, const float* kbar, const float* tau, const uint32_t* mask,
                        const float* dbias, float* dq, float* dk, float* mean_ws, float* rho_ws,
                        const PoolGrad& pg, int64_t fsb, int64_t fsc, const RouteParams& p,
                        hipStream_t st) {
    hipLaunchKernelGGL((route_bwd_row_kernel<T, D, GQ, KIND>), dim3(p.n_q, p.h_kv, p.batch),
                       dim3(kRbThreads), rb_list_bytes(p.tc) + kRbCache * sizeof(float), st, static_cast<const T*>(q), kbar, tau, mask, dbias,
                       dq, mean_ws, rho_ws, p);
    if (p.tc > 0)
        hipLaunchKernelGGL((route_bwd_col_kernel<T, D, GQ, KIND>), dim3(p.tc * p.h_kv * p.batch),
                           dim3(kColThreads), 0, st, static_cast<const T*>(q), kbar, tau, mask,
                           dbias, mean_ws, rho_ws, dk, pg, fsb, fsc, p);
}

template <typename T, int D, int GQ>
static void launch_rb_g(const void* q, const float* kbar, const float* tau, const uint32_t* mask,
                        const float* dbias, float* dq, float* dk, float* mean_ws, float* rho_ws,
                        const PoolGrad& pg, int64_t fsb, int64_t fsc, const RouteParams& p,
                        hipStream_t st) {
    switch (pow_kind(p.alpha)) {
        case kPowOne: launch_rb_k<T, D, GQ, kPowOne>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, pg, fsb, fsc, p, st); break;
        case kPowTwo: launch_rb_k<T, D, GQ, kPowTwo>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, pg, fsb, fsc, p, st); break;
        default: launch_rb_k<T, D, GQ, kPowGeneral>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, pg, fsb, fsc, p, st); break;
    }
}

template <typename T, int D>
static void launch_rb_d(const void* q, const float* kbar, const float* tau, const uint32_t* mask,
                        const float* dbias, float* dq, float* dk, float* mean_ws, float* rho_ws,
                        const PoolGrad& pg, int64_t fsb, int64_t fsc, const RouteParams& p,
                        hipStream_t st) {
    switch (p.g) {
        case 1: launch_rb_g<T, D, 1>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, pg, fsb, fsc, p, st); break;
        case 2: launch_rb_g<T, D, 2>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, pg, fsb, fsc, p, st); break;
        case 4: launch_rb_g<T, D, 4>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, pg, fsb, fsc, p, st); break;
        case 8: launch_rb_g<T, D, 8>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, pg, fsb, fsc, p, st); break;
        default: launch_rb_g<T, D, 16>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, pg, fsb, fsc, p, st); break;
    }
}

hipError_t launch_route_backward(const void* q, int dt, const float* kbar, const float* tau,
                                 const uint32_t* mask, const float* dbias, float* dq, float* dk,
                                 const PoolGrad& pg, const RouteParams& p, void* ws,
                                 hipStream_t st) {
    float* mean_ws = static_cast<float*>(ws);
    float* rho_ws = mean_ws + (size_t)p.batch * p.n_q * p.h_kv;
    // each chunk's dqbar goes straight to dqbar when no two chunks share a query, else through
    // the workspace and a fixed-order sum
    const bool shared = pg.qbar && ((p.batch > 1 && pg.sb == 0) || (p.tc > 1 && pg.sc == 0));
    PoolGrad g = pg;
    int64_t fsb = pg.sb, fsc = pg.sc;
    if (shared) {
        g.dqbar = reinterpret_cast<float*>(static_cast<char*>(ws) + route_backward_rows_bytes(p));
        fsb = (int64_t)p.tc * p.h_kv * p.head_dim;
        fsc = (int64_t)p.h_kv * p.head_dim;
    }
    if (dt == kBF16) {
        if (p.head_dim == 64) launch_rb_d<bf16_t, 64>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, g, fsb, fsc, p, st);
        else launch_rb_d<bf16_t, 128>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, g, fsb, fsc, p, st);
    } else {
        if (p.head_dim == 64) launch_rb_d<float, 64>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, g, fsb, fsc, p, st);
        else launch_rb_d<float, 128>(q, kbar, tau, mask, dbias, dq, dk, mean_ws, rho_ws, g, fsb, fsc, p, st);
    }
    if (shared) {
        const int nb = pg.sb ? p.batch : 1, ncc = pg.sc ? p.tc : 1;
        if (nb * ncc > 0) {
            if (p.head_dim == 64)
                hipLaunchKernelGGL(pool_qbar_reduce_kernel<64>, dim3(nb * ncc * p.h_kv), dim3(256), 0, st,
                                   g.dqbar, pg.dqbar, p.batch, p.tc, p.h_kv, pg.sb, pg.sc);
            else
                hipLaunchKernelGGL(pool_qbar_reduce_kernel<128>, dim3(nb * ncc * p.h_kv), dim3(256), 0, st,
                                   g.dqbar, pg.dqbar, p.batch, p.tc, p.h_kv, pg.sb, pg.sc);
        }
    }
    return hipGetLastError();
}

}  // namespace dash
