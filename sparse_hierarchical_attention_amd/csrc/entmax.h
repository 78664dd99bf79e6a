// alpha-entmax threshold of one row held in a wave's registers ("DashAttention",
// arXiv 2605.18753v1, §2 Eq. 2 and App. A Eq. 13).
//
// Element c of a row sits in lane c % 64, slot c / 64 of an NPL-slot array; slots past the row
// hold -inf and never contribute. KIND selects the exponent e = 1 / (alpha - 1): 1 (alpha = 2,
// sparsemax), 2 (alpha = 1.5) or general (any alpha in (1, 2), through exp2 / log2).
#pragma once

#include <math.h>

#include "common.h"

namespace dash {

enum { kPowGeneral = 0, kPowOne = 1, kPowTwo = 2 };

__host__ __device__ inline int pow_kind(float alpha) {
    return alpha == 2.0f ? kPowOne : (alpha == 1.5f ? kPowTwo : kPowGeneral);
}

// [t]_+^e
template <int KIND>
__device__ __forceinline__ float pow_e(float t, float e) {
    if (KIND == kPowOne) return fmaxf(t, 0.f);
    if (KIND == kPowTwo) {
        const float u = fmaxf(t, 0.f);
        return u * u;
    }
    return t > 0.f ? exp2f(e * __log2f(t)) : 0.f;
}

// ---- lane-group reductions. A "row" here is a DPP row of 16 lanes.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xb1, 0xf>(0.f, v);
    v += dpp_f<0x4e, 0xf>(0.f, v);
    v += dpp_f<0x141, 0xf>(0.f, v);
    v += dpp_f<0x140, 0xf>(0.f, v);
    return v;
}
__device__ __forceinline__ float row16_min(float v) {
    v = fminf(v, dpp_f<0xb1, 0xf>(INFINITY, v));
    v = fminf(v, dpp_f<0x4e, 0xf>(INFINITY, v));
    v = fminf(v, dpp_f<0x141, 0xf>(INFINITY, v));
    v = fminf(v, dpp_f<0x140, 0xf>(INFINITY, v));
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0xb1, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<0x4e, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<0x141, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<0x140, 0xf>(-INFINITY, v));
    return v;
}
// Sums across the four 16-lane rows: partner lanes l ^ 16 and l ^ 32 through the permlane swaps
// of gfx950 (common.h); the same sums, in the same order, as adding the partner's value.
__device__ __forceinline__ float pair16_sum(float v) { return rowpair_sum(v); }
__device__ __forceinline__ float pair32_sum(float v) { return halves_sum(v); }

// Reductions over a lane group: a 16-lane DPP row, or the whole wave (common.h).
template <int LANES> __device__ __forceinline__ float grp_sum(float v) {
    return LANES == 64 ? wave_sum(v) : row16_sum(v);
}
template <int LANES> __device__ __forceinline__ float grp_min(float v) {
    return LANES == 64 ? wave_min(v) : row16_min(v);
}
template <int LANES> __device__ __forceinline__ float grp_max(float v) {
    return LANES == 64 ? wave_max(v) : row16_max(v);
}

// Reductions of the threshold solver over a group of LANES lanes (16: one DPP row; 64: the wave).
template <int LANES>
struct LaneGroupReduce {
    __device__ __forceinline__ float max(float v) { return grp_max<LANES>(v); }
    // true once every lane of the wave is done (the loop exit must be wave-uniform)
    __device__ __forceinline__ bool all(bool done) { return __all(done); }
    __device__ __forceinline__ void gather(float& k, float& p1, float& p2, float& tmin,
                                           float& tout, bool) {
        p1 = grp_sum<LANES>(p1);
        p2 = grp_sum<LANES>(p2);
        k = grp_sum<LANES>(k);
        tmin = grp_min<LANES>(tmin);
        tout = grp_max<LANES>(tout);
    }
};

// Threshold tau of a row held by a lane group, with sum_c [x_c - tau]_+^e = 1 for its m >= 0
// entries. Each lane holds NS slots; slots at or past ns (uniform over the group) are not
// visited and slots past the row hold -inf. A row with m = 0 gets +inf. RED supplies the group's
// reductions (LaneGroupReduce, or a workgroup-wide one).
//
// f(tau) = sum [x - tau]_+^e - 1 is decreasing and convex on tau < max x, with its root in
// [max x - 1, max x - m^(1 - alpha)]. Starting from the left end, each pass gathers over the
// current support S = {x > tau}: its size k, sum of t = x - tau, sum of t^2, the smallest t in S
// and the largest t outside it (t_out <= 0), and solves the root d of f restricted to S:
//   e = 2 (alpha = 1.5): sum_S (t - d)^2 = 1 has the root d = (Q - 1) / (P + sqrt(P^2 - k(Q - 1)))
//   e = 1 (alpha = 2):   sum_S (t - d)   = 1 has the root d = (P - 1) / k
// If t_out <= d < t_min, S is also the support at tau + d, which is then exact.
// e = 1: from the left the restricted root is a lower bound (the terms of S that would turn
// negative pull it down), so tau + d is the next point and tau rises monotonically.
// e = 2: the restricted root over a superset of the support is an upper bound (its dropped terms
// are squares, so positive), over a subset a lower bound; tau + d is taken in turn from either
// side, while the bracket shrinks by those bounds and by the points where S changes (tau + t_min
// from the left, tau + t_out from the right). A step leaving the bracket is replaced by bisection.
// Other exponents: Newton steps from the left, until the step falls below fp32 resolution.
template <int NS, int KIND, class RED>
__device__ __forceinline__ float solve_tau_core(const float (&x)[NS], int ns, int m, float alpha,
                                                RED& red) {
    const float e = 1.0f / (alpha - 1.0f);
    float xm = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < ns) xm = fmaxf(xm, x[s]);
    xm = red.max(xm);
    float lo = xm - 1.0f;
    float hi = m > 1 ? xm - exp2f((1.0f - alpha) * __log2f((float)m)) : lo;
    float tau = m > 0 ? lo : INFINITY;
    bool done = m <= 1;
    for (int it = 0; it < 64; ++it) {
        if (red.all(done)) break;
        const float tr = done ? INFINITY : tau;
        float k = 0.f, p1 = 0.f, p2 = 0.f, tmin = INFINITY, tout = -INFINITY;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s >= ns) break;
            const float t = x[s] - tr;
            const bool in = t > 0.f;
            if (KIND == kPowGeneral) {
                if (in) {
                    const float lt = __log2f(t);
                    p2 += exp2f(e * lt);           // sum t^e
                    p1 += exp2f((e - 1.0f) * lt);  // sum t^(e-1)
                }
            } else {
                // t is never NaN: entries past the row and rows already done give t = -inf
                const float u = fmaxf(t, 0.f);
                k += in ? 1.f : 0.f;
                p1 += u;
                if (KIND == kPowTwo) {
                    p2 = fmaf(u, u, p2);
                    tout = fmaxf(tout, in ? -INFINITY : t);
                }
                tmin = fminf(tmin, in ? t : INFINITY);
            }
        }
        red.gather(k, p1, p2, tmin, tout, done);
        if (done) continue;
        float f, tn;
        if (KIND == kPowTwo) {
            f = p2 - 1.0f;
            const float disc = p1 * p1 - k * f;
            const bool root = k > 0.f && disc >= 0.f;
            const float d = root ? f / (p1 + sqrtf(disc)) : 0.f;
            if (root && d >= tout && d < tmin) {
                tau += d;
                done = true;
                continue;
            }
            if (f >= 0.f) {
                lo = fmaxf(lo, tau);
                if (root) {
                    hi = fminf(hi, tau + d);
                    if (d >= tmin) lo = fmaxf(lo, tau + tmin);
                }
            } else {
                hi = fminf(hi, tau);
                if (root) {
                    lo = fmaxf(lo, tau + d);
                    if (d < tout) hi = fminf(hi, tau + tout);
                }
            }
            tn = root ? tau + d : (p1 > 0.f ? tau + f / (2.0f * p1) : 0.5f * (lo + hi));
        } else if (KIND == kPowOne) {
            f = p1 - 1.0f;
            const float d = k > 0.f ? f / k : 0.f;
            if (f >= 0.f && k > 0.f && d < tmin) {
                tau += d;
                done = true;
                continue;
            }
            tn = k > 0.f ? tau + d : 0.5f * (lo + hi);
            if (f >= 0.f) lo = fmaxf(lo, tau); else hi = fminf(hi, tau);
        } else {
            f = p2 - 1.0f;
            tn = p1 > 0.f ? tau + f / (e * p1) : 0.5f * (lo + hi);
            if (f >= 0.f) lo = fmaxf(lo, tau); else hi = fminf(hi, tau);
        }
        if (!(tn >= lo && tn <= hi)) tn = 0.5f * (lo + hi);
        done = hi - lo <= 1e-7f * fmaxf(1.0f, fabsf(tau)) || fabsf(tn - tau) <= 1e-7f * fmaxf(1.0f, fabsf(tau));
        tau = tn;
    }
    return tau;
}

// A row held by a group of LANES lanes (16 or 64): slot s of a lane holds entry
// s * LANES + (lane % LANES).
template <int NS, int KIND, int LANES>
__device__ float solve_tau_exact(const float (&x)[NS], int ns, int m, float alpha) {
    LaneGroupReduce<LANES> red;
    return solve_tau_core<NS, KIND>(x, ns, m, alpha, red);
}

// One row over the whole wave (64 lanes, slot s holds entry 64 s + lane).
template <int NPL, int KIND>
__device__ __forceinline__ float solve_tau_reg(const float (&x)[NPL], int m, float alpha) {
    return solve_tau_exact<NPL, KIND, 64>(x, (m + 63) / 64, m, alpha);
}

// Smallest slot count NPL (a power of two) with 64 * NPL >= n.
__host__ inline int slots_for(int n) {
    int npl = 1;
    while (64 * npl < n) npl *= 2;
    return npl;
}

}  // namespace dash
