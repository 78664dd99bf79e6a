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

// Threshold tau with sum_c [x_c - tau]_+^e = 1 for a row of m >= 1 entries.
// f(tau) = sum [x - tau]_+^e - 1 is decreasing and convex on tau < max x, with its root in
// [max x - 1, max x - m^(1 - alpha)]. Newton steps from the left end increase monotonically to
// the root; a step that leaves the bracket (rounding) is replaced by bisection. For e in {1, 2}
// tau is then taken in closed form on its support S = {x > tau}: sum_S (x - tau)^e = 1.
template <int NPL, int KIND>
__device__ float solve_tau_reg(const float (&x)[NPL], int m, float alpha) {
    const float e = 1.0f / (alpha - 1.0f);
    float xmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i) xmax = fmaxf(xmax, x[i]);
    xmax = wave_max(xmax);
    if (m == 1) return xmax - 1.0f;
    float lo = xmax - 1.0f;
    float hi = xmax - exp2f((1.0f - alpha) * __log2f((float)m));
    float tau = lo;
    for (int it = 0; it < 64; ++it) {
        float s = 0.f, ds = 0.f;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const float t = x[i] - tau;
            if (KIND == kPowOne) {
                s += fmaxf(t, 0.f);
                ds += t > 0.f ? 1.f : 0.f;
            } else if (KIND == kPowTwo) {
                const float u = fmaxf(t, 0.f);
                s = fmaf(u, u, s);
                ds += u;
            } else if (t > 0.f) {
                const float lt = __log2f(t);
                s += exp2f(e * lt);
                ds += exp2f((e - 1.0f) * lt);
            }
        }
        s = wave_sum(s);
        ds = wave_sum(ds);
        const float f = s - 1.0f;
        if (f >= 0.f) lo = fmaxf(lo, tau); else hi = fminf(hi, tau);
        float tn = ds > 0.f ? tau + f / (e * ds) : 0.5f * (lo + hi);
        if (!(tn >= lo && tn <= hi)) tn = 0.5f * (lo + hi);
        const bool done = fabsf(tn - tau) <= 1e-7f * fmaxf(1.0f, fabsf(tau));
        tau = tn;
        if (done) break;
    }
    if (KIND == kPowGeneral) return tau;
    for (int rep = 0; rep < 3; ++rep) {
        float s1 = 0.f;
        int k = 0;
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (x[i] > tau) { s1 += x[i]; ++k; }
        s1 = wave_sum(s1);
        k = wave_sum_int(k);
        if (k == 0) break;
        float tn;
        if (KIND == kPowOne) {
            tn = (s1 - 1.0f) / (float)k;
        } else {
            const float mean = s1 / (float)k;
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (x[i] > tau) { const float dx = x[i] - mean; v = fmaf(dx, dx, v); }
            v = wave_sum(v);
            const float delta = (1.0f - v) / (float)k;  // (1 - k * variance) / k
            if (delta < 0.f) break;
            tn = mean - sqrtf(delta);
        }
        int k2 = 0;
#pragma unroll
        for (int i = 0; i < NPL; ++i) k2 += x[i] > tn ? 1 : 0;
        k2 = wave_sum_int(k2);
        if (!(tn >= lo - 1e-6f * fmaxf(1.0f, fabsf(lo)) && tn <= hi + 1e-6f * fmaxf(1.0f, fabsf(hi)))) break;
        tau = tn;
        if (k2 == k) break;
    }
    return tau;
}

// Smallest slot count NPL (a power of two) with 64 * NPL >= n.
__host__ inline int slots_for(int n) {
    int npl = 1;
    while (64 * npl < n) npl *= 2;
    return npl;
}

}  // namespace dash
