// Stage 2 for one new token per sequence: split-KV sparse attention ("DashAttention",
// arXiv 2605.18753v1, §3.5 "split-KV variant"; the output is that of §3.4 Prop. 1).
//
// The keys a (sequence, group) attends to -- those of its routed chunks and of its own chunk,
// in increasing order -- are cut into units of kDecUnit keys, and unit u goes to slot
// u % kDecodeSlots. decode_split_kernel: each wave owns one slot (and, for groups of more than
// four heads, one set of four heads) and walks its units with the keys and values in registers:
// a 16-byte load per lane holds a piece of one key row, a row of D elements spans D / 8 (bf16) or
// D / 4 (fp32) lanes, and one load instruction covers 64 / (that many) whole rows. Dot products
// run on packed bf16 pairs (v_dot2) and finish with DPP sums inside each row's lanes; the online
// softmax keeps one running maximum per head and per-lane partial sums. The waves of a
// workgroup merge their slots in LDS and write one partial (unnormalised output, max, sum) per
// head to the workspace. decode_combine_kernel merges the workgroups' partials in order.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dash {

constexpr int kDecodeSlots = 32;   // unit slots per (sequence, group)
constexpr int kDecUnit = 32;       // keys per unit
constexpr int kDecMaxWords = 256;  // 8192 chunks
constexpr float kDecLog2e = 1.4426950408889634f;

// Sum over aligned groups of LANES consecutive lanes (8, 16 or 32); every lane gets its group's sum.
template <int LANES>
__device__ __forceinline__ float seg_sum(float v) {
    v += dpp_f<0xb1, 0xf>(0.f, v);       // pairs
    v += dpp_f<0x4e, 0xf>(0.f, v);       // quads
    v += dpp_f<0x141, 0xf>(0.f, v);      // half rows (8 lanes)
    if (LANES >= 16) v += dpp_f<0x140, 0xf>(0.f, v);  // rows (16 lanes)
    if (LANES >= 32) v += __shfl_xor(v, 16, 64);
    return v;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// <q, k> over one 16-byte piece: q as 8 bf16 (4 packed pairs) or 4 floats.
__device__ __forceinline__ float piece_dot(const uint4& qp, const uint4& kp, bf16_t) {
    float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp.x),
                                              __builtin_bit_cast(bf16x2_t, kp.x), 0.f, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp.y),
                                        __builtin_bit_cast(bf16x2_t, kp.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp.z),
                                        __builtin_bit_cast(bf16x2_t, kp.z), d, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp.w),
                                           __builtin_bit_cast(bf16x2_t, kp.w), d, false);
}
__device__ __forceinline__ float piece_dot(const uint4& qp, const uint4& kp, float) {
    float d = __uint_as_float(qp.x) * __uint_as_float(kp.x);
    d = fmaf(__uint_as_float(qp.y), __uint_as_float(kp.y), d);
    d = fmaf(__uint_as_float(qp.z), __uint_as_float(kp.z), d);
    return fmaf(__uint_as_float(qp.w), __uint_as_float(kp.w), d);
}

// Elements of a 16-byte piece as floats.
__device__ __forceinline__ void unpack(const uint4& u, float (&f)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack(const uint4& u, float (&f)[4]) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
}

__host__ __device__ constexpr int dec_heads_per_wave(int g) { return g > 4 ? 4 : g; }
__host__ __device__ constexpr int dec_waves_per_slot(int g) { return g > 4 ? g / 4 : 1; }
// workgroups (of four waves) per (sequence, group)
__host__ __device__ constexpr int dec_workgroups(int g) {
    return kDecodeSlots * dec_waves_per_slot(g) / 4;
}

// workspace: [B, H_kv, dec_workgroups(g), g, D + 4] floats: D unnormalised outputs, max (log2),
// sum, two floats of padding (16-byte aligned records)
template <typename T, int D, int GQ>
__global__ __launch_bounds__(256) void decode_split_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           const T* __restrict__ v,
                                                           const uint32_t* __restrict__ mask,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ ws, AttnParams p) {
    constexpr int EPL = 16 / sizeof(T);          // elements per 16-byte piece
    constexpr int LPK = D / EPL;                 // lanes per key row
    constexpr int KPI = 64 / LPK;                // key rows per load instruction
    constexpr int NI = kDecUnit / KPI;           // loads per tensor and unit
    constexpr int WPS = dec_waves_per_slot(GQ);  // waves per slot (sets of four heads)
    constexpr int HPW = dec_heads_per_wave(GQ);  // heads per wave
    constexpr int SPW = 4 / WPS;                 // slots per workgroup
    constexpr int DS = D + 4;                    // workspace record
    static_assert(kDecUnit % KPI == 0 && LPK >= 8 && LPK <= 32, "unsupported head size");
    __shared__ __align__(16) T qs[GQ * D];
    __shared__ __align__(16) float part[4][HPW][DS];
    __shared__ int wtot[4];
    __shared__ uint16_t chunks[kDecMaxWords * 32];  // rank -> chunk

    const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = p.n_kv;  // cache capacity (the row stride of K and V)
    const int pos = seq_pos(p.ctx_lens, n - 1, n, b, 0);
    const int cp = pos / p.block;
    const uint32_t* mrow = mask + ((int64_t)b * p.h_kv + r) * p.nw;
    const float* brow = bias + ((int64_t)b * p.h_kv + r) * p.nc;

    // mask words of chunks 0..cp (own chunk included), one per thread, and their ranks
    const int nwr = cp / 32 + 1;
    uint32_t word = 0;
    if (tid < nwr) {
        word = mrow[tid];
        const int hi = cp - 32 * tid;
        if (hi < 31) word &= (2u << hi) - 1u;
        if (hi < 32) word |= 1u << hi;
    }
    for (int e = tid; e < GQ * D / EPL; e += 256)
        reinterpret_cast<uint4*>(qs)[e] =
            reinterpret_cast<const uint4*>(q + ((int64_t)b * p.h_q + r * GQ) * D)[e];
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        rank += i < wave ? wtot[i] : 0;
        total += wtot[i];
    }
    while (word) {
        const int bit = __builtin_ctz(word);
        word &= word - 1u;
        chunks[rank++] = (uint16_t)(32 * tid + bit);
    }
    __syncthreads();

    const int cs = wave / WPS;              // slot within the workgroup
    const int h0 = (wave % WPS) * HPW;      // first head of this wave within the group
    const int js = s * SPW + cs;            // slot within the (sequence, group)
    const int seg = lane / LPK, li = lane % LPK;
    const int upc = (p.block + kDecUnit - 1) / kDecUnit;  // units per chunk
    const int64_t kv_stride = (int64_t)p.h_kv * D;
    const T* kb = k + (int64_t)b * n * kv_stride + (int64_t)r * D + li * EPL;
    const T* vb = v + (int64_t)b * n * kv_stride + (int64_t)r * D + li * EPL;
    const float qk_scale = p.scale * kDecLog2e;

    uint4 qp[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
        qp[hh] = *reinterpret_cast<const uint4*>(&qs[(h0 + hh) * D + li * EPL]);
    float acc[HPW][EPL], m_run[HPW], l_run[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        m_run[hh] = -INFINITY;
        l_run[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
    }
    for (int u = js; u < total * upc; u += kDecodeSlots) {
        const int c = chunks[u / upc];
        const int k0 = c * p.block + (u % upc) * kDecUnit;
        const bool diag = c == cp;
        const int kend = diag ? pos + 1 : min((c + 1) * p.block, k0 + kDecUnit);
        if (k0 >= kend) continue;  // a unit of the own chunk past the query
        const float off = diag ? 0.f : brow[c] * kDecLog2e;
        uint4 kr[NI], vr[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = min(k0 + i * KPI + seg, kend - 1);  // rows past the end: clamped
            kr[i] = *reinterpret_cast<const uint4*>(kb + key * kv_stride);
            vr[i] = *reinterpret_cast<const uint4*>(vb + key * kv_stride);
        }
        float sc[HPW][NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bool valid = k0 + i * KPI + seg < kend;
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const float d = seg_sum<LPK>(piece_dot(qp[hh], kr[i], T()));
                sc[hh][i] = valid ? fmaf(d, qk_scale, off) : -INFINITY;
            }
        }
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            float mx = sc[hh][0];
#pragma unroll
            for (int i = 1; i < NI; ++i) mx = fmaxf(mx, sc[hh][i]);
#pragma unroll
            for (int o = LPK; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float m_new = fmaxf(m_run[hh], mx);
            const float corr = __builtin_amdgcn_exp2f(m_run[hh] - m_new);
            m_run[hh] = m_new;
            float l = l_run[hh] * corr;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                sc[hh][i] = __builtin_amdgcn_exp2f(sc[hh][i] - m_new);
                l += sc[hh][i];
            }
            l_run[hh] = l;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[hh][e] *= corr;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float vf[EPL];
            unpack(vr[i], vf);
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(sc[hh][i], vf[e], acc[hh][e]);
        }
    }
    // fold the key rows of the wave (lanes l, l + LPK, ... hold the same dimensions)
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
        for (int o = LPK; o < 64; o <<= 1) {
            l_run[hh] += __shfl_xor(l_run[hh], o, 64);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], o, 64);
        }
    }
    if (seg == 0) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
            for (int e = 0; e < EPL; e += 4)
                *reinterpret_cast<float4*>(&part[wave][hh][li * EPL + e]) =
                    make_float4(acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]);
            if (li == 0) {
                part[wave][hh][D] = m_run[hh];
                part[wave][hh][D + 1] = l_run[hh];
            }
        }
    }
    __syncthreads();
    // merge the workgroup's slots (waves cs * WPS + set, in slot order) per head; an empty slot
    // has max = -inf and sum = 0
    for (int e = tid; e < GQ * D; e += 256) {
        const int hg = e / D, d = e % D;
        const int set = hg / HPW, hh = hg % HPW;
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < SPW; ++c) mx = fmaxf(mx, part[c * WPS + set][hh][D]);
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int c = 0; c < SPW; ++c) {
            const float* pr = part[c * WPS + set][hh];
            const float f = pr[D] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pr[D] - mx);
            o = f > 0.f ? fmaf(f, pr[d], o) : o;
            l = fmaf(f, pr[D + 1], l);
        }
        float* out = ws + ((((int64_t)b * p.h_kv + r) * gridDim.x + s) * GQ + hg) * DS;
        out[d] = o;
        if (d == 0) {
            out[D] = mx;
            out[D + 1] = l;
        }
    }
}

template <typename T, int D, int NP>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws,
                                                            T* __restrict__ o, AttnParams p) {
    constexpr int DPL = D / 64;
    const int h = blockIdx.x, b = blockIdx.y;
    const int r = h / p.g, hh = h % p.g;
    const int lane = threadIdx.x;
    const float* base = ws + (((int64_t)b * p.h_kv + r) * NP * p.g + hh) * (D + 4);
    const int64_t part_stride = (int64_t)p.g * (D + 4);
    // all partial maxima, sums and outputs first (independent loads), then the weights
    float ms[NP], ls[NP], os[NP][DPL];
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        ms[s] = base[s * part_stride + D];
        ls[s] = base[s * part_stride + D + 1];
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) os[s][dd] = base[s * part_stride + lane + 64 * dd];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < NP; ++s) mx = fmaxf(mx, ms[s]);
    float l = 0.f, acc[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) acc[dd] = 0.f;
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        const float f = ms[s] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[s] - mx);
        l = fmaf(f, ls[s], l);
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) acc[dd] = f > 0.f ? fmaf(f, os[s][dd], acc[dd]) : acc[dd];
    }
    const float inv = 1.0f / l;
    T* orow = o + ((int64_t)b * p.h_q + h) * D;
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) store_elem(orow + lane + 64 * dd, acc[dd] * inv);
}

size_t decode_workspace_bytes(const AttnParams& p) {
    return (size_t)p.batch * p.h_kv * dec_workgroups(p.g) * p.g * (p.head_dim + 4) * sizeof(float);
}

template <typename T, int D>
static void launch_decode_t(const void* q, const void* k, const void* v, const uint32_t* mask,
                            const float* bias, void* o, const AttnParams& p, float* ws,
                            hipStream_t st) {
#define DASH_DEC(GG)                                                                           \
    hipLaunchKernelGGL((decode_split_kernel<T, D, GG>), dim3(dec_workgroups(GG), p.h_kv, p.batch), \
                       dim3(256), 0, st, static_cast<const T*>(q), static_cast<const T*>(k),     \
                       static_cast<const T*>(v), mask, bias, ws, p);                             \
    hipLaunchKernelGGL((decode_combine_kernel<T, D, dec_workgroups(GG)>), dim3(p.h_q, p.batch),  \
                       dim3(64), 0, st, ws, static_cast<T*>(o), p)
    switch (p.g) {
        case 1: DASH_DEC(1); break;
        case 2: DASH_DEC(2); break;
        case 4: DASH_DEC(4); break;
        case 8: DASH_DEC(8); break;
        default: DASH_DEC(16); break;
    }
#undef DASH_DEC
}

hipError_t launch_attn_decode(const void* q, const void* k, const void* v, int dt,
                              const uint32_t* mask, const float* bias, void* o,
                              const AttnParams& p, void* ws, hipStream_t st) {
    float* w = static_cast<float*>(ws);
    if (dt == kBF16) {
        if (p.head_dim == 64) launch_decode_t<bf16_t, 64>(q, k, v, mask, bias, o, p, w, st);
        else launch_decode_t<bf16_t, 128>(q, k, v, mask, bias, o, p, w, st);
    } else {
        if (p.head_dim == 64) launch_decode_t<float, 64>(q, k, v, mask, bias, o, p, w, st);
        else launch_decode_t<float, 128>(q, k, v, mask, bias, o, p, w, st);
    }
    return hipGetLastError();
}

}  // namespace dash
