// Device helpers shared by the libdash kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

constexpr int kWave = 64;

// Storage types: fp32 as float, bf16 as its raw 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (the hardware conversion of gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, (__bf16)f);
}

__device__ __forceinline__ void store_elem(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_elem(bf16_t* p, float x) { *p = f32_to_bf16(x); }

// Eight consecutive elements as floats (one 16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8(const bf16_t* p, float (&out)[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float (&out)[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Reductions over the 64 lanes of a wave with DPP (data-parallel primitives of the gfx9 ISA):
// swaps within quads, mirrors within half-rows and rows of 16 lanes, then the row broadcasts
// of lane 15 and lane 31 fold the four rows into lane 63, which every lane then reads.
// DPP controls: quad_perm [1,0,3,2] = 0xb1, [2,3,0,1] = 0x4e, row_half_mirror = 0x141,
// row_mirror = 0x140, row_bcast:15 = 0x142 (rows 1, 3), row_bcast:31 = 0x143 (rows 2, 3).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                  __builtin_bit_cast(int, v),
                                                                  CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xb1, 0xf>(0.f, v);
    v += dpp_f<0x4e, 0xf>(0.f, v);
    v += dpp_f<0x141, 0xf>(0.f, v);
    v += dpp_f<0x140, 0xf>(0.f, v);
    v += dpp_f<0x142, 0xa>(0.f, v);
    v += dpp_f<0x143, 0xc>(0.f, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Lanes l and l ^ 32 of a wave: v_permlane32_swap hands each lane its partner's value without a
// trip through LDS; every lane gets the same pair, so the result is the same in both halves.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Rows of 16 lanes in pairs (rows 0 and 1, rows 2 and 3): v_permlane16_swap hands each lane
// the value of the same lane in the other row of its pair; every lane gets its pair's result.
__device__ __forceinline__ float rowpair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float rowpair_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xb1, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<0x4e, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<0x141, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<0x140, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<0x142, 0xa>(-INFINITY, v));
    v = fmaxf(v, dpp_f<0x143, 0xc>(-INFINITY, v));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_min(float v) {
    v = fminf(v, dpp_f<0xb1, 0xf>(INFINITY, v));
    v = fminf(v, dpp_f<0x4e, 0xf>(INFINITY, v));
    v = fminf(v, dpp_f<0x141, 0xf>(INFINITY, v));
    v = fminf(v, dpp_f<0x140, 0xf>(INFINITY, v));
    v = fminf(v, dpp_f<0x142, 0xa>(INFINITY, v));
    v = fminf(v, dpp_f<0x143, 0xc>(INFINITY, v));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ int wave_sum_int(int v) {
    v += dpp_i<0xb1, 0xf>(0, v);
    v += dpp_i<0x4e, 0xf>(0, v);
    v += dpp_i<0x141, 0xf>(0, v);
    v += dpp_i<0x140, 0xf>(0, v);
    v += dpp_i<0x142, 0xa>(0, v);
    v += dpp_i<0x143, 0xc>(0, v);
    return __builtin_amdgcn_readlane(v, 63);
}

__host__ __device__ constexpr int div_up(int a, int b) { return (a + b - 1) / b; }

// Hand-over of data between the workgroups of one launch. Each XCD of the MI355X has its own L2,
// and a device-scope fence writes back and invalidates the whole L2 (a walk of every line), far
// too slow to issue from every workgroup. Data that one workgroup hands to another is therefore
// stored and loaded as device-scope relaxed atomics, which the hardware keeps coherent across the
// XCDs line by line (write-through stores, loads that do not trust a stale L2 copy). The writer
// waits until its stores are acknowledged before it takes a ticket (device-scope atomic add on a
// per-item counter); the workgroup that draws the last ticket then reads everything the others
// stored. Nothing ever waits for another workgroup.
__device__ __forceinline__ void handoff_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float handoff_load(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Called by every thread of the workgroup after its hand-over stores: true in the workgroup that
// took ticket n - 1 of *counter (n tickets are drawn per item), which also resets the counter to
// zero for the next launch. `flag` is one int of LDS.
__device__ __forceinline__ bool handoff_last(unsigned* counter, unsigned n, int* flag) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned t = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = t == n - 1;
        if (t == n - 1) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return *flag != 0;
}

}  // namespace dash
