// Stage 2 prefill for head dim 128 on bf16 MFMA, with K and V tiles moved by direct global->LDS
// loads ("DashAttention", arXiv 2605.18753v1, §3.3-3.4 Prop. 1; App. G Alg. 3), gfx950.
//
// A workgroup (4 waves) owns 128 query rows of one (sequence b, KV group r): T = 128 / g
// consecutive tokens times the g heads of the group, row = token * g + head. All rows share the
// group's chunk selection per token, so the workgroup walks the union of its tokens' selected
// chunks (their own diagonal chunks included) and masks, per row, the chunks its token did not
// select. Chunks of 64 or 128 keys are cut into tiles of 64 keys (69 KiB of LDS, 183 VGPRs: two
// workgroups per CU, one tile barrier per 64 keys); chunks of 32 keys are one tile each (35 KiB,
// 156 VGPRs: three workgroups per CU).
//
// Tiles reach LDS through buffer_load_dwordx4 ... lds: each wave instruction writes 1 KiB (lane i
// at byte 16 i) straight into LDS, so the next tile streams in while the current one is multiplied,
// with no registers held and nothing for the compiler to reorder. A tile's rows are stored in
// NB = KT / 4 blocks of four 256-byte rows (row r in block r % NB at slot r / NB, one load
// instruction per block). The LDS has 64 banks and serves a 128-bit read 16 lanes per cycle and a
// 64-bit read 32 lanes per cycle. K blocks are 1040 bytes apart, so the 16 rows a 16-lane group
// reads cover the 64 banks when they lie in 16 blocks (64-key tiles); in 32-key tiles (8 blocks,
// two slots) the K rows of odd slots hold their 16-byte pieces in the order piece ^ 8 for the
// same effect. V blocks are 1088 bytes apart, so the transposing V reads of a 32-lane group
// (4 rows, 8 dims each) cover the banks too. Every read is a lane base plus a constant. Two
// buffers each for K and V are separate LDS objects and the tile loop is unrolled by two, so
// the compiler sees that the reads of one buffer never wait for the loads into the other.
//
// Per wave (32 rows) and tile, with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   A = K rows (ds_read_b128), B = the wave's Q rows held in registers for the
//                 whole kernel; lane l of the accumulator holds query row l % 32 and 16 keys.
//   O^T += V^T P^T  B = P straight from the S accumulator (converted to bf16), A = V^T read with
//                 ds_read_b64_tr_b16: inside each 16-lane group the four 64-bit loads of lanes
//                 4v .. 4v + 3 form key v, and lane i receives dimension i of keys 0..3, which
//                 is the run of four keys the lane's P slots refer to.
// Softmax in the log2 domain: x = s * scale * log2(e) + d * log2(e). The running maximum m is
// only raised when a tile's maximum exceeds it by more than 8 (so exp2(x - m) <= 256 and the
// output, normalised by the sum taken against the same m, is unchanged); p = exp2(x - m) is a
// single FMA and exp2 per score. A row whose token did not select the chunk has x = -inf; the
// query's own chunk is causally masked on the raw scores, so every tile takes the same code.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dash {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = 128;              // head dim of this kernel
constexpr int kRows = 128;           // query rows per workgroup
constexpr int kThreads = 256;
constexpr int kTile = 64;            // keys per LDS tile (at most)
constexpr int kWords = 256;          // mask words of the union (8192 chunks)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;     // log2 headroom before the running maximum is raised

constexpr int kKBlock = 520;         // elements between K blocks (1040 bytes)
constexpr int kVBlock = 544;         // elements between V blocks (1088 bytes)

__device__ __forceinline__ i16x4 ds_read_tr16(const bf16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_void*)(p));
}

}  // namespace

template <int BLK, int GQ>
__global__ __launch_bounds__(kThreads, BLK < 64 ? 3 : 2) void attn_dma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const uint32_t* __restrict__ mask, const float* __restrict__ bias, bf16_t* __restrict__ o,
    float* __restrict__ lse, AttnParams p, int n_tiles) {
    // the body is device code only: the buffer descriptors it builds have no host type, and the
    // host pass needs just the launch stub
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int T = kRows / GQ;            // tokens per workgroup
    constexpr int KT = BLK < kTile ? BLK : kTile;  // keys per tile
    constexpr int NSUB = BLK / KT;
    constexpr int MT = KT / 32;              // 32-key M-tiles of S^T
    constexpr int KSTEP = KT / 16;           // 16-key k-steps of P V
    constexpr int DT = kD / 32;              // 32-dim M-tiles of O^T
    constexpr int NB = KT / 4;               // blocks of four rows per tile
    constexpr int NLD = NB / 4;              // load instructions (blocks) per wave and tensor
    __shared__ __align__(16) bf16_t K0[NB * kKBlock];
    __shared__ __align__(16) bf16_t K1[NB * kKBlock];
    __shared__ __align__(16) bf16_t V0[NB * kVBlock];
    __shared__ __align__(16) bf16_t V1[NB * kVBlock];
    __shared__ uint32_t uni[kWords];

    int gr;
    {
        const int bh = p.batch * p.h_kv, x = blockIdx.x;
        gr = bh % 8 == 0 ? (x % 8) + 8 * ((x / 8) % (bh / 8)) : x % bh;
    }
    const int tile = n_tiles - 1 - blockIdx.x / (p.batch * p.h_kv);
    const int b = gr / p.h_kv, r = gr % p.h_kv;
    const int n = p.n_kv;
    const int tile0 = tile * T;                        // first row of the tile among the n_q rows
    const int tile_end = min(tile0 + T, p.n_q);
    const int c_first = (p.q_pos0 + tile0) / BLK, c_last = (p.q_pos0 + tile_end - 1) / BLK;
    const int nwt = c_last / 32 + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, G = lane >> 5;
    const int row = wave * 32 + j;
    const int tok = row / GQ, hl = row % GQ;
    const int rowi = tile0 + tok;                       // the row among the n_q rows
    const int pos = p.q_pos0 + rowi;                    // its token position
    const bool valid = rowi < p.n_q;
    const int cpos = pos / BLK;
    const int64_t qrow = (int64_t)b * p.n_q + rowi;
    const int64_t qrow_c = (int64_t)b * p.n_q + min(rowi, p.n_q - 1);  // rows past the end read the last
    const uint32_t* mrow = mask + (qrow_c * p.h_kv + r) * p.nw;
    const float* brow = bias + (qrow_c * p.h_kv + r) * p.nc;

    // union of the tile tokens' selections (bits past a token's own chunk ignored)
    for (int w = tid; w < nwt; w += kThreads) uni[w] = 0u;
    __syncthreads();
    for (int idx = tid; idx < T * nwt; idx += kThreads) {
        const int t = idx / nwt, w = idx % nwt;
        const int ps = tile0 + t;
        if (ps >= p.n_q) continue;
        const int hi = (p.q_pos0 + ps) / BLK - 32 * w;
        if (hi < 0) continue;
        uint32_t word = mask[(((int64_t)b * p.n_q + ps) * p.h_kv + r) * p.nw + w];
        if (hi < 31) word &= (2u << hi) - 1u;
        if (hi < 32) word |= 1u << hi;
        if (word) atomicOr(&uni[w], word);
    }
    __syncthreads();
    // the union's next chunk after c (-1 when none): the same walk in every thread
    auto next_chunk = [&](int c) -> int {
        int w = (c + 1) >> 5;
        if (w >= nwt) return -1;
        uint32_t word = uni[w] & (~0u << ((c + 1) & 31));
        while (true) {
            if (word) return 32 * w + __builtin_ctz(word);
            if (++w >= nwt) return -1;
            word = uni[w];
        }
    };

    // this wave's Q rows as the B operand of S^T = K Q^T (k-slot order shared with K's reads)
    bf16x8 qf[kD / 16];
    {
        const bf16_t* qp = q + (qrow_c * p.h_q + r * GQ + hl) * kD + 8 * G;
#pragma unroll
        for (int s = 0; s < kD / 16; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 16 * s));
    }
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
    float m_used = -INFINITY, l_run = 0.f;
    const float qk_scale = p.scale * kLog2e;
    const int64_t kv_row_stride = (int64_t)p.h_kv * kD;
    const bf16_t* kbase = k + (int64_t)b * n * kv_row_stride + (int64_t)r * kD;
    const bf16_t* vbase = v + (int64_t)b * n * kv_row_stride + (int64_t)r * kD;

    // LDS element offsets of this lane's reads: K piece 2 ks + G of row j (+ 32 mt rows), and the
    // transposing V reads of rows v_key (+ 8) at dims 32 dt + v_dim (+ 16 ks rows)
    // K rows in odd slots of a block hold their 16-byte pieces in the order piece ^ 8, so that the
    // 16 rows one 16-lane group reads (two slots of eight blocks) cover all 64 banks: reads of
    // pieces 0-7 (k-steps 0-3) start at kl_lo, pieces 8-15 at kl_hi, each plus a constant offset
    static_assert((NB == 8 && MT == 1) || (NB == 16 && MT == 2), "tiles of 32 or 64 keys");
    const int kl_base = (j % NB) * kKBlock + (j / NB) * kD + 8 * G;   // + 16 ks
    const int k_odd = NB == 8 ? (j / NB) & 1 : 0;
    const int kl_lo = kl_base + 64 * k_odd, kl_hi = kl_base - 64 * k_odd;
    int vl_base[2];                                                    // + ks (16 / NB) kD + 32 dt
    {
        const int grp = lane >> 4, kl = lane & 15;
        const int v_key = 4 * (grp >> 1) + (kl >> 2);
        const int v_dim = 16 * (grp & 1) + 4 * (kl & 3);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rr = v_key + 8 * h;
            vl_base[h] = (rr % NB) * kVBlock + (rr / NB) * kD + v_dim;
        }
    }

    // one tile (chunk c, 32-key part sub) into K / V buffers: wave w fills blocks
    // NLD w .. NLD (w + 1) - 1, one instruction each; lane i fetches piece i % 16 of the block's
    // row i / 16, i.e. tile row b + NB (i / 16). The loads go through buffer descriptors over this
    // (sequence, KV head)'s rows. The whole byte offset (the tile's start plus the lane's fixed
    // offset within a tile) goes in the per-lane offset, the one the descriptor's range check
    // covers (the scalar offset is outside it), so rows past the sequence read as zero and never
    // touch the next sequence or memory past the tensor (every query masks them causally).
    const uint32_t row_bytes = (uint32_t)kv_row_stride * 2u;
    const uint32_t span = (uint32_t)((n - 1) * kv_row_stride + kD) * 2u;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, (int)span, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, (int)span, 0x00020000);
    uint32_t loff[NLD], loff_k[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int rr = NLD * wave + i + NB * (lane >> 4);
        loff[i] = rr * row_bytes + (uint32_t)((lane & 15) * 16);
        // K: the slot's pieces swizzled (lane >> 4 is the row's slot in its block)
        loff_k[i] = rr * row_bytes + (uint32_t)(((lane & 15) ^ (NB == 8 ? 8 * ((lane >> 4) & 1) : 0)) * 16);
    }
    auto dma = [&](bf16_t* Kd, bf16_t* Vd, int c, int sub) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)(c * BLK + sub * KT) * row_bytes;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int blk = NLD * wave + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(Kd + blk * kKBlock), 16, loff_k[i] + soff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(Vd + blk * kVBlock), 16, loff[i] + soff, 0, 0, 0);
        }
    };

    int c = next_chunk(-1), sub = 0;  // every tile has at least its own chunk
    // this row's mask word and bias for a chunk, loaded without a branch (chunk clamped into
    // range); they are loaded one tile ahead, before that tile's K and V, so that they have
    // landed by the barrier that ends the tile before and are read without waiting
    uint32_t mword;
    float dval;
    auto row_view = [&](int cc) __attribute__((always_inline)) {
        const int cq = valid ? min(cc, cpos) : 0;
        mword = mrow[cq >> 5];
        dval = brow[cq];
    };

    // the work on one tile held in (Kc, Vc), while the next one streams into (Kn, Vn)
    auto step = [&](const bf16_t* Kc, const bf16_t* Vc, bf16_t* Kn, bf16_t* Vn)
        __attribute__((always_inline)) {
        const int key0 = c * BLK + sub * KT;
        const bool sel = valid && c <= cpos && (c == cpos || ((mword >> (c & 31)) & 1u));
        const float dcur = dval;
        const int c_nx = sub + 1 < NSUB ? c : next_chunk(c);
        const int sub_nx = sub + 1 < NSUB ? sub + 1 : 0;
        // after the last tile the current one is loaded again into the idle buffers (never read)
        const int c_ld = c_nx >= 0 ? c_nx : c;
        row_view(c_ld);
        dma(Kn, Vn, c_ld, c_nx >= 0 ? sub_nx : sub);
        // a wave none of whose rows selected the chunk has nothing to add (every score -inf)
        if (__any(sel)) {
            const float off = sel ? (c == cpos ? 0.f : dcur * kLog2e) : -INFINITY;
            const bool causal = c >= c_first;  // some row's own chunk: mask keys past each row

            // S^T = K Q^T, the M-tiles' accumulation chains interleaved. The MFMA blocks run at a
            // raised wave priority, so that of the two waves sharing a SIMD the one starting its
            // matrix work issues first and the other's softmax fills the issue slots meanwhile. K
            // fragments are read two k-steps ahead of their MFMAs (a ring of three), so that LDS
            // latency stays off the matrix pipe.
            __builtin_amdgcn_s_setprio(1);
            f32x16 s[MT];
    #pragma unroll
            for (int mt = 0; mt < MT; ++mt) s[mt] = f32x16{};
            {
                constexpr int KS = kD / 16;
                bf16x8 ka[3][MT];
                auto kread = [&](int ks, bf16x8 (&dst)[MT]) __attribute__((always_inline)) {
    #pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        dst[mt] = *reinterpret_cast<const bf16x8*>(Kc + (ks < 4 ? kl_lo : kl_hi) + 16 * ks + mt * (32 / NB) * kD);
                };
                kread(0, ka[0]);
                kread(1, ka[1]);
    #pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 2 < KS) kread(ks + 2, ka[(ks + 2) % 3]);
    #pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % 3][mt], qf[ks], s[mt], 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            // keys past the row's own position score -inf; x = s * scale log2(e) + off is then -inf
            // too (scale > 0), as it is for every key of a row that did not select the chunk
            if (causal) {
    #pragma unroll
                for (int mt = 0; mt < MT; ++mt)
    #pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        const int key = key0 + 32 * mt + 8 * (rr >> 2) + 4 * G + (rr & 3);
                        if (key > pos) s[mt][rr] = -INFINITY;
                    }
            }
            float smax = -INFINITY;
    #pragma unroll
            for (int mt = 0; mt < MT; ++mt)
    #pragma unroll
                for (int rr = 0; rr < 16; ++rr) smax = fmaxf(smax, s[mt][rr]);
            const float xmax = fmaf(halves_max(smax), qk_scale, off);
            // raise the running maximum only when needed (rare once a row has seen its peak)
            const bool raise = xmax > m_used + kLazyMax;
            if (__any(raise)) {
                const float m_new = raise ? xmax : m_used;
                const float corr = m_used == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_used - m_new);
                l_run *= corr;
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= corr;
                m_used = m_new;
            }
            // p = exp2(x - m) as one FMA and exp2; the row sum stays per lane (this half's keys)
            // until the end, since both halves scale it by the same factors
            const float off_m = off - (m_used == -INFINITY ? 0.f : m_used);
            bf16x8 pf[KSTEP];
    #pragma unroll
            for (int ks = 0; ks < KSTEP; ++ks)
    #pragma unroll
                for (int vv = 0; vv < 8; ++vv) {
                    const float pe = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][8 * (ks & 1) + vv], qk_scale, off_m));
                    l_run += pe;
                    pf[ks][vv] = (__bf16)pe;
                }

            // O^T += V^T P^T, V^T through transposing reads issued one k-step ahead of their MFMAs
            __builtin_amdgcn_s_setprio(1);
            {
                bf16x8 va[2][DT];
                auto vread = [&](int ks, bf16x8 (&dst)[DT]) __attribute__((always_inline)) {
    #pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const i16x4 lo = ds_read_tr16(Vc + vl_base[0] + ks * (16 / NB) * kD + 32 * dt);
                        const i16x4 hi = ds_read_tr16(Vc + vl_base[1] + ks * (16 / NB) * kD + 32 * dt);
                        dst[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
                };
                vread(0, va[0]);
    #pragma unroll
                for (int ks = 0; ks < KSTEP; ++ks) {
                    if (ks + 1 < KSTEP) vread(ks + 1, va[(ks + 1) & 1]);
    #pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks & 1][dt], pf[ks], acc[dt], 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        // the next tile has landed in every wave's part, and every wave is done with this one
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();
        c = c_nx;
        sub = sub_nx;
    };

    row_view(c);
    dma(K0, V0, c, 0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    while (true) {
        step(K0, V0, K1, V1);
        if (c < 0) break;
        step(K1, V1, K0, V0);
        if (c < 0) break;
    }

    l_run = halves_sum(l_run);
    if (!valid) return;
    const float inv_l = 1.0f / l_run;
    bf16_t* orow = o + (qrow * p.h_q + r * GQ + hl) * kD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int d0 = 32 * dt + 8 * qd + 4 * G;
            bf16x4 ov;
#pragma unroll
            for (int u = 0; u < 4; ++u) ov[u] = (__bf16)(acc[dt][4 * qd + u] * inv_l);
            *reinterpret_cast<bf16x4*>(orow + d0) = ov;
        }
    if (lse && G == 0) lse[qrow * p.h_q + r * GQ + hl] = (m_used + __log2f(l_run)) * kLn2;
#endif
}

template <int BLK>
static void launch_dma_blk(const void* q, const void* k, const void* v, const uint32_t* mask,
                           const float* bias, void* o, float* lse, const AttnParams& p,
                           hipStream_t st) {
    const int T = kRows / p.g;
    const int n_tiles = div_up(p.n_q, T);
    dim3 grid(p.batch * p.h_kv * n_tiles);
#define DASH_DMA(GG)                                                                        \
    hipLaunchKernelGGL((attn_dma_kernel<BLK, GG>), grid, dim3(kThreads), 0, st,             \
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),        \
                       static_cast<const bf16_t*>(v), mask, bias, static_cast<bf16_t*>(o), \
                       lse, p, n_tiles)
    switch (p.g) {
        case 1: DASH_DMA(1); break;
        case 2: DASH_DMA(2); break;
        case 4: DASH_DMA(4); break;
        case 8: DASH_DMA(8); break;
        default: DASH_DMA(16); break;
    }
#undef DASH_DMA
}

hipError_t launch_attn_prefill_dma(const void* q, const void* k, const void* v,
                                  const uint32_t* mask, const float* bias, void* o, float* lse,
                                  const AttnParams& p, hipStream_t st) {
    if (p.block == 32) launch_dma_blk<32>(q, k, v, mask, bias, o, lse, p, st);
    else if (p.block == 64) launch_dma_blk<64>(q, k, v, mask, bias, o, lse, p, st);
    else launch_dma_blk<128>(q, k, v, mask, bias, o, lse, p, st);
    return hipGetLastError();
}

}  // namespace dash
