// Decode-stage W4A16 / W3A16 product for 1 <= M <= 16 rows of activations
// (the decode kernel of the llm-awq README feature list):
//   y[m][n] = sum_g D[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// HBM-bound: every packed weight byte is read once.  The product runs on
// v_mfma_f32_16x16x32_f16 with the activations as the A operand (M rows,
// zero-padded to 16) and the weights as the B operand, so the cost per
// weight stays flat up to M = 16.
//
// Work split.  The packed format stores tile (b, g) = 16 rows x group g as 64
// lane slots of 16 bytes (slot s = 16h + j: row j, quarter h), contiguous
// along g, with the 16 scales and zeros of the tile in [b][g][16] order.
// Persistent workgroups of WK waves own row blocks blockIdx.x, +gridDim.x,
// ... (the grid is sized to the machine).  Their waves take the groups
// round-robin, so each step of a workgroup reads WK consecutive tiles and a
// block's slab is swept front to back.  Each wave streams its tiles (1 KB
// wave load each, plus the tile's scales and zeros) through a ring of U
// register slots with a fixed-order load stream, so U tiles stay in flight,
// and stages in LDS only the x columns of its own groups.  k_gemv_x1 (x fits
// in LDS, the decode case) stages x once and walks its blocks one after the
// other; k_gemv_xs (larger M * K) sweeps K in slices and keeps one
// accumulator per owned block across the slices.
//
// Dequantization is exact: OR 0x6400 turns a 4-bit code q into the fp16
// value 1024 + q and subtracting 1024 + z leaves q - z, so each group's
// four MFMAs give sum_k x (q - z) with fp32 accumulation; the group scale
// then multiplies the four accumulator lanes of that row (the accumulator
// column of lane s is its own row j).  The waves' partial sums meet in LDS
// and wave 0 adds them in a fixed order: the result is deterministic.
#include "awq_internal.h"

namespace awq {
namespace {

#ifndef AWQ_GEMV_WAVES
#define AWQ_GEMV_WAVES 8
#endif
#ifndef AWQ_GEMV_XBUF
#define AWQ_GEMV_XBUF 65536
#endif
constexpr int kGemvWaves = AWQ_GEMV_WAVES;    // waves per workgroup
constexpr int kGemvXBuf = AWQ_GEMV_XBUF;      // LDS bytes for x staged once (k_gemv_x1)
#ifndef AWQ_GEMV_CU_WAVES
#define AWQ_GEMV_CU_WAVES 16
#endif
constexpr int kGemvCuWaves = AWQ_GEMV_CU_WAVES;  // resident waves per CU for persistent grids
// tiles in flight per wave when x is staged once: 2 while a wave has at most 4
// tiles per row block (a deeper ring only moves dequantization and MFMA work
// behind the last byte to land), 4 for longer rows (measured on MI355X:
// 4096x4096 4.9 us with 2 vs 5.1 with 4; 11008x4096 8.0 us with 4 vs 9.1)
#ifndef AWQ_GEMV_RING_SHORT
#define AWQ_GEMV_RING_SHORT 2
#endif
constexpr int kGemvRingShort = AWQ_GEMV_RING_SHORT;
constexpr int kGemvRingLong = 4;

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// fp16 operand (q - z) of 8 int4 codes in one packed word; zz = 1024 + z for
// the even pairs, zz16 = 64 + z for the odd pairs (see int4_word_pairs).
__device__ __forceinline__ half8_t dequant_word_int4(uint32_t w, half2_t zz, half2_t zz16) {
    uint32_t pr[4];
    int4_word_pairs(w, pr);
    half8_t b;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const half2_t p = as_half2(pr[t]) - ((t & 1) ? zz16 : zz);
        b[2 * t] = p[0];
        b[2 * t + 1] = p[1];
    }
    return b;
}

// fp16 operand (q - z) of int3 codes 8s..8s+7 of a lane slot (pairs 4s..4s+3)
__device__ __forceinline__ half8_t dequant_int3(const uint32_t* w, int s, half2_t zz) {
    half8_t b;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const half2_t p = as_half2(int3_pair_bits(w, 4 * s + t)) - zz;
        b[2 * t] = p[0];
        b[2 * t + 1] = p[1];
    }
    return b;
}

template <int WQ>
struct Slot { uint32_t w[WQ]; };

template <int WQ>
__device__ __forceinline__ Slot<WQ> load_slot(const uint32_t* p) {
    Slot<WQ> s;
    if constexpr (WQ == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        s.w[0] = v.x; s.w[1] = v.y; s.w[2] = v.z; s.w[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < WQ; ++i) s.w[i] = p[i];
    }
    return s;
}

struct Params { _Float16 d, z; };

// x staged once per workgroup (all of x fits in LDS): the common decode case.
//
// Each wave streams its tiles through a ring of U register slots: slot u holds
// item i0 + u of the current block (items are the wave's groups g = wave + WK i,
// padded per block to a multiple of U), and right after the item has been
// consumed the slot is refilled with the item U places further on, which may
// belong to the workgroup's next block.  The load stream is branch-free: items
// past the wave's groups or past the last block are issued as buffer loads at an
// out-of-range offset, which return zero without touching memory.  With a fixed
// number of loads between a slot's fill and its use the compiler waits on
// exactly that slot (vmcnt(3 (U - 1))), so U tiles stay in flight per wave
// through the whole sweep, across row blocks and the reduction barrier.
// minimum waves per SIMD (HIP launch-bounds meaning): 4 keeps two 8-wave
// workgroups resident per CU (<= 128 VGPRs)
#ifndef AWQ_GEMV_MINBLK
#define AWQ_GEMV_MINBLK 4
#endif

// cache policy of the weight tile loads: nt (non-temporal; each byte is read
// once per launch).  Measured on MI355X against the default policy: 4096x4096
// 4.40 vs 4.69 us, 4096x11008 7.09 vs 7.55 us, 8192x28672 / 28672x8192 about
// 3 % faster; sc1 alone changed nothing.  x keeps the default: every
// workgroup reads it.
#ifndef AWQ_GEMV_CPOL
#define AWQ_GEMV_CPOL 2
#endif

constexpr uint32_t kBufferOutOfRange = 0x80000000u;   // > every buffer's size (< 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
    // raw buffer (stride 0): byte offsets, range-checked against `bytes`
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <int WQ>
__device__ __forceinline__ Slot<WQ> buffer_slot(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Slot<WQ> s;
    if constexpr (WQ == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AWQ_GEMV_CPOL);
        s.w[0] = v[0]; s.w[1] = v[1]; s.w[2] = v[2]; s.w[3] = v[3];
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, AWQ_GEMV_CPOL);
        s.w[0] = v[0]; s.w[1] = v[1]; s.w[2] = v[2];
    }
    return s;
}

// a tile's scale and zero as loaded: the aligned 32-bit word holding the
// lane's entry (and its neighbour's), one register each, reduced to the lane's
// half only when the tile is consumed -- narrowing or packing the values at
// load time would make the compiler wait for the loads right away
struct RawParams { uint32_t d, z; };

__device__ __forceinline__ _Float16 low_half(uint32_t v) {
    return __builtin_bit_cast(_Float16, (unsigned short)v);
}

// Kernel arguments.  Entry [1] of the weight arrays is the second layer of a
// fused pair (FUSE: gate = [0], up = [1]); inv_s is read only with SCALE.
struct GemvArgs {
    const _Float16* x;
    const float* inv_s;                      // fp32 [K]: x'[m][k] = fp16(x[m][k] * inv_s[k])
    const uint32_t* qweight[2];
    const _Float16* scales[2];
    const _Float16* zeros[2];
    _Float16* y;
    int M, N, K;
};

// x' = fp16_rne(fp32(x) * inv_s) of one 16-byte chunk of 8 activations
__device__ __forceinline__ uint4 scale_chunk(uint4 v, const float* s) {
    const _Float16* h = reinterpret_cast<const _Float16*>(&v);
    uint4 o;
    _Float16* oh = reinterpret_cast<_Float16*>(&o);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // the fp32 product is rounded before the fp16 conversion (the empty asm
        // keeps the compiler from fusing both into one rounding of the exact
        // product, which differs in the rare double-rounding cases)
        float t = (float)h[e] * s[e];
        asm volatile("" : "+v"(t));
        oh[e] = (_Float16)t;
    }
    return o;
}

// output of a fused gate/up pair from the fp32 sums: SiLU(g) * u, rounded once
__device__ __forceinline__ _Float16 silu_mul(float g, float u) {
    return (_Float16)(g / (1.0f + expf(-g)) * u);
}

// the buffer descriptors of one layer's packed tiles and parameters
struct LayerRsrc { __amdgpu_buffer_rsrc_t q, s, z; };

// acc += D * sum_k x[j][k] * (q[k] - z) over one tile: the four k32 MFMAs of
// a group with x (rows j >= M read row 0) as the A operand from LDS at xa and
// the slot's exact (q - z) as the B operand; the group scale multiplies the
// accumulator lanes of the lane's row.
//
// With 64-wide groups (GS = 64) one MFMA mixes both groups of the tile (its
// k32 slice takes 8 codes from each quarter), so the lane multiplies its
// operand by its own group's scale first: (q - z) * D rounded once to fp16,
// and the MFMA accumulates straight into acc.
template <int BITS, int WQ, int GS>
__device__ __forceinline__ void accumulate_tile(const Slot<WQ>& w, const RawParams& p, const _Float16* xa,
                                                uint32_t psh, float4_t& acc) {
    const _Float16 zh = low_half(p.z >> psh);
    const _Float16 zb = (_Float16)1024.0f + zh;
    const _Float16 zb16 = (_Float16)64.0f + zh;
    const half2_t zz = {zb, zb}, zz16 = {zb16, zb16};
    half8_t bop[4];
    if constexpr (BITS == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) bop[q] = dequant_word_int4(w.w[q], zz, zz16);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) bop[q] = dequant_int3(w.w, q, zz);
    }
    if constexpr (GS == 64) {
        const _Float16 dh = low_half(p.d >> psh);
        const half2_t dd = {dh, dh};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const half2_t v = (half2_t){bop[q][2 * t], bop[q][2 * t + 1]} * dd;
                bop[q][2 * t] = v[0];
                bop[q][2 * t + 1] = v[1];
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8_t*>(xa + 8 * q), bop[q],
                                                         acc, 0, 0, 0);
    } else {
        float4_t accg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8_t*>(xa + 8 * q), bop[q],
                                                          accg, 0, 0, 0);
        const float d = (float)low_half(p.d >> psh);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(d, accg[r], acc[r]);
    }
}

// SCALE: x is multiplied by inv_s while it is staged (each lane loads the
// scale of its first 4 x chunks next to them, 32 bytes per chunk, and that of
// further chunks after the ring's first loads; XL <= 8).  FUSE: the workgroup computes row block b of two
// layers that read the same x (gate, then up): each wave's ring walks its
// gate tiles of the block, then its up tiles, into two accumulators, and the
// block's output is SiLU(gate) * up.
template <int BITS, int GS, int WK, int U, int XL, bool SCALE, bool FUSE>
__global__ __launch_bounds__(64 * WK, AWQ_GEMV_MINBLK) void k_gemv_x1(GemvArgs a) {
    static_assert(!SCALE || XL <= 8, "scaled staging: at most 8 x loads per lane");
    constexpr int SE = SCALE ? (XL < 4 ? XL : 4) : 0;  // chunks whose inv_s is loaded with x
    constexpr int WQ = BITS == 4 ? 4 : 3;
    constexpr int NH = FUSE ? 2 : 1;                   // layers per row block
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int M = a.M, N = a.N, K = a.K;
    const int G = K / kGroup;
    const int NB = (N + 15) / 16;
    const int XS = K + 8;                              // halves per staged x row
    _Float16* xs = reinterpret_cast<_Float16*>(smem);
    float4_t* red = reinterpret_cast<float4_t*>(smem + (((size_t)M * XS * 2 + 15) & ~(size_t)15));

    const int tid = threadIdx.x;
    // FUSE picks a layer's buffer descriptors by the ring position, which
    // depends on wave: stating that wave is uniform keeps them in SGPRs
    const int lane = tid & 63, wave = FUSE ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
    const int j = lane & 15, h = lane >> 4;
    const int nw = wave < G ? (G - wave + WK - 1) / WK : 0;   // groups g = wave + WK i of a block
    const int nwp = (nw + U - 1) / U * U;                       // ring items per block and layer
    const int IB = NH * nwp;                                    // ring items per block
    const _Float16* xa0 = xs + (size_t)(j < M ? j : 0) * XS + 32 * h;
    const uint32_t psh = 16u * (uint32_t)(j & 1);              // the lane's half of a param word

    // the launcher guarantees every buffer is < 2^31 bytes
    const uint32_t tiles = (uint32_t)NB * (uint32_t)G;
    // scales / zeros: [block][group][16], kGroup / GS groups per tile
    LayerRsrc L[NH];
#pragma unroll
    for (int l = 0; l < NH; ++l) {
        L[l].q = buffer_rsrc(a.qweight[l], tiles * 64u * WQ * 4u);
        L[l].s = buffer_rsrc(a.scales[l], tiles * (32u * kGroup / GS));
        L[l].z = buffer_rsrc(a.zeros[l], tiles * (32u * kGroup / GS));
    }
    // this lane's parameter group within a tile: its quarter's (GS = 64)
    const uint32_t pgrp = GS == 64 ? (uint32_t)(h >> 1) : 0u;
    // ring item f of block b: layer f / nwp, group wave + WK (f % nwp)
    auto load = [&](int b, int f, Slot<WQ>& w, RawParams& p) {
        const bool up = FUSE && f >= nwp;              // wave-uniform
        const int i = up ? f - nwp : f;
        const bool ok = b < NB && i < nw;
        const uint32_t t = (uint32_t)b * (uint32_t)G + (uint32_t)(wave + WK * i);
        const uint32_t oq = ok ? (t * 64u + (uint32_t)lane) * (WQ * 4u) : kBufferOutOfRange;
        const uint32_t op = ok ? ((t * (kGroup / GS) + pgrp) * 16u + (uint32_t)(j & ~1)) * 2u
                               : kBufferOutOfRange;
        const LayerRsrc& r = up ? L[NH - 1] : L[0];
        w = buffer_slot<WQ>(r.q, oq);
        p.d = __builtin_amdgcn_raw_buffer_load_b32(r.s, op, 0, 0);
        p.z = __builtin_amdgcn_raw_buffer_load_b32(r.z, op, 0, 0);
    };

    // Each wave stages only the x columns of its own groups (the same groups in
    // every block), so it waits for no other wave before its sweep.  Lanes
    // 16p'..16p'+15 of load p carry the 256-byte (group, row) pair
    // q = (lane >> 4) + 4p as 16-byte chunks; pairs past the wave's nw * M are
    // out-of-range loads whose zeros land in row 0's padding xs[K..K+7], which
    // no read touches.  x is loaded before the ring and the stores are
    // unconditional, so they wait for the x loads alone, and the loads in
    // flight on entry to the sweep are ordered as in the sweep itself.
    const int pairs = nw * M;
    const uint32_t mdiv = 65536u / (uint32_t)M + 1u;   // q / M = (q * mdiv) >> 16 for q < 2048, M <= 16
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, (uint32_t)M * (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t ri = buffer_rsrc(a.inv_s, SCALE ? (uint32_t)K * 4u : 0u);
    uint4 xv[XL];
    uint32_t xat[XL];
    float sv[SE > 0 ? SE : 1][8];
    auto load_inv_s = [&](int p, float* out) {
        const uint32_t q = (uint32_t)((lane >> 4) + 4 * p);
        const uint32_t i = (q * mdiv) >> 16;
        const uint32_t col = (uint32_t)kGroup * (uint32_t)(wave + WK * (int)i) + 8u * (uint32_t)j;
        const uint32_t so = (int)q < pairs ? col * 4u : kBufferOutOfRange;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const auto f = __builtin_amdgcn_raw_buffer_load_b128(ri, so + 16u * c, 0, 0);
            // through a scalar: a bit_cast of the vector element itself
            // keeps only element 0 of the load with this compiler
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t u = f[e];
                out[4 * c + e] = __builtin_bit_cast(float, u);
            }
        }
    };
#pragma unroll
    for (int p = 0; p < XL; ++p) {
        const uint32_t q = (uint32_t)((lane >> 4) + 4 * p);
        const uint32_t i = (q * mdiv) >> 16, m = q - i * (uint32_t)M;
        const uint32_t col = (uint32_t)kGroup * (uint32_t)(wave + WK * (int)i) + 8u * (uint32_t)j;
        const bool ok = (int)q < pairs;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(
            rx, ok ? (m * (uint32_t)K + col) * 2u : kBufferOutOfRange, 0, 0);
        xv[p] = make_uint4(v[0], v[1], v[2], v[3]);
        xat[p] = ok ? m * (uint32_t)XS + col : (uint32_t)K;
        if (p < SE) load_inv_s(p, sv[p < SE ? p : 0]);
    }
    Slot<WQ> ring[U];
    RawParams pr[U];
    int b = blockIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load(b, u, ring[u], pr[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < XL; ++p) {
        uint4 v = xv[p];
        if constexpr (SCALE) {
            if (p < SE) {
                v = scale_chunk(v, sv[p < SE ? p : 0]);
            } else {
                // chunks past the first 4: inv_s loaded only now (behind the
                // ring, once per workgroup), so it never shares registers with
                // the first chunks' scales
                float t[8];
                load_inv_s(p, t);
                v = scale_chunk(v, t);
            }
        }
        *reinterpret_cast<uint4*>(xs + xat[p]) = v;
    }
    // the wave's own LDS stores complete before its lanes read each other's chunks
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // grid <= NB, so every workgroup has a first block; a loop without an entry
    // test keeps the compiler from sinking the ring loads above into it
    int buf = 0;
    do {
        const int bn = b + gridDim.x;                  // next block of this workgroup
        float4_t acc[NH];
#pragma unroll
        for (int l = 0; l < NH; ++l) acc[l] = (float4_t){0.f, 0.f, 0.f, 0.f};
        for (int f0 = 0; f0 < IB; f0 += U) {
            // nwp is a multiple of U: a ring round belongs to one layer
            const bool upr = FUSE && f0 >= nwp;
            const int i0 = upr ? f0 - nwp : f0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u;
                if (i < nw) {                          // wave-uniform; loads stay outside
                    const _Float16* xa = xa0 + (size_t)(wave + WK * i) * kGroup;
                    if (FUSE && upr)
                        accumulate_tile<BITS, WQ, GS>(ring[u], pr[u], xa, psh, acc[NH - 1]);
                    else
                        accumulate_tile<BITS, WQ, GS>(ring[u], pr[u], xa, psh, acc[0]);
                }
                // refill the slot with the item U places on (this block or the next)
                const int k = f0 + u + U;
                const bool here = k < IB;
                load(here ? b : bn, here ? k : k - IB, ring[u], pr[u]);
            }
        }
#pragma unroll
        for (int l = 0; l < NH; ++l) red[((buf * NH + l) * WK + wave) * 64 + lane] = acc[l];
        __syncthreads();
        if (wave == 0) {
            float4_t sum[NH];
#pragma unroll
            for (int l = 0; l < NH; ++l) {
                sum[l] = red[((buf * NH + l) * WK) * 64 + lane];
#pragma unroll
                for (int w = 1; w < WK; ++w) {
                    const float4_t o = red[((buf * NH + l) * WK + w) * 64 + lane];
                    sum[l][0] += o[0]; sum[l][1] += o[1]; sum[l][2] += o[2]; sum[l][3] += o[3];
                }
            }
            const int n = 16 * b + j;
            if (n < N) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * h + r;
                    if (m < M)
                        a.y[(size_t)m * N + n] = FUSE ? silu_mul(sum[0][r], sum[NH - 1][r]) : (_Float16)sum[0][r];
                }
            }
        }
        buf ^= 1;
        b = bn;
    } while (b < NB);
}


using GemvFn = void (*)(GemvArgs);

// x too large for LDS at once (M rows, M * K > 32K halves): K is swept in
// slices of SG = WK * U groups, x staged one slice at a time, each wave
// staging only its own U groups' columns (no workgroup barrier).  A
// persistent workgroup owns up to BMAX row blocks (blockIdx.x + k gridDim.x)
// and keeps one accumulator per block across all slices, so every staged x
// slice serves all of them.  Per slice and block each wave has exactly U
// items, one ring round: the slice body is fully unrolled and its load
// stream fixed (items past G or past the last block are out-of-range loads),
// so the compiler's waits cover exactly one ring slot; the next slice's x is
// loaded into registers during the current slice, ahead of its ring loads.
// The waves' partial sums meet in LDS once per block at the end.
//
// SCALE: each wave also loads the inv_s of its U = 2 groups of the next slice
// (one 16-byte load per lane), parks it in its own 1 KB of LDS while staging,
// and multiplies every x chunk by the 8 values of the chunk's columns on the
// way into the x slice; with 8 x loads per lane (M >= 13) the next slice's x
// and inv_s are loaded at the end of the current slice rather than at its
// start, which keeps them out of the registers live during the sweep.  FUSE: the workgroup owns one
// row block of two layers reading the same x (gate, up; BMAX = 1) and keeps an
// accumulator for each; the block's output is SiLU(gate) * up.
template <int BITS, int GS, int WK, int U, int BMAX, int XL, bool SCALE, bool FUSE>
__global__ __launch_bounds__(64 * WK, AWQ_GEMV_MINBLK) void k_gemv_xs(GemvArgs a) {
    static_assert(!FUSE || BMAX == 1, "a fused pair takes the two accumulators");
    static_assert(!SCALE || U == 2, "a wave's inv_s slice is 64 lanes x 4 floats = 2 groups");
    constexpr int WQ = BITS == 4 ? 4 : 3;
    constexpr int SG = WK * U;                         // groups per slice
    constexpr int XS = SG * kGroup + 8;                // halves per staged x row
    constexpr int NA = FUSE ? 2 : BMAX;                // accumulators: (block, layer) items
    constexpr bool LATE = SCALE && XL > 4;             // next slice's x loaded after the sweep
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int M = a.M, N = a.N, K = a.K;
    _Float16* xs = reinterpret_cast<_Float16*>(smem);
    float4_t* red = reinterpret_cast<float4_t*>(smem);   // after the sweep, over x
    const int G = K / kGroup;
    const int NB = (N + 15) / 16;
    const int NS = (G + SG - 1) / SG;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, h = lane >> 4;
    const _Float16* xa0 = xs + (size_t)(j < M ? j : 0) * XS + 32 * h;
    const uint32_t psh = 16u * (uint32_t)(j & 1);
    // SCALE: this wave's inv_s of the slice being staged, [U][kGroup] fp32
    float* sw = reinterpret_cast<float*>(smem + (((size_t)M * XS * 2 + 15) & ~(size_t)15)) + wave * U * kGroup;

    const uint32_t tiles = (uint32_t)NB * (uint32_t)G;
    constexpr int NH = FUSE ? 2 : 1;
    LayerRsrc L[NH];
#pragma unroll
    for (int l = 0; l < NH; ++l) {
        L[l].q = buffer_rsrc(a.qweight[l], tiles * 64u * WQ * 4u);
        // scales / zeros: [block][group][16], kGroup / GS groups per tile
        L[l].s = buffer_rsrc(a.scales[l], tiles * (32u * kGroup / GS));
        L[l].z = buffer_rsrc(a.zeros[l], tiles * (32u * kGroup / GS));
    }
    // this lane's parameter group within a tile: its quarter's (GS = 64)
    const uint32_t pgrp = GS == 64 ? (uint32_t)(h >> 1) : 0u;
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, (uint32_t)M * (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t ri = buffer_rsrc(a.inv_s, SCALE ? (uint32_t)K * 4u : 0u);

    // accumulator item k: block blockIdx.x + k gridDim.x, or (FUSE) layer k of block blockIdx.x
    auto item_block = [&](int k) { return FUSE ? (int)blockIdx.x : (int)blockIdx.x + k * (int)gridDim.x; };
    // item (s, k, u): item k's tile of group s SG + wave + WK u
    auto load = [&](int s, int k, int u, Slot<WQ>& w, RawParams& p) {
        const int b = item_block(k);
        const int g = s * SG + wave + WK * u;
        const bool ok = b < NB && g < G;
        const uint32_t t = (uint32_t)b * (uint32_t)G + (uint32_t)g;
        const uint32_t oq = ok ? (t * 64u + (uint32_t)lane) * (WQ * 4u) : kBufferOutOfRange;
        const uint32_t op = ok ? ((t * (kGroup / GS) + pgrp) * 16u + (uint32_t)(j & ~1)) * 2u
                               : kBufferOutOfRange;
        const LayerRsrc& r = (FUSE && k == 1) ? L[NH - 1] : L[0];
        w = buffer_slot<WQ>(r.q, oq);
        p.d = __builtin_amdgcn_raw_buffer_load_b32(r.s, op, 0, 0);
        p.z = __builtin_amdgcn_raw_buffer_load_b32(r.z, op, 0, 0);
    };
    // the wave's x of slice s: (group u, row m) pairs q = (lane >> 4) + 4p as
    // 16-byte chunks; pairs past U * M land in row 0's padding xs[SG*128 ..]
    const uint32_t mdiv = 65536u / (uint32_t)M + 1u;   // q / M = (q * mdiv) >> 16 for q < 2048, M <= 16
    auto x_at = [&](int p) -> uint32_t {               // LDS position of chunk p (recomputed: registers)
        const uint32_t q = (uint32_t)((lane >> 4) + 4 * p);
        const uint32_t u = (q * mdiv) >> 16, m = q - u * (uint32_t)M;
        const uint32_t col = (uint32_t)kGroup * (uint32_t)(wave + WK * (int)u) + 8u * (uint32_t)j;
        return (int)q < U * M ? m * (uint32_t)XS + col : (uint32_t)(SG * kGroup);
    };
    auto load_x = [&](int s, uint4* xv) {
#pragma unroll
        for (int p = 0; p < XL; ++p) {
            const uint32_t q = (uint32_t)((lane >> 4) + 4 * p);
            const uint32_t u = (q * mdiv) >> 16, m = q - u * (uint32_t)M;
            const int g = s * SG + wave + WK * (int)u;
            const bool ok = (int)q < U * M && g < G;
            const uint32_t off = (m * (uint32_t)K + (uint32_t)kGroup * (uint32_t)g + 8u * (uint32_t)j) * 2u;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? off : kBufferOutOfRange, 0, 0);
            xv[p] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    // SCALE: lane l carries inv_s of group l / 32 of the wave's pair, columns 4 (l % 32) ..
    auto load_s = [&](int s) -> uint4 {
        const int g = s * SG + wave + WK * (lane >> 5);
        const uint32_t off = ((uint32_t)kGroup * (uint32_t)g + 4u * (uint32_t)(lane & 31)) * 4u;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(ri, g < G ? off : kBufferOutOfRange, 0, 0);
        return make_uint4(v[0], v[1], v[2], v[3]);
    };

    uint4 xv[XL];
    uint4 sv = make_uint4(0, 0, 0, 0);
    Slot<WQ> ring[U];
    RawParams pr[U];
    load_x(0, xv);
    if constexpr (SCALE) sv = load_s(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load(0, 0, u, ring[u], pr[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
    float4_t acc[NA];
#pragma unroll
    for (int k = 0; k < NA; ++k) acc[k] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // NS >= 1: no entry test, so the loads above stay where they are
    int s = 0;
    do {
        // stage slice s (this wave's reads of slice s - 1 precede in program order)
        if constexpr (SCALE) {
            *reinterpret_cast<uint4*>(sw + 4 * lane) = sv;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int p = 0; p < XL; ++p) {
                const uint32_t q = (uint32_t)((lane >> 4) + 4 * p);
                const uint32_t u = min((q * mdiv) >> 16, (uint32_t)(U - 1));   // pairs past U * M: any
                float f[8];
                *reinterpret_cast<float4*>(f) = *reinterpret_cast<const float4*>(sw + u * kGroup + 8 * j);
                *reinterpret_cast<float4*>(f + 4) = *reinterpret_cast<const float4*>(sw + u * kGroup + 8 * j + 4);
                *reinterpret_cast<uint4*>(xs + x_at(p)) = scale_chunk(xv[p], f);
            }
        } else {
#pragma unroll
            for (int p = 0; p < XL; ++p) *reinterpret_cast<uint4*>(xs + x_at(p)) = xv[p];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!LATE) {
            load_x(s + 1, xv);
            if constexpr (SCALE) sv = load_s(s + 1);
        }
#pragma unroll
        for (int k = 0; k < NA; ++k) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = s * SG + wave + WK * u;
                if (item_block(k) < NB && g < G)     // wave-uniform
                    accumulate_tile<BITS, WQ, GS>(ring[u], pr[u], xa0 + (size_t)(wave + WK * u) * kGroup, psh, acc[k]);
                // refill: the same group of the next item, or of the first item in the next slice
                if (k + 1 < NA)
                    load(s, k + 1, u, ring[u], pr[u]);
                else
                    load(s + 1, 0, u, ring[u], pr[u]);
            }
        }
        if constexpr (LATE) {
            // the next slice's x and inv_s only now, behind the ring refills of
            // its first tiles (needed right after its staging anyway): they are
            // not live during the sweep, which keeps M >= 13 within 128 VGPRs
            __builtin_amdgcn_sched_barrier(0);
            load_x(s + 1, xv);
            sv = load_s(s + 1);
        }
        ++s;
    } while (s < NS);

    __syncthreads();                                   // every wave is done with x
    if constexpr (FUSE) {
        red[(0 * WK + wave) * 64 + lane] = acc[0];
        red[(1 * WK + wave) * 64 + lane] = acc[1];
        __syncthreads();
        const int b = blockIdx.x;
        if (wave == 0) {
            float4_t sum[2];
#pragma unroll
            for (int l = 0; l < 2; ++l) {
                sum[l] = red[(l * WK) * 64 + lane];
#pragma unroll
                for (int w = 1; w < WK; ++w) {
                    const float4_t o = red[(l * WK + w) * 64 + lane];
                    sum[l][0] += o[0]; sum[l][1] += o[1]; sum[l][2] += o[2]; sum[l][3] += o[3];
                }
            }
            const int n = 16 * b + j;
            if (n < N) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * h + r;
                    if (m < M) a.y[(size_t)m * N + n] = silu_mul(sum[0][r], sum[1][r]);
                }
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < BMAX; ++k) {
            const int buf = k & 1;
            red[(buf * WK + wave) * 64 + lane] = acc[k];
            __syncthreads();
            const int b = blockIdx.x + k * gridDim.x;
            if (wave == 0 && b < NB) {
                float4_t sum = red[(buf * WK) * 64 + lane];
#pragma unroll
                for (int w = 1; w < WK; ++w) {
                    const float4_t o = red[(buf * WK + w) * 64 + lane];
                    sum[0] += o[0]; sum[1] += o[1]; sum[2] += o[2]; sum[3] += o[3];
                }
                const int n = 16 * b + j;
                if (n < N) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 4 * h + r;
                        if (m < M) a.y[(size_t)m * N + n] = (_Float16)sum[r];
                    }
                }
            }
        }
    }
}

constexpr int kGemvSliceRing = 2;                      // U of k_gemv_xs: slices of 2 * WK groups

template <int BITS, int GS, bool SC, bool FU, int WK, int BMAX>
GemvFn pick_xs_loads(int xl) {
    if (xl <= 2) return k_gemv_xs<BITS, GS, WK, kGemvSliceRing, BMAX, 2, SC, FU>;
    if (xl <= 4) return k_gemv_xs<BITS, GS, WK, kGemvSliceRing, BMAX, 4, SC, FU>;
    return k_gemv_xs<BITS, GS, WK, kGemvSliceRing, BMAX, 8, SC, FU>;
}
template <int BITS, int GS, bool SC, bool FU, int WK>
GemvFn pick_xs(int bmax, int xl) {
    if constexpr (FU) return pick_xs_loads<BITS, GS, SC, FU, WK, 1>(xl);
    else return bmax <= 1 ? pick_xs_loads<BITS, GS, SC, FU, WK, 1>(xl)
                          : pick_xs_loads<BITS, GS, SC, FU, WK, 2>(xl);
}

// k_gemv_x1 instance: ring depth (short rows: 2, else 4) and the number of
// 16-byte x loads per lane that stage a wave's (group, row) pairs (<= 12:
// M * K <= 32768 gives at most 48 pairs per wave; <= 8 with SCALE)
template <int BITS, int GS, bool SC, bool FU, int U>
GemvFn pick_x1_loads(int xl) {
    if (xl <= 1) return k_gemv_x1<BITS, GS, kGemvWaves, U, 1, SC, FU>;
    if (xl <= 2) return k_gemv_x1<BITS, GS, kGemvWaves, U, 2, SC, FU>;
    if (xl <= 4) return k_gemv_x1<BITS, GS, kGemvWaves, U, 4, SC, FU>;
    if (xl <= 8) return k_gemv_x1<BITS, GS, kGemvWaves, U, 8, SC, FU>;
    if constexpr (!SC) return k_gemv_x1<BITS, GS, kGemvWaves, U, 12, SC, FU>;
    return nullptr;
}
template <int BITS, int GS, bool SC, bool FU>
GemvFn pick_x1(bool short_rows, int xl) {
    return short_rows ? pick_x1_loads<BITS, GS, SC, FU, kGemvRingShort>(xl)
                      : pick_x1_loads<BITS, GS, SC, FU, kGemvRingLong>(xl);
}

int set_lds(GemvFn kern, size_t lds) {
    if (lds <= 64 * 1024) return 0;
    return (int)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// the K-sliced kernel with WK waves per workgroup
template <int BITS, int GS, bool SC, bool FU, int WK>
int launch_xs(const GemvArgs& a, int cus, hipStream_t st) {
    const int M = a.M, N = a.N;
    const int NB = (N + 15) / 16;
    constexpr int SG = WK * kGemvSliceRing;
    const size_t red = 2 * (size_t)WK * 64 * 16;
    const size_t xsl = ((size_t)M * (SG * kGroup + 8) * 2 + 15) & ~(size_t)15;
    const size_t lds = max(xsl + (SC ? (size_t)SG * kGroup * 4 : 0), red);
    const int per_cu = max(1, min(kGemvCuWaves / WK, (int)((160 * 1024) / lds)));
    int grid = FU ? NB : max(min(NB, cus * per_cu), (NB + 1) / 2);
    // long rows at M >= 8: two blocks per workgroup stage x half as often, which
    // pays once the halved grid still covers every CU (MI355X, 28672x8192 at
    // M = 8 / 16: 35.4 -> 32.7 / 46.0 -> 38.5 us; K = 4096 or 11008, or fewer
    // blocks, measured slower)
    if (!FU && WK == kGemvWaves && M >= 8 && a.K >= 16384 && (NB + 1) / 2 >= cus) grid = (NB + 1) / 2;
    const int bmax = (NB + grid - 1) / grid;
    auto kern = pick_xs<BITS, GS, SC, FU, WK>(bmax, (kGemvSliceRing * M + 3) / 4);
    if (int e = set_lds(kern, lds)) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WK), lds, st, a);
    return 0;
}

// SC: inv_s folded into the x staging; FU: a gate/up pair with the SiLU * up output
template <int BITS, int GS, bool SC, bool FU>
int launch_bits(const GemvArgs& a, hipStream_t st) {
    const int M = a.M, N = a.N, K = a.K;
    const int G = K / kGroup;
    const int NB = (N + 15) / 16;
    constexpr size_t WQ = BITS == 4 ? 4 : 3;
    constexpr int NH = FU ? 2 : 1;
    // the kernels address their buffers with 32-bit offsets (the API rejects
    // larger matrices)
    if ((size_t)NB * G * 64 * WQ * 4 >= ((size_t)1 << 31)) return (int)hipErrorInvalidValue;
    const int cus = device_cu_count();
    const int xl1 = ((G + kGemvWaves - 1) / kGemvWaves * M + 3) / 4;   // x1: x loads per lane
    if ((size_t)M * (K + 8) * 2 <= (size_t)kGemvXBuf && (!SC || xl1 <= 8)) {
        // x staged once; persistent workgroups (as many as fit on a CU by LDS,
        // at most kGemvCuWaves waves)
        const size_t red = 2 * NH * (size_t)kGemvWaves * 64 * 16;
        const size_t lds = (((size_t)M * (K + 8) * 2 + 15) & ~(size_t)15) + red;
        auto kern = pick_x1<BITS, GS, SC, FU>(G <= 4 * kGemvWaves, xl1);
        if (!kern) return (int)hipErrorInvalidValue;
        if (int e = set_lds(kern, lds)) return e;
        const int per_cu = max(1, min(kGemvCuWaves / kGemvWaves, (int)((160 * 1024) / lds)));
        const int grid = min(NB, cus * per_cu);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kGemvWaves), lds, st, a);
    } else {
        // K in slices; up to 2 row blocks per workgroup (4 per workgroup reads
        // x half as often but spills at M = 16; measured on MI355X, 8192x28672
        // at M = 16: 39.5 us with 2, 41.8 us with 4); a fused pair is one block
        // of two layers, which reads x as often.  Wide layers (>= 1024 row
        // blocks) take 4-wave workgroups (slices of 8 groups, twice as many
        // workgroups per CU): 8192x28672 at M = 4 27.4 -> 24.9 us, M = 16 37.8
        // -> 36.7 us; narrower ones keep 8 waves (4096x4096 at M = 16: 5.9 vs
        // 6.0 us)
        const int e = NB >= 1024 ? launch_xs<BITS, GS, SC, FU, 4>(a, cus, st)
                                 : launch_xs<BITS, GS, SC, FU, kGemvWaves>(a, cus, st);
        if (e) return e;
    }
    return (int)hipGetLastError();
}

template <bool SC, bool FU>
int launch_mode(const GemvArgs& a, int bits, int group_size, hipStream_t st) {
    if (group_size == 64)
        return bits == 4 ? launch_bits<4, 64, SC, FU>(a, st) : launch_bits<3, 64, SC, FU>(a, st);
    return bits == 4 ? launch_bits<4, 128, SC, FU>(a, st) : launch_bits<3, 128, SC, FU>(a, st);
}

}  // namespace

int device_cu_count() {
    // per call (the runtime caches device attributes), for the current device
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
        return v;
    return 256;
}

int launch_gemv(const void* x, const float* inv_s, const void* qweight, const void* scales,
                const void* zeros, const void* qweight2, const void* scales2, const void* zeros2,
                void* y, int M, int N, int K, int bits, int group_size, hipStream_t st) {
    GemvArgs a{};
    a.x = (const _Float16*)x;
    a.inv_s = inv_s;
    a.qweight[0] = (const uint32_t*)qweight;
    a.scales[0] = (const _Float16*)scales;
    a.zeros[0] = (const _Float16*)zeros;
    a.qweight[1] = (const uint32_t*)qweight2;
    a.scales[1] = (const _Float16*)scales2;
    a.zeros[1] = (const _Float16*)zeros2;
    a.y = (_Float16*)y;
    a.M = M; a.N = N; a.K = K;
    const bool fuse = qweight2 != nullptr;
    if (inv_s)
        return fuse ? launch_mode<true, true>(a, bits, group_size, st)
                    : launch_mode<true, false>(a, bits, group_size, st);
    return fuse ? launch_mode<false, true>(a, bits, group_size, st)
                : launch_mode<false, false>(a, bits, group_size, st);
}

}  // namespace awq
