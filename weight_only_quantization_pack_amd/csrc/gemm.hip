// Context-stage (prefill) W4A16 GEMM and the dense fp16 loss GEMM of the
// scale search, both on fp16 MFMA with fp32 accumulation.
//
// Y[m][n] = sum_k X[m][k] * B[n][k]   ("NT": both operands K-contiguous)
//
// W4A16 (k_gemm_w4; context kernel of the llm-awq README feature list,
// version "gemm" of the transformers quantization_config).  B is the packed
// packed weight: tile (b, g) = 16 rows x group g, lane slot s = 16h + j
// holding row j's codes 32h..32h+31, which is exactly the B-operand layout
// of v_mfma_f32_16x16x32_f16 for the four k32 steps of the group (step i
// uses word i of every slot, physical k = 128g + 32h + 8i + e).  So each
// wave loads its B tiles straight from HBM/L2 into registers (one 16-byte
// load per tile per lane, prefetched a group ahead) and dequantizes them in
// registers: OR 0x6400 gives 1024 + q in fp16, subtracting 1024 + z is
// exact, one fp16 multiply by the group scale gives w_hat.  Only A (the
// fp16 activations) goes through LDS: global_load_lds_dwordx4 writes each
// 128 x 128 A tile straight to LDS (no register staging), double-buffered,
// with the 16-byte chunks of a row XOR-swizzled by the row so that the
// MFMA operand reads (8 rows per LDS phase) hit distinct banks.
// A workgroup (4 waves) owns a 128 x 256 output tile; each wave a 128 x 64
// strip (8 x 4 MFMA blocks, 128 fp32 accumulators per lane), so per k32 step
// a wave reads 8 A fragments from LDS and dequantizes 4 B fragments for 32
// MFMAs.  The pipelined kernel also has 128 x 384 and 128 x 448 tiles, and
// takes a template wave count: 128 x 256 and 128 x 384 run as 8 waves of 2 or
// 3 column blocks (two waves per SIMD), 128 x 448 as 4 waves of 7 (224
// accumulators per lane in AGPRs, the same A fragments feeding 56 MFMAs); the
// tile count of N = 6144 or 14336 becomes a whole number of rounds on 256 CUs.
// Each XCD (workgroup id mod 8) takes one block of the tile grid, cut per
// shape so that its L2 serves the activation rows and weight columns its
// tiles share (xcd_rows_for).
//
// Two schedules of that tile: k_gemm_w4 double-buffers A and B (one K-step
// ahead) at two workgroups per CU; k_gemm_w4p keeps three K-steps in flight
// (four 32 KB A buffers, four B register slots) at one workgroup per CU, with
// the next k32 substep's A fragments and B operands prepared under the
// current substep's MFMAs.  gemm_tile_choice picks the kernel and tile width
// from the rounds each option takes on the CUs.
//
// Loss GEMM (k_loss_gemm_p): B = D_alpha = W - w_hat_alpha / s_alpha (fp16,
// in a tiled layout the search's error kernel writes), the pipelined kernel's
// schedule with fp16 B operands, and an epilogue that sums Y^2 per tile
// instead of storing Y.
#include <climits>
#include <type_traits>

#include "awq_internal.h"

namespace awq {
namespace {

// wave priority of k_gemm_w4 while it issues a K-step's MFMAs: its two
// workgroups per CU put two waves on each SIMD, and the one in its MFMA phase
// goes first while the other loads and dequantizes (MI355X, M = 2048:
// 4096x6144 118-119 vs 123-124 us, 4096x14336 284-289 vs 291-292 us)
#ifndef AWQ_GEMM_PRIO
#define AWQ_GEMM_PRIO 1
#endif

// the k_gemm_w4p tiles with at least this many 16-column blocks per wave
// dequantize each B tile just before its MFMAs (fewer live registers)
#ifndef AWQ_GEMM_ILV
#define AWQ_GEMM_ILV 7
#endif

// raw buffer resource over `bytes` bytes (byte offsets, range-checked)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from buffer byte offset voff + soff straight into LDS at
// lds + 16 * lane (a direct-to-LDS buffer load)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff,
                                                  uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// The 16-byte chunk position that holds global chunk kc of A row r in LDS is
// kc ^ a_swz(r).  An A-fragment read has lane (j, hq) fetch chunk 4 hq + s of
// row 16 i + j; measured on MI355X (SQ_LDS_BANK_CONFLICT), XOR-ing with r & 15
// costs 4 conflict cycles per 8-cycle ds_read_b128, while any bit permutation
// of r & 15 that puts bit 0 or 1 of the row into bit 2 of the XOR is free of
// conflicts.  a_swz swaps bits 0 and 2.
__device__ __forceinline__ int a_swz(int r) {
    return (r & 0xA) | ((r & 1) << 2) | ((r >> 2) & 1);
}

namespace w4 {
constexpr int GM = 128, GN = 256, GK = 128;    // workgroup tile; GK = one group
constexpr int ROW_BYTES = GK * 2;              // one A row of a K-step in LDS
constexpr int ABUF = GM * ROW_BYTES;           // 32 KB per A buffer
}  // namespace w4

// fp16 B operand w_hat = (q - z) * D of the 8 int4 codes of one packed word;
// zz = 1024 + z (even pairs), zz16 = 64 + z (odd pairs, see int4_word_pairs)
__device__ __forceinline__ half8_t dequant_scaled(uint32_t w, half2_t zz, half2_t zz16, half2_t dd) {
    uint32_t pr[4];
    int4_word_pairs(w, pr);
    half8_t b;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const half2_t p = (as_half2(pr[t]) - ((t & 1) ? zz16 : zz)) * dd;
        b[2 * t] = p[0];
        b[2 * t + 1] = p[1];
    }
    return b;
}

// fp16 B operand w_hat = (q - z) * D of 8 int3 codes held in the low 24 bits
// of v (code e at bits 3e..3e+2); zz = 1024 + z
__device__ __forceinline__ half8_t dequant_scaled_int3(const uint32_t* w, int s, half2_t zz, half2_t dd) {
    half8_t b;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const half2_t p = (as_half2(int3_pair_bits(w, 4 * s + t)) - zz) * dd;
        b[2 * t] = p[0];
        b[2 * t + 1] = p[1];
    }
    return b;
}

__global__ __launch_bounds__(256, 2) void k_gemm_w4(
    const _Float16* __restrict__ A, const uint32_t* __restrict__ qw,
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    _Float16* __restrict__ Y, int M, int N, int K) {
    using namespace w4;
    __shared__ __attribute__((aligned(16))) unsigned char As[2 * ABUF];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: SGPR math
    const int j = lane & 15, hq = lane >> 4;
    const int G = K / kGroup;
    const int NB = (N + 15) / 16;
    const int nTn = (N + GN - 1) / GN, nTm = (M + GM - 1) / GM;
    const int nT = nTn * nTm;

    // XCD-aware order: workgroup t runs on XCD t % 8; give each XCD a
    // contiguous run of row-major tiles so that its tiles share A rows
    int t = blockIdx.x;
    if (nT % 8 == 0) t = (t % 8) * (nT / 8) + t / 8;
    const int m0 = (t / nTn) * GM, n0 = (t % nTn) * GN;

    // A: 32 direct-to-LDS instructions per K-step (1 KB = 4 rows each), 8 per
    // wave.  Lane l of instruction rg writes LDS chunk p = l & 15 of row
    // r = 4 rg + (l >> 4), which holds the row's global chunk p ^ a_swz(r), so
    // that the A-fragment reads are free of bank conflicts.
    // 32-bit element offsets into A (the launcher guarantees M * K < 2^31)
    uint32_t a_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int rg = wave * 8 + i;
        const int r = 4 * rg + (lane >> 4);
        const int kc = (lane & 15) ^ a_swz(r);
        const int grow = min(m0 + r, M - 1);          // rows past M: any valid row (never stored)
        a_off[i] = (uint32_t)grow * (uint32_t)K + 8u * kc;
    }
    auto issue_a = [&](int kt, int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int rg = wave * 8 + i;
            __builtin_amdgcn_global_load_lds((global_void_t*)(A + a_off[i] + (uint32_t)kt * GK),
                                             (lds_void_t*)(As + buf * ABUF + rg * 1024), 16, 0, 0);
        }
    };

    // B: this wave's four 16-row blocks of the 256-column tile
    // tile index of this wave's four 16-row blocks at group 0 (N * K / 2048 < 2^31)
    uint32_t tbase[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int blk = min(n0 / 16 + wave * 4 + c, NB - 1);   // blocks past N: never stored
        tbase[c] = (uint32_t)blk * (uint32_t)G;
    }
    uint4 bq[4], bq_next[4];
    half2_t bp[4], bp_next[4];                          // (scale, zero) of each block's row j
    auto load_b = [&](int g, uint4* q, half2_t* p) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t tt = tbase[c] + (uint32_t)g;
            q[c] = *reinterpret_cast<const uint4*>(qw + (size_t)(tt * 256u + 4u * lane));
            p[c] = (half2_t){scales[tt * 16u + j], zeros[tt * 16u + j]};
        }
    };

    float4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = (float4_t){0.f, 0.f, 0.f, 0.f};

    issue_a(0, 0);
    load_b(0, bq, bp);
    for (int kt = 0; kt < G; ++kt) {
        const int buf = kt & 1;
        __builtin_amdgcn_s_waitcnt(0);                 // this wave's A(kt) landed in LDS
        __syncthreads();                               // everyone's A(kt) landed; A(kt-1) reads done
        if (kt + 1 < G) {
            issue_a(kt + 1, buf ^ 1);
            load_b(kt + 1, bq_next, bp_next);
        }
        half2_t zz[4], zz16[4], dd[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const _Float16 zb = (_Float16)1024.0f + bp[c][1];
            const _Float16 zb16 = (_Float16)64.0f + bp[c][1];
            zz[c] = (half2_t){zb, zb};
            zz16[c] = (half2_t){zb16, zb16};
            dd[c] = (half2_t){bp[c][0], bp[c][0]};
        }
        const unsigned char* abuf = As + buf * ABUF;
#if AWQ_GEMM_PRIO
        __builtin_amdgcn_s_setprio(AWQ_GEMM_PRIO);
#endif
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8_t b[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w = s == 0 ? bq[c].x : s == 1 ? bq[c].y : s == 2 ? bq[c].z : bq[c].w;
                b[c] = dequant_scaled(w, zz[c], zz16[c], dd[c]);
            }
            const int kc = 4 * hq + s;                  // A chunk matching the B k-slots
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 16 * i + j;
                const half8_t a = *reinterpret_cast<const half8_t*>(
                    abuf + r * ROW_BYTES + ((kc ^ a_swz(r)) << 4));
                // weights as the A operand, activations as B: the accumulator of
                // lane 16 hq + j then holds output row m = 16 i + j and the four
                // consecutive columns 16 c + 4 hq + r
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[c], a, acc[i][c], 0, 0, 0);
            }
            // schedule hint: 4 LDS reads up front, then (4 MFMAs, 1 LDS read) x 4 so
            // reads run ahead of their MFMAs, then the remaining 16 MFMAs each
            // followed by up to 3 VALU ops (the next step's dequantization)
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
        }
#if AWQ_GEMM_PRIO
        __builtin_amdgcn_s_setprio(0);
#endif
#pragma unroll
        for (int c = 0; c < 4; ++c) { bq[c] = bq_next[c]; bp[c] = bp_next[c]; }
    }

    // accumulator of lane 16 hq + j, block (i, c): row m = 16 i + j, columns
    // 16 c + 4 hq + r (r = 0..3) -> one 8-byte store when all four are in range
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int m = m0 + 16 * i + j;
        if (m >= M) continue;
        _Float16* yrow = Y + (size_t)m * N;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int n = n0 + wave * 64 + 16 * c + 4 * hq;
            const half2_t lo = {(_Float16)acc[i][c][0], (_Float16)acc[i][c][1]};
            const half2_t hi = {(_Float16)acc[i][c][2], (_Float16)acc[i][c][3]};
            if (n + 3 < N && ((N & 3) == 0)) {
                *reinterpret_cast<uint2*>(yrow + n) = make_uint2(as_u32(lo), as_u32(hi));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) yrow[n + r] = (_Float16)acc[i][c][r];
            }
        }
    }
}

// S-stage pipeline: A tiles of K-steps kt+1 .. kt+S-1 are in flight to LDS
// (S buffers of 32 KB) and the matching B tiles and parameters to registers
// (S slots) while step kt is computed, so a K-step's MFMA work (128 per
// wave) need not cover a full memory latency.  The K loop is unrolled by S so
// that every register slot and LDS buffer index is static; steps past the
// last group (the last round runs whole) re-load group G - 1 (valid
// addresses, never consumed), which keeps the load stream the same every step: 20 loads per step and wave
// (8 A direct-to-LDS, 4 B tiles, 4 scale words, 4 zero words).
//
// Split K (part != nullptr): workgroup (tile, blockIdx.y) covers groups
// [blockIdx.y * gsplit, +gsplit) and writes its fp32 partial tile to
// part[blockIdx.y][M][N]; k_splitk_reduce adds the splits in order.
template <int BITS, int GS, int S, int GMT, int NBW, int WV = 4, bool SC = false>
__global__ __launch_bounds__(64 * WV, 1) void k_gemm_w4p(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    _Float16* __restrict__ Y, float* __restrict__ part, const float* __restrict__ inv_s,
    int M, int N, int K, int gsplit, int xcd_rows) {
    using namespace w4;
    static_assert(GMT == 128 || GMT == 64 || GMT == 32 || GMT == 16, "16- to 128-row tiles");
    constexpr int FR = GMT / 16;                       // 16-row A fragments (and row groups per wave)
    constexpr int ABUFT = GMT * ROW_BYTES;             // one A buffer
    constexpr int TN = 16 * NBW * WV;                  // tile columns: NBW 16-column blocks per wave
    constexpr int FRL = 4 * FR / WV;                   // A row groups (4 rows) each wave loads
    // S x ABUFT of A buffers; with SC each wave's own copy of the K-step's 128
    // inv_s values follows, S x WV x 512 bytes
    extern __shared__ __attribute__((aligned(16))) unsigned char As[];
    unsigned char* const isb_base = As + S * ABUFT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, hq = lane >> 4;
    const int G = K / kGroup;
    const int g_begin = (int)blockIdx.y * gsplit;      // this workgroup's groups: [g_begin, g_begin + NGS)
    const int NGS = min(G - g_begin, gsplit);
    const int NB = (N + 15) / 16;
    const int nTn = (N + TN - 1) / TN, nTm = (M + GMT - 1) / GMT;
    const int nT = nTn * nTm;
    // XCD-aware tile order: workgroup ids go round-robin over the 8 XCDs, so
    // XCD x runs ids x, x + 8, ...  The tile grid is cut into xcd_rows row
    // blocks times 8 / xcd_rows column blocks, one per XCD, walked row-major,
    // so that an XCD's L2 serves the activation rows and weight columns its
    // tiles share (the host picks the cut; 0: tiles in id order)
    int tm, tn;
    if (xcd_rows > 0) {
        const int xcd = (int)blockIdx.x & 7, u = (int)blockIdx.x >> 3;
        const int R = nTm / xcd_rows, C = nTn / (8 / xcd_rows);      // tiles of one XCD's block
        tm = (xcd / (8 / xcd_rows)) * R + u / C;
        tn = (xcd % (8 / xcd_rows)) * C + u % C;
    } else {
        tm = (int)blockIdx.x / nTn;
        tn = (int)blockIdx.x % nTn;
    }
    const int m0 = tm * GMT, n0 = tn * TN;

    uint32_t a_off[FRL];
#pragma unroll
    for (int i = 0; i < FRL; ++i) {
        const int rg = wave * FRL + i;
        const int r = 4 * rg + (lane >> 4);
        const int kc = (lane & 15) ^ a_swz(r);
        const int grow = min(m0 + r, M - 1);
        a_off[i] = (uint32_t)grow * (uint32_t)K + 8u * kc;
    }
    uint32_t tbase[NBW];
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
        const int blk = min(n0 / 16 + wave * NBW + c, NB - 1);
        tbase[c] = (uint32_t)blk * (uint32_t)G;
    }
    const uint32_t psh = 16u * (uint32_t)(j & 1);      // the lane's half of a parameter word
    // scales / zeros [block][group][16]: kGroup / GS groups per tile; with
    // 64-wide groups a lane's quarter hq selects the tile's first or second
    const uint32_t pgrp = GS == 64 ? (uint32_t)(hq >> 1) : 0u;

    constexpr int WQ = BITS == 4 ? 4 : 3;              // words per lane slot
    // Every load is a buffer load whose per-lane byte offset is fixed for the
    // whole K loop and whose step-dependent part (group, tile) is wave-uniform
    // and goes in the scalar offset: no per-step vector address arithmetic.
    const uint32_t tiles_all = (uint32_t)NB * (uint32_t)G;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, tiles_all * 256u * WQ);
    // scales / zeros: kGroup / GS groups of 16 fp16 values per tile
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(scales, tiles_all * (32u * kGroup / GS));
    const __amdgpu_buffer_rsrc_t rze = make_rsrc(zeros, tiles_all * (32u * kGroup / GS));
    const __amdgpu_buffer_rsrc_t ris = make_rsrc(inv_s, SC ? (uint32_t)K * 4u : 0u);
    const uint32_t q_voff = 4u * WQ * (uint32_t)lane;
    const uint32_t p_voff = 2u * (pgrp * 16u + (uint32_t)(j & ~1));
    // loads per step and wave: A, B tiles, D and z words (and with SC the inv_s copy)
    constexpr int LPS = FRL + 3 * NBW + (SC ? 1 : 0);
    // the 128-row tiles spread the next step's loads over the substeps
    // (part p behind substep 4 p / NBW), the others issue them as one unit
    // before the compute: the folded-scale form waits for step kt + 1 inside
    // the substeps, and 64-row tiles measured 5 % slower spread (one wave per
    // SIMD: a wave stalled on the memory pipeline leaves its SIMD's MFMA unit
    // idle whichever substep it stalls in).  MI355X, M = 2048: 8 x 2 (14336 x
    // 4096) 231-236 -> 221-228 us; with the buffer loads' freed registers
    // also 4 x 7 (4096 x 14336, 1023 -> 1073-1079 TFLOP/s) and 8 x 3 at three
    // stages (4096 x 6144, 991 -> 1025-1031; four stages spill when spread)
    constexpr bool SPREAD = !SC && GMT == 128;
    static_assert(LPS * (S - 2) <= 63, "vmcnt counts to 63");
    struct BStage { uint32_t q[NBW][WQ]; uint32_t d[NBW], z[NBW]; };
    // part p (0..NBW-1) of step kt's loads: the A row groups i with
    // i * NBW / FR = p (direct to LDS buffer `slot`), B tile p of this wave and
    // its scale and zero words
    auto issue_part = [&](int kt, int slot, BStage& bs, int p) {
        const uint32_t g = (uint32_t)(g_begin + min(kt, NGS - 1));
        if constexpr (SC) {
            if (p == 0 && lane < 32)
                buffer_load_lds16(ris, isb_base + (slot * WV + wave) * 512, 16u * (uint32_t)lane, g * GK * 4u);
        }
#pragma unroll
        for (int i = 0; i < FRL; ++i) {
            if (i * NBW / FRL != p) continue;
            const int rg = wave * FRL + i;
            buffer_load_lds16(rx, As + slot * ABUFT + rg * 1024, 2u * a_off[i], g * GK * 2u);
        }
        const uint32_t tt = tbase[p] + g;
        if constexpr (BITS == 4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rq, q_voff, tt * 1024u, 0);
            bs.q[p][0] = v[0]; bs.q[p][1] = v[1]; bs.q[p][2] = v[2]; bs.q[p][3] = v[3];
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b96(rq, q_voff, tt * 768u, 0);
            bs.q[p][0] = v[0]; bs.q[p][1] = v[1]; bs.q[p][2] = v[2];
        }
        bs.d[p] = __builtin_amdgcn_raw_buffer_load_b32(rsc, p_voff, tt * (kGroup / GS) * 32u, 0);
        bs.z[p] = __builtin_amdgcn_raw_buffer_load_b32(rze, p_voff, tt * (kGroup / GS) * 32u, 0);
    };
    auto issue = [&](int kt, int slot, BStage& bs) {
#pragma unroll
        for (int p = 0; p < NBW; ++p) issue_part(kt, slot, bs, p);
    };

    float4_t acc[FR][NBW];
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int c = 0; c < NBW; ++c) acc[i][c] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // One K-step: four k32 substeps of NBW FR MFMAs.  The A fragments (FR LDS
    // reads) and B operands (NBW dequantized words) of substep s + 1 are produced while
    // the MFMAs of substep s run, so that neither LDS latency nor the
    // dequantization sits between two MFMA groups.
    // mid(s) runs after substep s's MFMAs have issued (they execute while it runs)
    auto compute = [&](const BStage& bs, const unsigned char* abuf, auto&& mid) {
        half2_t zz[NBW], zz16[NBW], dd[NBW];
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
            const _Float16 z = __builtin_bit_cast(_Float16, (unsigned short)(bs.z[c] >> psh));
            const _Float16 d = __builtin_bit_cast(_Float16, (unsigned short)(bs.d[c] >> psh));
            const _Float16 zb = (_Float16)1024.0f + z, zb16 = (_Float16)64.0f + z;
            zz[c] = (half2_t){zb, zb};
            zz16[c] = (half2_t){zb16, zb16};
            dd[c] = (half2_t){d, d};
        }
        auto read_a = [&](int s, half8_t* a) {
            const int kc = 4 * hq + s;
#pragma unroll
            for (int i = 0; i < FR; ++i) {
                const int r = 16 * i + j;
                a[i] = *reinterpret_cast<const half8_t*>(abuf + r * ROW_BYTES + ((kc ^ a_swz(r)) << 4));
            }
        };
        auto dequant = [&](int s, half8_t* b) {
#pragma unroll
            for (int c = 0; c < NBW; ++c) {
                if constexpr (BITS == 4) {
                    b[c] = dequant_scaled(bs.q[c][s], zz[c], zz16[c], dd[c]);
                } else {
                    // substep s takes the slot's code pairs 4s..4s+3
                    b[c] = dequant_scaled_int3(bs.q[c], s, zz[c], dd[c]);
                }
            }
        };
        if constexpr (NBW >= AWQ_GEMM_ILV) {
            // registers for one tile's B operand only: each tile is dequantized
            // just before its FR MFMAs, under the previous tile's
            half8_t a_cur[FR];
            read_a(0, a_cur);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                half8_t a_nxt[FR];
                if (s < 3) read_a(s + 1, a_nxt);
#pragma unroll
                for (int c = 0; c < NBW; ++c) {
                    half8_t b;
                    if constexpr (BITS == 4) b = dequant_scaled(bs.q[c][s], zz[c], zz16[c], dd[c]);
                    else b = dequant_scaled_int3(bs.q[c], s, zz[c], dd[c]);
#pragma unroll
                    for (int i = 0; i < FR; ++i)
                        acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a_cur[i], acc[i][c], 0, 0, 0);
                }
                mid(s);
                if (s < 3) {
#pragma unroll
                    for (int i = 0; i < FR; ++i) a_cur[i] = a_nxt[i];
                }
            }
            return;
        }
        half8_t a_cur[FR], b_cur[NBW];
        read_a(0, a_cur);
        dequant(0, b_cur);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8_t a_nxt[FR], b_nxt[NBW];
            if (s < 3) {
                read_a(s + 1, a_nxt);
                dequant(s + 1, b_nxt);
            }
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int c = 0; c < NBW; ++c)
                    acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b_cur[c], a_cur[i], acc[i][c], 0, 0, 0);
            mid(s);
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < FR; ++i) a_cur[i] = a_nxt[i];
#pragma unroll
                for (int c = 0; c < NBW; ++c) b_cur[c] = b_nxt[c];
            }
        }
    };

    // SC: x' = fp16(fp32(x) * inv_s) in place, over the A chunks this wave
    // loaded itself into buffer `slot` (lane l of row group rg wrote the 16
    // bytes at rg * 1024 + 16 l: row 4 rg + l / 16, global chunk
    // (l % 16) ^ a_swz(row)), once its loads of that step have landed; the other
    // waves see the scaled rows after the next barrier.  Each fp32 product is
    // rounded once (v_fma_mix_f32 of the fp16 value, inv_s and -0, which keeps
    // the sign of a zero product), then the pair to fp16 (v_cvt_pk_f16_f32,
    // round to nearest even).
    // chunks [i0, i0 + NC) of this wave's rows in buffer `slot`: every LDS read
    // first, then the products, then the writes, so the reads' latencies overlap
    auto scale_chunks = [&](int slot, int i0, auto nc) {
        constexpr int NC = decltype(nc)::value;
        const unsigned char* isb = isb_base + (slot * WV + wave) * 512;
        uint4 v[NC];
        float4 s0[NC], s1[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int rg = wave * FRL + i0 + c;
            const int kc = (lane & 15) ^ a_swz(4 * rg + (lane >> 4));
            v[c] = *reinterpret_cast<const uint4*>(As + slot * ABUFT + rg * 1024 + 16 * lane);
            s0[c] = *reinterpret_cast<const float4*>(isb + 32 * kc);
            s1[c] = *reinterpret_cast<const float4*>(isb + 32 * kc + 16);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float sv[8] = {s0[c].x, s0[c].y, s0[c].z, s0[c].w, s1[c].x, s1[c].y, s1[c].z, s1[c].w};
            const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float t0, t1;
                asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]"
                    : "=v"(t0) : "v"(w[e]), "v"(sv[2 * e]), "s"(0x80000000u));
                asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                    : "=v"(t1) : "v"(w[e]), "v"(sv[2 * e + 1]), "s"(0x80000000u));
                asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(o[e]) : "v"(t0), "v"(t1));
            }
            v[c] = make_uint4(o[0], o[1], o[2], o[3]);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c)
            *reinterpret_cast<uint4*>(As + slot * ABUFT + (wave * FRL + i0 + c) * 1024 + 16 * lane) = v[c];
    };
    // all FRL chunks of a step, in groups of SCG (the registers of SCG chunks live at once)
    constexpr int SCG0 = (GMT == 64 || NBW >= 7) ? 4 : (NBW <= 2 ? 1 : 2);
    constexpr int SCG = SCG0 < FRL ? SCG0 : FRL;
    static_assert(!SC || FRL % SCG == 0, "the chunk groups cover a step's chunks");
    auto scale_group = [&](int slot, int q) {
        // the wide 128-row tiles keep the scaling apart from the MFMA code
        // around it (interleaved, the registers of both spill); the others
        // leave it to the scheduler to interleave
        if constexpr (GMT == 128 && NBW >= 3) __builtin_amdgcn_sched_barrier(0);
        scale_chunks(slot, q * SCG, std::integral_constant<int, SCG>{});
    };

    // the loads of every step are issued as one unit in the same order, in the
    // prologue as in the loop, so that the compiler's per-register wait counts
    // agree on loop entry and along the back edge
    BStage bs[S];
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        issue(s, s, bs[s]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SC) {
        // step 0 is scaled here; step kt + 1 under the MFMAs of step kt
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS * (S - 2)));
#pragma unroll
        for (int q = 0; q < FRL / SCG; ++q) scale_group(0, q);
        __builtin_amdgcn_sched_barrier(0);
    }
    // NGS >= 1; a loop without an entry test keeps the compiler from sinking the
    // prologue's register loads behind one (out of the order above)
    int kt0 = 0;
    do {
#pragma unroll
        for (int st = 0; st < S; ++st) {
            const int kt = kt0 + st;
            // step kt has landed once at most the S - 2 later steps' loads are outstanding
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS * (S - 2)));
            // every wave's A(kt) is in LDS and its reads of A(kt-1) are done.  A
            // bare barrier: __syncthreads() is a release fence that would also
            // drain the later steps' direct-to-LDS loads (vmcnt(0))
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const int ls = (st + S - 1) % S;       // the slot step kt + S - 1 loads into
            if constexpr (!SPREAD) issue(kt + S - 1, ls, bs[ls]);
            __builtin_amdgcn_sched_barrier(0);
            // the last round may run past G: those steps keep the load stream
            // (and so the compiler's wait counts) uniform but compute nothing
            auto mid = [&](int s) {
                if constexpr (SPREAD) {
                    // part p of step kt + S - 1's loads right behind substep
                    // 4 p / NBW's MFMAs: the wave's wait for the shared memory
                    // pipeline then passes while those MFMAs execute
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int p = 0; p < NBW; ++p)
                        if (p * 4 / NBW == s) issue_part(kt + S - 1, ls, bs[ls], p);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (SC) {
                    // step kt + 1 has landed once at most the S - 2 steps after it
                    // are in flight.  8 x 2 tiles scale one chunk after each
                    // substep (their next-substep operands leave few registers);
                    // the others scale all of them after substep 1 (64-row
                    // tiles) or, where the next substep's operands fill the
                    // registers (8 x 3, 4 x 7), after the last substep
                    constexpr int NG = FRL / SCG;            // chunk groups per step
                    constexpr int S0 = NBW <= 2 ? 0 : (GMT == 64 ? 1 : 3);
                    if (s == S0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS * (S - 2)));
                    if constexpr (NG == 4) {
                        scale_group((st + 1) % S, s);
                    } else {
                        if (s == S0) {
#pragma unroll
                            for (int q = 0; q < NG; ++q) scale_group((st + 1) % S, q);
                        }
                    }
                }
            };
            if (kt < NGS) {
                compute(bs[st], As + st * ABUFT, mid);
            } else if constexpr (SPREAD) {
                issue(kt + S - 1, ls, bs[ls]);
            }
        }
        kt0 += S;
    } while (kt0 < NGS);

    if (part != nullptr) {
        float* prow0 = part + (size_t)blockIdx.y * M * N;
#pragma unroll
        for (int i = 0; i < FR; ++i) {
            const int m = m0 + 16 * i + j;
            if (m >= M) continue;
            float* prow = prow0 + (size_t)m * N;
#pragma unroll
            for (int c = 0; c < NBW; ++c) {
                const int n = n0 + wave * 16 * NBW + 16 * c + 4 * hq;
                if (n + 3 < N && ((N & 3) == 0)) {
                    *reinterpret_cast<float4_t*>(prow + n) = acc[i][c];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) prow[n + r] = acc[i][c][r];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FR; ++i) {
        const int m = m0 + 16 * i + j;
        if (m >= M) continue;
        _Float16* yrow = Y + (size_t)m * N;
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
            const int n = n0 + wave * 16 * NBW + 16 * c + 4 * hq;
            const half2_t lo = {(_Float16)acc[i][c][0], (_Float16)acc[i][c][1]};
            const half2_t hi = {(_Float16)acc[i][c][2], (_Float16)acc[i][c][3]};
            if (n + 3 < N && ((N & 3) == 0)) {
                *reinterpret_cast<uint2*>(yrow + n) = make_uint2(as_u32(lo), as_u32(hi));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) yrow[n + r] = (_Float16)acc[i][c][r];
            }
        }
    }
}

// Loss GEMM of the scale search: partials[z][tile] = sum over the tile's
// valid entries of (X . D_z^T)^2, X = X_cal fp16 [M][K], D_z = W - w_hat_z / s_z
// (one batch entry per alpha, b_batch_stride halves apart) in the tiled layout
// the search's error kernel writes: 16-row x 128-column tiles, each k32 step
// of a tile one contiguous 1 KB run in MFMA operand order (lane 16 hq + j:
// row j, columns 32 hq + 8 q .. + 7, the packed weights' order, which with
// a_swz reads X conflict-free; columns 32 q + 8 hq had half the LDS cycles in
// bank conflicts).  The prefill kernel's schedule with an
// fp16 B: X goes to LDS by direct-to-LDS loads (the swizzled 128-row buffers,
// S stages of one 128-wide K-step) and each wave streams its NBW D blocks
// straight into registers, four 1 KB wave loads per block and K-step (read
// row-major, D's 256-byte row pieces 8 KB apart cost ~13 % more time).  Rows
// past M or N load clamped rows (or the padding rows of the last block) and
// are left out of the sum, which is formed in a fixed order (lanes in fp32,
// then the waves in fp64).  Tiles are numbered column-major, so the XCD that
// runs eight consecutive tiles shares each D tile between the row tiles in
// its L2.  X may be batched too (a_batch_stride halves per batch entry).
//
// The block-output search of a gate/up pair (EPI_MLP_*) runs the same
// schedule with NBW = 2 over D rows [gate; up] (I rows each, I a multiple of
// 128): wave w takes gate block i0 / 16 + w and the up block of the same
// rows, so each lane holds g and u (or their quantization errors) for the
// same (token, channel) pairs, and the epilogue forms the block's
// intermediate activation there instead of summing squares:
//   EPI_MLP_REF: D = [Wg; Wu] itself: g, u and h = SiLU(g) u (fp32) to ref[3][M][I]
//   EPI_MLP_DH:  D = errors W - w_hat / s of the pair (dg = X Dg^T = g - g_q):
//                dh = fp16(SiLU(g - dg)(u - du) - h) to dh[z][M][I] (the change
//                of the intermediate activation)
enum { EPI_SQ = 0, EPI_MLP_REF = 1, EPI_MLP_DH = 2 };

struct LossOut {
    double* partials;          // EPI_SQ: [n_batch][tiles]
    float* ref;                // EPI_MLP_*: g, u, h fp32 [3][M][I]
    _Float16* dh;              // EPI_MLP_DH: [n_batch][M][I]
    int I;                     // EPI_MLP_*: intermediate channels (gate rows)
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <int S, int NBW, int WV, int EPI = EPI_SQ>
__global__ __launch_bounds__(64 * WV, 1) void k_loss_gemm_p(
    const _Float16* __restrict__ x, const _Float16* __restrict__ D, LossOut out,
    int M, int N, int K, long long a_batch_stride, long long b_batch_stride) {
    using namespace w4;
    static_assert(EPI == EPI_SQ || NBW == 2, "the MLP epilogues pair one gate and one up block");
    constexpr int GMT = 128, FR = GMT / 16;
    constexpr int ABUFT = GMT * ROW_BYTES;             // one X buffer (32 KB)
    // tile columns: D rows, or (MLP) intermediate channels (one gate and one up block per wave)
    constexpr int TN = EPI == EPI_SQ ? 16 * NBW * WV : 16 * WV;
    constexpr int FRL = 4 * FR / WV;                   // X row groups (4 rows) each wave loads
    constexpr int LPS = FRL + 4 * NBW;                 // loads per step and wave
    static_assert(LPS * (S - 2) <= 63, "vmcnt counts to 63");
    extern __shared__ __attribute__((aligned(16))) unsigned char As[];   // S x ABUFT
    __shared__ double wsum[WV];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, hq = lane >> 4;
    const int G = K / kGroup;
    const int NC = EPI == EPI_SQ ? N : out.I;          // tile columns span
    const int nTn = (NC + TN - 1) / TN, nTm = (M + GMT - 1) / GMT;
    const int nT = nTn * nTm;
    int t = blockIdx.x;
    if (nT % 8 == 0) t = (t % 8) * (nT / 8) + t / 8;
    const int m0 = (t % nTm) * GMT, n0 = (t / nTm) * TN;
    const _Float16* Dz = D + (size_t)blockIdx.y * (size_t)b_batch_stride;
    x += (size_t)blockIdx.y * (size_t)a_batch_stride;

    uint32_t a_off[FRL];
#pragma unroll
    for (int i = 0; i < FRL; ++i) {
        const int rg = wave * FRL + i;
        const int r = 4 * rg + (lane >> 4);
        const int kc = (lane & 15) ^ a_swz(r);
        a_off[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + 8u * kc;
    }
    // D block blk, group g: the tile at (blk G + g) 2048 halves, k32 step q at
    // + 512 q, lane 16 hq + j at + 8 lane (row j, columns 32 hq + 8 q ..)
    // buffer loads: per-lane byte offsets fixed for the K loop, the group's
    // offset (wave-uniform) in the scalar operand; D blocks past the rows the
    // layer has are clamped to its last block (read, never summed)
    const int NB16 = (N + 15) / 16;
    const int nbk = EPI == EPI_SQ ? NB16 : 2 * (out.I / 16);   // D blocks of one batch entry
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(Dz, (uint32_t)nbk * (uint32_t)G * 4096u);
    uint32_t bblk[NBW];                                // block offset of each D block, in tiles
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
        int blk;
        if constexpr (EPI == EPI_SQ) blk = min(n0 / 16 + wave * NBW + c, NB16 - 1);
        else blk = (c == 0 ? 0 : out.I / 16) + n0 / 16 + wave;   // gate block, then the same rows of up
        bblk[c] = (uint32_t)blk * (uint32_t)G;
    }
    const uint32_t d_voff = 16u * (uint32_t)lane;
    struct BStage { half8_t b[NBW][4]; };
    // part p (0..3) of step kt's loads: the X row groups i with i * 4 / FRL == p
    // (direct to LDS buffer `slot`) and the k32 step p of every D block
    auto issue_part = [&](int kt, int slot, BStage& bs, int p) {
        const uint32_t g = (uint32_t)min(kt, G - 1);
#pragma unroll
        for (int i = 0; i < FRL; ++i) {
            if (i * 4 / FRL != p) continue;
            const int rg = wave * FRL + i;
            buffer_load_lds16(rx, As + slot * ABUFT + rg * 1024, 2u * a_off[i], g * GK * 2u);
        }
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rd, d_voff, (bblk[c] + g) * 4096u + 1024u * p, 0);
            bs.b[c][p] = __builtin_bit_cast(half8_t, v);
        }
    };
    auto issue = [&](int kt, int slot, BStage& bs) {
#pragma unroll
        for (int p = 0; p < 4; ++p) issue_part(kt, slot, bs, p);
    };

    float4_t acc[FR][NBW];
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int c = 0; c < NBW; ++c) acc[i][c] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // mid(q) runs after substep q's MFMAs have issued
    auto compute = [&](const BStage& bs, const unsigned char* abuf, auto&& mid) {
        auto read_a = [&](int q, half8_t* a) {
            const int kc = 4 * hq + q;
#pragma unroll
            for (int i = 0; i < FR; ++i) {
                const int r = 16 * i + j;
                a[i] = *reinterpret_cast<const half8_t*>(abuf + r * ROW_BYTES + ((kc ^ a_swz(r)) << 4));
            }
        };
        half8_t a_cur[FR];
        read_a(0, a_cur);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            half8_t a_nxt[FR];
            if (q < 3) read_a(q + 1, a_nxt);
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int c = 0; c < NBW; ++c)
                    acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bs.b[c][q], a_cur[i], acc[i][c], 0, 0, 0);
            mid(q);
            if (q < 3) {
#pragma unroll
                for (int i = 0; i < FR; ++i) a_cur[i] = a_nxt[i];
            }
        }
    };

    BStage bs[S];
#pragma unroll
    for (int st = 0; st < S - 1; ++st) {
        __builtin_amdgcn_sched_barrier(0);
        issue(st, st, bs[st]);
    }
    __builtin_amdgcn_sched_barrier(0);
    int kt0 = 0;
    do {
#pragma unroll
        for (int st = 0; st < S; ++st) {
            const int kt = kt0 + st;
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS * (S - 2)));
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            // step kt + S - 1's loads, part q right behind substep q's MFMAs:
            // a wave's wait for the shared memory pipeline then passes while
            // those MFMAs execute (steps past G keep the load stream uniform)
            const int ls = (st + S - 1) % S;
            auto mid = [&](int q) {
                __builtin_amdgcn_sched_barrier(0);
                issue_part(kt + S - 1, ls, bs[ls], q);
                __builtin_amdgcn_sched_barrier(0);
            };
            if (kt < G) compute(bs[st], As + st * ABUFT, mid);
            else issue(kt + S - 1, ls, bs[ls]);
        }
        kt0 += S;
    } while (kt0 < G);

    if constexpr (EPI != EPI_SQ) {
        // lane 16 hq + j, fragment i: token m0 + 16 i + j, channels
        // n0 + 16 wave + 4 hq + r (r = 0..3); acc[i][0] is the gate's, acc[i][1] the up's
        const int I = out.I;
        const int col = n0 + 16 * wave + 4 * hq;
#pragma unroll
        for (int i = 0; i < FR; ++i) {
            const int m = m0 + 16 * i + j;
            if (m >= M) continue;
            const size_t e = (size_t)m * I + col;
            if constexpr (EPI == EPI_MLP_REF) {
                float4_t h;
#pragma unroll
                for (int r = 0; r < 4; ++r) h[r] = silu_f(acc[i][0][r]) * acc[i][1][r];
                *reinterpret_cast<float4_t*>(out.ref + e) = acc[i][0];
                *reinterpret_cast<float4_t*>(out.ref + (size_t)M * I + e) = acc[i][1];
                *reinterpret_cast<float4_t*>(out.ref + 2 * (size_t)M * I + e) = h;
            } else {
                const float4_t g0 = *reinterpret_cast<const float4_t*>(out.ref + e);
                const float4_t u0 = *reinterpret_cast<const float4_t*>(out.ref + (size_t)M * I + e);
                const float4_t h0 = *reinterpret_cast<const float4_t*>(out.ref + 2 * (size_t)M * I + e);
                half2_t dv[2];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // D = W - w_hat / s, so the quantized pair's outputs are g - dg and u - du
                    const float d = silu_f(g0[r] - acc[i][0][r]) * (u0[r] - acc[i][1][r]) - h0[r];
                    dv[r >> 1][r & 1] = (_Float16)d;
                }
                *reinterpret_cast<uint2*>(out.dh + (size_t)blockIdx.y * M * I + e) =
                    make_uint2(as_u32(dv[0]), as_u32(dv[1]));
            }
        }
        return;
    }
    // accumulator of lane 16 hq + j, block (i, c): X row m0 + 16 i + j, D row
    // n0 + 16 (wave NBW + c) + 4 hq + r
    float sq = 0.0f;
#pragma unroll
    for (int i = 0; i < FR; ++i) {
        const bool mv = m0 + 16 * i + j < M;
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
            const int n = n0 + wave * 16 * NBW + 16 * c + 4 * hq;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (mv && n + r < N) sq = __builtin_fmaf(acc[i][c][r], acc[i][c][r], sq);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
    if (lane == 0) wsum[wave] = (double)sq;
    __syncthreads();
    if (tid == 0) {
        double tot = wsum[0];
#pragma unroll
        for (int w = 1; w < WV; ++w) tot += wsum[w];
        out.partials[(size_t)blockIdx.y * nT + blockIdx.x] = tot;
    }
}

// y[i] = fp16(sum over s = 0 .. splits-1 of part[s][i]), in that order.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part,
                                                       _Float16* __restrict__ y, long long mn,
                                                       int splits) {
    const long long i0 = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i0 >= mn) return;
    if (i0 + 3 < mn && (mn & 3) == 0) {
        float4_t acc = *reinterpret_cast<const float4_t*>(part + i0);
        for (int s = 1; s < splits; ++s) {
            const float4_t v = *reinterpret_cast<const float4_t*>(part + (size_t)s * mn + i0);
            acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
        }
        const half2_t lo = {(_Float16)acc[0], (_Float16)acc[1]};
        const half2_t hi = {(_Float16)acc[2], (_Float16)acc[3]};
        *reinterpret_cast<uint2*>(y + i0) = make_uint2(as_u32(lo), as_u32(hi));
    } else {
        for (long long i = i0; i < i0 + 4 && i < mn; ++i) {
            float a = part[i];
            for (int s = 1; s < splits; ++s) a += part[(size_t)s * mn + i];
            y[i] = (_Float16)a;
        }
    }
}

constexpr int kGemmStages = 4;

// tile height of the pipelined kernel: the smallest of 16, 32 and 64 rows
// that holds M (a taller tile would spend its MFMAs and A reads on padding
// rows; MI355X, Llama-70B MLP shapes with split K, cold: M = 16 52-56 ->
// 34-35 us, M = 32 54 -> 43-44 us against 64-row tiles), else 128
int w4p_rows(int M) { return M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128; }

int w4p_tiles(int M, int N, int nbw = 4) {
    const int rows = w4p_rows(M);
    if (rows == 16) nbw = 1;                           // 64-column tiles (launch_w4p)
    else if (rows <= 64) nbw = 2;                      // 128-column tiles
    return ((N + 64 * nbw - 1) / (64 * nbw)) * ((M + rows - 1) / rows);
}

// The XCD cut of the pipelined kernel's tile grid (see k_gemm_w4p): with a
// row blocks and 8 / a column blocks, each XCD reads its activation rows once
// and its weight columns once, so the L2 misses are about (8 / a) x the
// activation bytes + a x the weight bytes; the a in {1, 2, 4, 8} that
// divides the grid and minimises that is taken (0 when the grid does not
// split into 8 equal blocks).  Example, M = 2048 (16 row tiles): 4096 x 14336
// (16.8 MB of activations, 29 MB of weights, 32 column tiles) a = 2,
// 14336 x 4096 (58.7 MB, 29 MB) a = 4.
int xcd_rows_for(int M, int N, int K, int bits, int gmt, int tn) {
    const int nTm = (M + gmt - 1) / gmt, nTn = (N + tn - 1) / tn;
    const double xb = 2.0 * M * K, wb = (double)N * K * bits / 8 + 4.0 * N * (K / kGroup);
    int best = 0;
    double best_cost = 0;
    for (const int a : {8, 4, 2, 1}) {
        if (nTm % a != 0 || nTn % (8 / a) != 0) continue;
        const double cost = (8 / a) * xb + a * wb;
        if (best == 0 || cost < best_cost) { best = a; best_cost = cost; }
    }
    return best;
}

template <int GMT, int NBW, int WV, bool SC>
int launch_w4p_rows_sc(const void* x, const void* qweight, const void* scales, const void* zeros,
                       void* y, float* part, const float* inv_s, int M, int N, int K, int bits,
                       int group_size, int splits, int gsplit, hipStream_t st) {
    // 64-row tiles with the folded scale keep a fifth stage, since each step
    // must land one step earlier to be scaled.  NBW = 7 spilled at four
    // stages before the buffer loads freed its address registers; with them
    // four measure 1-2.5 % faster than three (4096x14336, M = 2048)
    // 8 x 3 tiles with their loads spread over the substeps: three stages
    // (four spill)
    constexpr int S = (SC && GMT == 64) ? kGemmStages + 1
                    : (NBW == 3 && !SC) ? kGemmStages - 1 : kGemmStages;
    const int nT = ((N + 16 * NBW * WV - 1) / (16 * NBW * WV)) * ((M + GMT - 1) / GMT);
    const size_t lds = (size_t)S * GMT * w4::ROW_BYTES + (SC ? (size_t)S * WV * 512 : 0);
    auto kern = group_size == 64
                    ? (bits == 4 ? k_gemm_w4p<4, 64, S, GMT, NBW, WV, SC> : k_gemm_w4p<3, 64, S, GMT, NBW, WV, SC>)
                    : (bits == 4 ? k_gemm_w4p<4, 128, S, GMT, NBW, WV, SC> : k_gemm_w4p<3, 128, S, GMT, NBW, WV, SC>);
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(kern, dim3(nT, splits), dim3(64 * WV), lds, st, (const _Float16*)x,
                       (const uint32_t*)qweight, (const _Float16*)scales, (const _Float16*)zeros,
                       (_Float16*)y, part, inv_s, M, N, K, gsplit,
                       xcd_rows_for(M, N, K, bits, GMT, 16 * NBW * WV));
    return (int)hipGetLastError();
}

// inv_s (or NULL): the activation scale folded into the A tiles
template <int GMT, int NBW, int WV = 4>
int launch_w4p_rows(const void* x, const void* qweight, const void* scales, const void* zeros,
                    void* y, float* part, const float* inv_s, int M, int N, int K, int bits,
                    int group_size, int splits, int gsplit, hipStream_t st) {
    return inv_s ? launch_w4p_rows_sc<GMT, NBW, WV, true>(x, qweight, scales, zeros, y, part, inv_s, M, N,
                                                          K, bits, group_size, splits, gsplit, st)
                 : launch_w4p_rows_sc<GMT, NBW, WV, false>(x, qweight, scales, zeros, y, part, nullptr, M,
                                                           N, K, bits, group_size, splits, gsplit, st);
}

// nbw: the 128-row tile's width in 64-column units (4, 6 or 7; see
// gemm_tile_choice).  256 and 384 columns run as 8 waves of 2 or 3 16-column
// blocks (two waves per SIMD hide each other's waits: MI355X, M = 2048,
// 14336x4096 877-886 -> 890-919 TFLOP/s, 4096x6144 919-942 -> 960-986),
// 448 columns as 4 waves of 7 (8 waves cannot split it).  16-, 32- and
// 64-row tiles (batched decode) are narrower: 8 waves of 1 block (128
// columns, two waves per SIMD) at 32 and 64 rows, 4 waves of 1 block (64
// columns) at 16 rows, whose split K aims at two workgroups per CU
// (gemm_splits).  More tiles than 256-column ones means fewer splits.
// MI355X, cold weights, medians of runs alternated with 4 waves of 4 blocks
// (256 columns): Llama-70B MLP 8192x28672 / 28672x8192 at M = 32 40.1 / 39.0
// -> 36.2 / 36.9 us, M = 64 52.3 / 50.6 -> 49.2 / 49.4; Llama-7B 4096x4096,
// 11008x4096, 4096x11008 at M = 64 18.9, 23.9, 20.9 -> 13.2, 17.5, 17.7 us.
// At 16 rows, against 128-column tiles split for one workgroup per CU (which
// themselves took the 70B shapes from 33.1 / 32.7 to 32.6 / 32.3 us and the
// 7B ones from 12.6, 16.8, 13.9 to 9.6, 13.3, 12.3): 70B 33.0 / 32.8 -> 32.8
// / 31.3, 7B 9.5, 13.4, 12.3 -> 8.4, 13.3, 11.5 us.  Two workgroups per CU at
// 32 and 64 rows made the 7B shapes slower (11008x4096 at M = 32 14.6 ->
// 18.0 us).
int launch_w4p(const void* x, const void* qweight, const void* scales, const void* zeros, void* y,
               float* part, const float* inv_s, int M, int N, int K, int bits, int group_size,
               int splits, int gsplit, hipStream_t st, int nbw = 4) {
    switch (w4p_rows(M)) {
    case 16:
        return launch_w4p_rows<16, 1, 4>(x, qweight, scales, zeros, y, part, inv_s, M, N, K, bits, group_size,
                                         splits, gsplit, st);
    case 32:
        return launch_w4p_rows<32, 1, 8>(x, qweight, scales, zeros, y, part, inv_s, M, N, K, bits, group_size,
                                         splits, gsplit, st);
    case 64:
        return launch_w4p_rows<64, 1, 8>(x, qweight, scales, zeros, y, part, inv_s, M, N, K, bits, group_size,
                                         splits, gsplit, st);
    default:
        break;
    }
    if (nbw == 6)
        return launch_w4p_rows<128, 3, 8>(x, qweight, scales, zeros, y, part, inv_s, M, N, K, bits,
                                          group_size, splits, gsplit, st);
    if (nbw == 7)
        return launch_w4p_rows<128, 7>(x, qweight, scales, zeros, y, part, inv_s, M, N, K, bits,
                                       group_size, splits, gsplit, st);
    return launch_w4p_rows<128, 2, 8>(x, qweight, scales, zeros, y, part, inv_s, M, N, K, bits,
                                      group_size, splits, gsplit, st);
}

// The GEMM's kernel and tile for M > 64: 16-column blocks per wave (4, 6 or
// 7) of the pipelined one-workgroup-per-CU kernel, or 0 for the
// double-buffered kernel at two workgroups per CU (int4, 128-wide groups
// only).  A CU's time is taken as proportional to the tiles it runs times
// their width, so each candidate costs ceil(tiles / slots) * NBW; a round of
// the two-per-CU kernel (two 4-block tiles per CU, one's loads under the
// other's MFMAs) is priced at 7, below the 8 of two pipelined rounds.  The
// cheapest wins, ties going to the wider tile (fewer A reads from LDS per
// MFMA).  MI355X, M = 2048: 4096x14336 NBW 7 (512 tiles, two rounds) 881-892
// vs 828-839 TFLOP/s for the two-per-CU kernel (896 tiles) and 732-739 for
// NBW 4 (four rounds); 4096x6144 NBW 6 (256 tiles) 989-1015 vs 862 and 717;
// 14336x4096 NBW 4 (256 tiles) 943 vs NBW 6 775, NBW 7 670.  M <= 64
// (16- to 64-row tiles) takes the 128-column tiles of launch_w4p.
int gemm_tile_choice(int M, int N, int bits, int group_size, int cus) {
    if (w4p_rows(M) <= 64) return 4;
    int best = 4, best_cost = INT_MAX;
    for (const int nbw : {7, 6, 4}) {
        const int rounds = (w4p_tiles(M, N, nbw) + cus - 1) / cus;
        if (rounds * nbw < best_cost) { best = nbw; best_cost = rounds * nbw; }
    }
    if (bits == 4 && group_size == 128) {
        const int rounds2 = (w4p_tiles(M, N) + 2 * cus - 1) / (2 * cus);
        if (rounds2 * 7 < best_cost) best = 0;
    }
    return best;
}

}  // namespace

int gemm_splits(int M, int N, int K) {
    // split K only while the tiles leave at least half the workgroup slots
    // idle: one slot per CU, two for the 16-row tiles (4 waves of 64 columns
    // with a small footprint: two workgroups put two waves on each SIMD); each
    // split keeps >= 8 groups (two rounds of the 4-step pipeline), <= 16 splits
    const int nT = w4p_tiles(M, N);
    const int slots = device_cu_count() * (w4p_rows(M) == 16 ? 2 : 1);
    const int G = K / kGroup;
    int s = min(min(slots / nT, G / 8), 16);
    if (s < 2) return 1;
    const int gsplit = (G + s - 1) / s;
    return (G + gsplit - 1) / gsplit;                  // no empty split
}

size_t gemm_splitk_workspace_bytes(int M, int N, int K) {
    const int s = gemm_splits(M, N, K);
    return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

int launch_gemm_splitk(const void* x, const float* inv_s, const void* qweight, const void* scales,
                       const void* zeros, void* y, int M, int N, int K, int bits, int group_size,
                       void* workspace, hipStream_t st) {
    const int s = gemm_splits(M, N, K);
    if (s <= 1) return launch_gemm(x, inv_s, qweight, scales, zeros, y, M, N, K, bits, group_size, st);
    if ((unsigned long long)M * K >= (1ull << 31) || (unsigned long long)N * K / 8 >= (1ull << 31))
        return (int)hipErrorInvalidValue;
    const int G = K / kGroup;
    const int gsplit = (G + s - 1) / s;
    float* part = static_cast<float*>(workspace);
    int err = launch_w4p(x, qweight, scales, zeros, y, part, inv_s, M, N, K, bits, group_size, s, gsplit,
                         st);
    if (err) return err;
    const long long mn = (long long)M * N;
    const long long blocks = (mn / 4 + 1 + 255) / 256;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, st, part, (_Float16*)y,
                       mn, s);
    return (int)hipGetLastError();
}

int launch_gemm(const void* x, const float* inv_s, const void* qweight, const void* scales,
                const void* zeros, void* y, int M, int N, int K, int bits, int group_size,
                hipStream_t st) {
    // the kernel uses 32-bit element offsets into x and into the packed tiles
    if ((unsigned long long)M * K >= (1ull << 31) || (unsigned long long)N * K / 8 >= (1ull << 31))
        return (int)hipErrorInvalidValue;
    const int nT = ((N + w4::GN - 1) / w4::GN) * ((M + w4::GM - 1) / w4::GM);
    int nbw = gemm_tile_choice(M, N, bits, group_size, device_cu_count());
    // the folded activation scale lives in the pipelined kernel only
    if (nbw == 0 && inv_s != nullptr) nbw = 4;
    if (nbw > 0) {
        return launch_w4p(x, qweight, scales, zeros, y, nullptr, inv_s, M, N, K, bits, group_size, 1,
                          K / kGroup, st, nbw);
    } else {
        hipLaunchKernelGGL(k_gemm_w4, dim3(nT), dim3(256), 0, st, (const _Float16*)x,
                           (const uint32_t*)qweight, (const _Float16*)scales, (const _Float16*)zeros,
                           (_Float16*)y, M, N, K);
    }
    return (int)hipGetLastError();
}

// the loss GEMM's form: 3 stages, 8 waves of 2 D blocks (128 x 256 tiles);
// MI355X, 4096 x 4096, T = 512, 20 alphas, whole search over three runs: 0.71 ms,
// 4 stages 0.72 ms, 4 waves of 4 blocks 0.73-0.74 ms (2 or 3 stages); the
// 128 x 128 register-staged kernel it replaced (row-major D) 0.79-0.81 ms
constexpr int kLossS = 3, kLossNBW = 2, kLossWV = 8;
constexpr int kLossTN = 16 * kLossNBW * kLossWV;     // D rows per tile

size_t loss_gemm_tiles(int T, int N) {
    return (size_t)((N + kLossTN - 1) / kLossTN) * (size_t)((T + 127) / 128);
}

namespace {
template <int EPI>
int launch_loss_kernel(const void* X, long long a_stride, const void* D, long long d_stride, int T,
                       int N, int K, int n_batch, const LossOut& out, hipStream_t st) {
    // the kernel addresses one batch entry of D and of X with 32-bit byte offsets
    const size_t d_rows = EPI == EPI_SQ ? (size_t)(N + 15) / 16 * 16 : 2 * (size_t)out.I;
    if (d_rows * (size_t)K * 2 >= (1ull << 32) || (size_t)T * (size_t)K * 2 >= (1ull << 32))
        return (int)hipErrorInvalidValue;
    auto kern = k_loss_gemm_p<kLossS, kLossNBW, kLossWV, EPI>;
    const size_t lds = (size_t)kLossS * 128 * w4::ROW_BYTES;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    const size_t tiles = EPI == EPI_SQ ? loss_gemm_tiles(T, N)
                                       : (size_t)(out.I / (16 * kLossWV)) * (size_t)((T + 127) / 128);
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles, n_batch), dim3(64 * kLossWV), lds, st,
                       (const _Float16*)X, (const _Float16*)D, out, T, N, K, a_stride, d_stride);
    return (int)hipGetLastError();
}
}  // namespace

int launch_loss_gemm(const void* X, long long a_stride, const void* D, long long d_stride, int T,
                     int N, int K, int n_batch, double* partials, hipStream_t st) {
    LossOut out{};
    out.partials = partials;
    return launch_loss_kernel<EPI_SQ>(X, a_stride, D, d_stride, T, N, K, n_batch, out, st);
}

int launch_mlp_gemm(const void* X, const void* D, long long d_stride, int T, int I, int K,
                    int n_batch, bool ref, float* gu_ref, _Float16* dh, hipStream_t st) {
    LossOut out{};
    out.ref = gu_ref;
    out.dh = dh;
    out.I = I;
    return ref ? launch_loss_kernel<EPI_MLP_REF>(X, 0, D, d_stride, T, 2 * I, K, n_batch, out, st)
               : launch_loss_kernel<EPI_MLP_DH>(X, 0, D, d_stride, T, 2 * I, K, n_batch, out, st);
}

}  // namespace awq
