// Internal declarations shared by the HIP sources of libawq (gfx950 only).
//
// The whole library is compiled with -ffp-contract=off: every fused
// multiply-add in these sources is written out with __builtin_fmaf, so the
// quantizer's fp32 arithmetic is exactly the IEEE sequence it states.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <initializer_list>

#include "../../include/awq.h"

namespace awq {

constexpr int kGroup = 128;          // codes per packed tile, and the default q_group_size
constexpr int kWave = 64;            // CDNA wavefront width

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint16_t half_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ _Float16 bits_half(uint16_t b) { return __builtin_bit_cast(_Float16, b); }

// Largest fp16 value <= d, for positive finite d >= 2^-24: convert to nearest
// (v_cvt_f16_f32, round-half-even, fp16 denormals kept) and step one fp16
// down when that rounded up.  +inf from overflow steps down to 65504.
__device__ __forceinline__ uint16_t f16_bits_round_down(float d) {
    _Float16 h = (_Float16)d;
    uint16_t b = half_bits(h);
    if ((float)h > d) b = (uint16_t)(b - 1);
    return b;
}

// (x & mask) | bits in one VALU instruction.  The compiler otherwise often
// emits a separate AND and OR for the int4 -> fp16 exponent trick.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask), "v"(bits));
    return r;
}

// The fp16 pair (1024 + q[2t], 1024 + q[2t+1]) of a packed int4 word: the two
// codes sit at bits 4t..4t+3 and 16+4t..19+4t, and OR 0x6400 makes each the
// low mantissa bits of an fp16 number with exponent 2^10.
__device__ __forceinline__ uint32_t int4_pair_bits(uint32_t w, int t) {
    return and_or(w >> (4 * t), 0x000F000Fu, 0x64006400u);
}

// The fp16 pair (1024 + c[2P], 1024 + c[2P+1]) of a packed int3 lane slot (3
// words, codes c[0..31]): pairs P < 15 sit at bits 3t..3t+2 / 16+3t..18+3t of
// word P / 5 (t = P % 5), so one shift and one AND-OR give them; bit b of
// c[30] and c[31] is bit 15 / 31 of word b.  P is a compile-time constant.
__device__ __forceinline__ uint32_t int3_pair_bits(const uint32_t* w, int P) {
    if (P < 15) return and_or(w[P / 5] >> (3 * (P % 5)), 0x00070007u, 0x64006400u);
    uint32_t r = and_or(w[0] >> 15, 0x00010001u, 0x64006400u);
    r = and_or(w[1] >> 14, 0x00020002u, r);
    return and_or(w[2] >> 13, 0x00040004u, r);
}

// The four fp16 pairs of a packed int4 word with one shift.  Pairs t = 0, 2
// (code nibbles at bits 0..3 / 16..19 of w and of w >> 8) use exponent 2^10,
// giving 1024 + q; pairs t = 1, 3 (nibbles at bits 4..7 / 20..23) are OR-ed
// in place under 0x5400 = 64.0, whose mantissa step is 1/16, giving 64 + q.
// Subtracting 1024 + z resp. 64 + z leaves q - z exactly in every lane.
__device__ __forceinline__ void int4_word_pairs(uint32_t w, uint32_t p[4]) {
    const uint32_t w8 = w >> 8;
    p[0] = and_or(w, 0x000F000Fu, 0x64006400u);
    p[1] = and_or(w, 0x00F000F0u, 0x54005400u);
    p[2] = and_or(w8, 0x000F000Fu, 0x64006400u);
    p[3] = and_or(w8, 0x00F000F0u, 0x54005400u);
}

// Group parameters of one quantization group from its (already reduced)
// minimum and maximum of v = w * s.  Every result is the one IEEE fp32
// arithmetic gives (correctly rounded division, round-half-even rint); the
// divisions are replaced by multiplications where the result provably
// cannot differ, with the division kept for the rare lanes near a rounding
// boundary.
struct GroupParams {
    float delta;       // D as fp32 (exactly the stored fp16 value)
    float zero;        // integer zero point z, as fp32
    float rd;          // 1 / D within 1 fp32 ulp (v_rcp_f32)
    uint16_t dbits;    // the stored fp16 scale
};

// f16_bits_round_down(fp32(num / DEN)) for positive finite num.  m = num *
// fp32(1 / DEN) is within 2^-23 relative (under 2 ulp) of the exact quotient
// and its fp32 rounding within 2.5 ulp, so when m is in fp16's normal range
// and more than 8 fp32 ulps from every fp16 value (the 13 bits below fp16's
// precision not within 8 of 0 or 2^13; a binade edge at most doubles the
// distance in m's ulps) both round down to the same fp16.  Lanes outside that
// (rare: one ballot) divide.
template <int DEN>
__device__ __forceinline__ uint16_t f16_down_quotient(float num) {
    float m = num * (1.0f / (float)DEN);
    const uint32_t low = __builtin_bit_cast(uint32_t, m) & 0x1FFFu;
    const bool slow = !(m >= 0x1p-14f && m < 0x1p15f) || low < 8u || low > 0x1FF8u;
    if (__builtin_amdgcn_ballot_w64(slow)) {
        if (slow) {
            // an opaque copy keeps the division inside this branch (the
            // compiler otherwise computes it on every lane and selects)
            float n = num;
            asm volatile("" : "+v"(n));
            m = n / (float)DEN;
        }
    }
    return f16_bits_round_down(m);
}

// Scale and zero point of a group from its min and max (fp32, IEEE).
// zero_point (asymmetric): range widened to contain 0, D = largest fp16 <=
// max(hi - lo, 1e-5) / Q, z = clamp(rint(-lo / D), 0, Q).  Symmetric
// (zero_point false, "Quantizing a model with AutoAWQ"): D = largest fp16 <=
// max(max |v|, 1e-5) / (2^(b-1) - 1) and the fixed z = 2^(b-1), so codes
// rint(v / D) + z keep the same unsigned storage and (q - z) * D dequant.
// z is decided in fixed point as the codes are (quant_codes_b2): 0 <= -lo / D
// <= Q / (1 - 2^-10) < 16.4, so t = -lo * (1/D) + 128.5 + 3 * 2^-16 lies in
// [128, 256) with its integer part minus 128 in bits 16..22; a fraction of at
// least 6 * 2^-16 decides rint(-lo / D) (the argument of quant_codes_b2).
template <int Q, bool ZP>
__device__ __forceinline__ GroupParams group_params(float vmin, float vmax) {
    GroupParams p;
    if constexpr (ZP) {
        const float lo = fminf(vmin, 0.0f);
        const float hi = fmaxf(vmax, 0.0f);
        const float span = fmaxf(hi - lo, 1e-5f);
        p.dbits = f16_down_quotient<Q>(span);
        p.delta = (float)bits_half(p.dbits);
        p.rd = __builtin_amdgcn_rcpf(p.delta);
        const uint32_t T = __builtin_bit_cast(uint32_t, __builtin_fmaf(-lo, p.rd, 128.5f + 0x3p-16f));
        const bool near = (T & 0xFFFFu) <= 5u;
        float z = (float)((T >> 16) & 0xFFu);
        if (__builtin_amdgcn_ballot_w64(near)) {
            if (near) z = __builtin_rintf(-lo / p.delta);
        }
        p.zero = fminf(fmaxf(z, 0.0f), (float)Q);
    } else {
        const float amax = fmaxf(fmaxf(-vmin, vmax), 1e-5f);   // max |v|: negation is exact
        p.dbits = f16_down_quotient<(Q - 1) / 2>(amax);
        p.delta = (float)bits_half(p.dbits);
        p.rd = __builtin_amdgcn_rcpf(p.delta);
        p.zero = (float)((Q + 1) / 2);
    }
    return p;
}

template <int Q>
__device__ __forceinline__ uint32_t quant_code(float v, const GroupParams& p) {
    float c = __builtin_rintf(v / p.delta) + p.zero;
    c = fminf(fmaxf(c, 0.0f), (float)Q);
    return (uint32_t)c;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_void_t;

// s_waitcnt immediate (gfx9): wait until at most n vector-memory ops are
// outstanding, no wait on lgkm/exp counters
constexpr unsigned vmcnt_imm(unsigned n) { return (n & 15u) | ((n >> 4) << 14) | (7u << 4) | (15u << 8); }

// The codes of NV values of one group, each equal to quant_code's, in
// bits 16..19 of T[i] (bits 20..23 zero), decided without a division or a
// rounding instruction.  One fma forms t = v * (1/D) + (z + 128.5 + 3 * 2^-16),
// clamped to [128.25, 128.5 + Q]; there fp32 values are multiples of 2^-16,
// so the float's bits 16..22 hold the integer part of t - 128 and bits 0..15
// its fraction F.  t is within 2^-17 (the fma's rounding) + 16.4 * 2^-23 (1/D
// from v_rcp_f32, within 1 ulp; |v / D| <= 16.4) < 0.63 * 2^-16 of
// v / D + z + 1/2 + 3 * 2^-16, so
// F >= 6 * 2^-16 puts v / D + z more than 2.3 * 2^-16 above and 1/2 - 6 * 2^-16
// below a half-integer: its integer part is then rint(v / D) + z for the
// exact quotient and for its rounding to fp32 (within 2^-20) alike, with no
// tie.  The clamp bounds give F = 1/4 and 1/2 for codes 0 and Q, which
// clamping the rounded quotient also gives.  Lanes with some F <= 5 * 2^-16
// (rare: one ballot) take quant_code's division for all their values.
template <int Q, int NV>
__device__ __forceinline__ void quant_codes_b2(const float* v, const GroupParams& p, uint32_t* T) {
    const float rd = p.rd;
    const float zb = p.zero + (128.5f + 0x3p-16f);   // exact: z <= 15
    uint32_t fmin = 0xFFFFu;                          // least fraction F, in units of 2^-16
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(v[i], rd, zb), 128.25f, 128.5f + Q);
        T[i] = __builtin_bit_cast(uint32_t, t);
        fmin = min(fmin, T[i] & 0xFFFFu);
    }
    const bool near = fmin <= 5u;
    if (__builtin_amdgcn_ballot_w64(near)) {
        if (near) {
#pragma unroll
            for (int i = 0; i < NV; ++i) T[i] = quant_code<Q>(v[i], p) << 16;
        }
    }
}

// Codes 2i and 2i + 1 (bits 16..19 of T[2i], T[2i + 1]) as one magic pair:
// bits 0..3 and 16..19.
__device__ __forceinline__ uint32_t code_pair(const uint32_t* T, int i) {
    return ((T[2 * i] >> 16) & 0xFFu) | (T[2 * i + 1] & 0x00FF0000u);
}

// ---------------------------------------------------------------------------
// host-side launchers (each .hip file owns its kernels); they return 0 or a
// hipError_t value.  Arguments have been validated by the C ABI layer.
// ---------------------------------------------------------------------------
int launch_quantize_pack(const void* W, const float* s, int N, int K, int bits, int group_size,
                         int zero_point, void* qweight, void* scales, void* zeros, hipStream_t st);
int launch_scale_activations(const void* x, const float* s, void* x_out, int M, int K,
                             hipStream_t st);
int launch_dequantize(const void* qweight, const void* scales, const void* zeros, void* W_hat, int N,
                      int K, int bits, int group_size, hipStream_t st);
// compute units of the current device
int device_cu_count();

// decode product; inv_s (or NULL) folds the activation scale into the x
// load; qweight2 (or NULL) makes it the fused gate/up pair (gate = the first
// layer, up = the second, y = SiLU(gate) * up)
int launch_gemv(const void* x, const float* inv_s, const void* qweight, const void* scales,
                const void* zeros, const void* qweight2, const void* scales2, const void* zeros2,
                void* y, int M, int N, int K, int bits, int group_size, hipStream_t st);
// prefill product; inv_s (or NULL) folds the activation scale into the A tiles
int launch_gemm(const void* x, const float* inv_s, const void* qweight, const void* scales,
                const void* zeros, void* y, int M, int N, int K, int bits, int group_size,
                hipStream_t st);
// split-K prefill: number of K splits for this shape on the current device
// (1: no split, no workspace) and the fp32 partial workspace it needs
int gemm_splits(int M, int N, int K);
size_t gemm_splitk_workspace_bytes(int M, int N, int K);
int launch_gemm_splitk(const void* x, const float* inv_s, const void* qweight, const void* scales,
                       const void* zeros, void* y, int M, int N, int K, int bits, int group_size,
                       void* workspace, hipStream_t st);
// fused: the workspace of the fused loss kernel (no D buffer), else the default
size_t search_workspace_bytes(int T, int N, int K, int n_alpha, bool fused);
size_t loss_gemm_tiles(int T, int N);
// rows of one alpha's D in the loss GEMM's tiled layout (N rounded up to 16)
inline size_t loss_rows(int N) { return (size_t)(N + 15) / 16 * 16; }
// D: n_batch entries of loss_rows(N) x K fp16 in that layout (written by the
// search's error kernel)
// X batched by a_stride halves and D by d_stride halves per batch entry
int launch_loss_gemm(const void* X, long long a_stride, const void* D, long long d_stride, int T,
                     int N, int K, int n_batch, double* partials, hipStream_t st);
// the block-output search of a gate/up pair: D = [gate; up] rows (I each, I a
// multiple of 128) in the loss GEMM's tiled layout, d_stride halves per batch
// entry.  ref: D holds the weights themselves; writes g, u, h = SiLU(g) u
// (fp32 [3][T][I]) to gu_ref.  Otherwise D holds their quantization errors and
// the change of h, fp16 [n_batch][T][I], goes to dh.
int launch_mlp_gemm(const void* X, const void* D, long long d_stride, int T, int I, int K,
                    int n_batch, bool ref, float* gu_ref, _Float16* dh, hipStream_t st);
// layers searched together (shared input): at most this many
constexpr int kMaxSearchLayers = 8;
// Ws / Ns: host arrays of n_layers device weight pointers and row counts;
// the layers' rows in order form the N = sum Ns rows of the search
// the gate/up scale searched on the MLP block's output (Wd [K_out][I] kept)
size_t search_mlp_workspace_bytes(int T, int K, int I, int K_out, int n_alpha);
int launch_search_mlp(const void* Wg, const void* Wu, const void* Wd, int K_out, const void* X_cal, int T,
                      int K, int I, const float* alphas, int n_alpha, int bits, int group_size,
                      int zero_point, float* s_out, float* loss_out, int* best_out, void* workspace,
                      hipStream_t st);
int launch_search(const void* const* Ws, const int* Ns, int n_layers, const void* X_cal, int T, int K,
                  const float* alphas, int n_alpha, int bits, int group_size, int zero_point,
                  float* s_out, float* loss_out, int* best_out, void* workspace, bool fused,
                  hipStream_t st);

}  // namespace awq
