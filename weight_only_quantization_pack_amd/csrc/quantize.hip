// Group quantization + packing (format 3) and the activation-side divide.
//
// What is computed: round-to-nearest quantization of W*diag(s) in groups of
// 128 (or 64) input channels, with an fp16 scale and an integer zero point
// per group, asymmetric or symmetric ("Quantizing a model with AutoAWQ":
// w_bit, q_group_size, zero_point; llm-awq README "Usage" step 3, real INT4
// weights).
//
// Layout of the work: one wavefront per packed tile (16-row block b,
// group g).  Lane slot s = 16h + j quantizes the 32 codes of row 16b + j in
// quarter h of the group (four 16-byte loads of W), the group's min/max is
// met across the four lanes of that row (xor-shuffles 16 and 32), and the
// wave writes its tile as one contiguous 1 KB store (768 B for bits 3) in
// the packed slot order, so the decode and prefill kernels can read a
// tile with one contiguous wave load.  The group scales and zeros go to the
// same tile order ([block][g][16]).  Rows past N are written as zeros.
// The kernel is HBM-bound (offline).
#include "awq_internal.h"

namespace awq {
namespace {

__device__ __forceinline__ void unpack8(const uint4& raw, float* f) {
    const _Float16* h = reinterpret_cast<const _Float16*>(&raw);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}

// One wave per tile; BITS selects 4 words (int4) or 3 words (int3) per slot.
// GS = 128: one group per tile; GS = 64: two (quarters 0-1 and 2-3 of a row).
template <int BITS, bool ZP, int GS>
__global__ __launch_bounds__(256) void k_quantize_pack(
    const _Float16* __restrict__ W, const float* __restrict__ s, int N, int K,
    long long n_tiles, uint32_t* __restrict__ qweight, uint16_t* __restrict__ scales,
    uint16_t* __restrict__ zeros) {
    constexpr int Q = (1 << BITS) - 1;
    constexpr int WQ = BITS == 4 ? 4 : 3;
    const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;                      // whole wave
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, h = lane >> 4;
    const int G = K / kGroup;
    const int b = (int)(tile / G), g = (int)(tile % G);
    const int n = 16 * b + j;
    const bool valid = n < N;
    const int k0 = kGroup * g + 32 * h;
    float v[32];
    if (valid) {
        const uint4* src = reinterpret_cast<const uint4*>(W + (size_t)n * K + k0);
#pragma unroll
        for (int c = 0; c < 4; ++c) unpack8(src[c], v + 8 * c);
        if (s != nullptr) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float4 sc = *reinterpret_cast<const float4*>(s + k0 + 4 * c);
                v[4 * c] *= sc.x; v[4 * c + 1] *= sc.y; v[4 * c + 2] *= sc.z; v[4 * c + 3] *= sc.w;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
    // the four quarters of row j sit in lanes j, j+16, j+32, j+48; a 64-group
    // is quarters {0,1} or {2,3}
    mn = fminf(mn, __shfl_xor(mn, 16)); mx = fmaxf(mx, __shfl_xor(mx, 16));
    if constexpr (GS == 128) {
        mn = fminf(mn, __shfl_xor(mn, 32)); mx = fmaxf(mx, __shfl_xor(mx, 32));
    }
    const GroupParams p = group_params<Q, ZP>(mn, mx);

    uint32_t T[32];
    quant_codes_b2<Q, 32>(v, p, T);                   // = quant_code of each value, << 16
    uint32_t out[WQ];
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t word = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) word |= code_pair(T, 4 * i + t) << (4 * t);
            out[i] = word;
        }
    } else {
        // pair P < 15 at bits 3t / 16 + 3t of word P / 5; bit b of codes 30 and
        // 31 at bits 15 and 31 of word b
        out[0] = out[1] = out[2] = 0;
#pragma unroll
        for (int P = 0; P < 15; ++P) out[P / 5] |= code_pair(T, P) << (3 * (P % 5));
        const uint32_t c30 = T[30] >> 16, c31 = T[31] >> 16;
#pragma unroll
        for (int b = 0; b < 3; ++b) out[b] |= (((c30 >> b) & 1u) << 15) | (((c31 >> b) & 1u) << 31);
    }
    uint32_t* dst = qweight + ((size_t)tile * 64 + lane) * WQ;
    if constexpr (BITS == 4) {
        *reinterpret_cast<uint4*>(dst) = valid ? make_uint4(out[0], out[1], out[2], out[3])
                                               : make_uint4(0, 0, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < 3; ++i) dst[i] = valid ? out[i] : 0u;
    }
    if (GS == 128 ? h == 0 : (h & 1) == 0) {  // tiled: [block][group][row in block]
        const size_t pidx = (GS == 128 ? (size_t)tile : 2 * (size_t)tile + (h >> 1)) * 16 + j;
        scales[pidx] = valid ? p.dbits : (uint16_t)0;
        zeros[pidx] = valid ? half_bits((_Float16)p.zero) : (uint16_t)0;
    }
}

// x_out[m][k] = fp16_rne(fp32(x[m][k]) / s[k]); 8 elements per lane.
__global__ __launch_bounds__(256) void k_scale_activations(
    const uint4* __restrict__ x, const float* __restrict__ s, uint4* __restrict__ x_out, int K,
    long long n_chunks) {
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_chunks) return;
    const int k0 = (int)(t % (K / 8)) * 8;
    float v[8];
    unpack8(x[t], v);
    uint4 out;
    _Float16* h = reinterpret_cast<_Float16*>(&out);
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)(v[i] / s[k0 + i]);
    x_out[t] = out;
}

// Fake quantization (llm-awq README "Usage" step 2, --q_backend fake): the
// packed layer back to fp16 w_hat = fp16_rne((q - z) * D), the exact product
// of a small integer and an fp16 value rounded once.  One wave per tile, lane
// (row j, quarter h) writes the 32 values of its slot with four 16-byte stores.
template <int BITS, int GS>
__global__ __launch_bounds__(256) void k_dequantize(const uint32_t* __restrict__ qweight,
                                                   const _Float16* __restrict__ scales,
                                                   const _Float16* __restrict__ zeros,
                                                   _Float16* __restrict__ W_hat, int N, int K,
                                                   long long n_tiles) {
    constexpr int WQ = BITS == 4 ? 4 : 3;
    const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, h = lane >> 4;
    const int G = K / kGroup;
    const int b = (int)(tile / G), g = (int)(tile % G);
    const int n = 16 * b + j;
    if (n >= N) return;                               // padding rows: nothing to write
    const uint32_t* src = qweight + ((size_t)tile * 64 + lane) * WQ;
    uint32_t w[WQ];
#pragma unroll
    for (int i = 0; i < WQ; ++i) w[i] = src[i];
    const size_t pidx = (GS == 128 ? (size_t)tile : 2 * (size_t)tile + (h >> 1)) * 16 + j;
    const float d = (float)scales[pidx], z = (float)zeros[pidx];
    uint32_t c[32];
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 32; ++i) c[i] = (w[i / 8] >> (4 * ((i % 8) / 2) + 16 * (i % 2))) & 15u;
    } else {
#pragma unroll
        for (int P = 0; P < 15; ++P) {
            c[2 * P] = (w[P / 5] >> (3 * (P % 5))) & 7u;
            c[2 * P + 1] = (w[P / 5] >> (16 + 3 * (P % 5))) & 7u;
        }
        c[30] = ((w[0] >> 15) & 1u) | ((w[1] >> 14) & 2u) | ((w[2] >> 13) & 4u);
        c[31] = ((w[0] >> 31) & 1u) | ((w[1] >> 30) & 2u) | ((w[2] >> 29) & 4u);
    }
    uint4 out[4];
    _Float16* o = reinterpret_cast<_Float16*>(out);
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] = (_Float16)(((float)c[i] - z) * d);
    uint4* dst = reinterpret_cast<uint4*>(W_hat + (size_t)n * K + kGroup * g + 32 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = out[i];
}

}  // namespace

template <int GS>
static auto pick_quantize(int bits, int zero_point) {
    return bits == 4 ? (zero_point ? k_quantize_pack<4, true, GS> : k_quantize_pack<4, false, GS>)
                     : (zero_point ? k_quantize_pack<3, true, GS> : k_quantize_pack<3, false, GS>);
}

int launch_quantize_pack(const void* W, const float* s, int N, int K, int bits, int group_size,
                         int zero_point, void* qweight, void* scales, void* zeros, hipStream_t st) {
    const long long n_tiles = (long long)((N + 15) / 16) * (K / kGroup);
    const long long grid = (n_tiles + 3) / 4;
    auto kern = group_size == 64 ? pick_quantize<64>(bits, zero_point) : pick_quantize<128>(bits, zero_point);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const _Float16*)W, s, N, K,
                       n_tiles, (uint32_t*)qweight, (uint16_t*)scales, (uint16_t*)zeros);
    return (int)hipGetLastError();
}

int launch_scale_activations(const void* x, const float* s, void* x_out, int M, int K,
                             hipStream_t st) {
    const long long n_chunks = (long long)M * K / 8;
    const int block = 256;
    const long long grid = (n_chunks + block - 1) / block;
    hipLaunchKernelGGL(k_scale_activations, dim3((unsigned)grid), dim3(block), 0, st,
                       (const uint4*)x, s, (uint4*)x_out, K, n_chunks);
    return (int)hipGetLastError();
}

int launch_dequantize(const void* qweight, const void* scales, const void* zeros, void* W_hat, int N,
                      int K, int bits, int group_size, hipStream_t st) {
    const long long n_tiles = (long long)((N + 15) / 16) * (K / kGroup);
    const long long grid = (n_tiles + 3) / 4;
    auto kern = group_size == 64 ? (bits == 4 ? k_dequantize<4, 64> : k_dequantize<3, 64>)
                                 : (bits == 4 ? k_dequantize<4, 128> : k_dequantize<3, 128>);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint32_t*)qweight,
                       (const _Float16*)scales, (const _Float16*)zeros, (_Float16*)W_hat, N, K, n_tiles);
    return (int)hipGetLastError();
}

}  // namespace awq
