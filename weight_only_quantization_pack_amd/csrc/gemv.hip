// Decode-stage W4A16 / W3A16 product for 1 <= M <= 16 rows of activations
// (the decode kernel of the llm-awq README feature list):
//   y[m][n] = sum_g D[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// Bandwidth-bound: every packed weight byte is read once from HBM.  One
// wavefront owns one output row n at a time; its lanes stride over the row
// in 16-byte chunks (32 int4 codes, all inside one group), so each wave load
// instruction reads 1 KB of contiguous HBM.  Per chunk the codes are
// unpacked in registers with the fp16 exponent trick (OR 0x6400 turns a
// 4-bit code q into the fp16 value 1024 + q), the zero is removed exactly
// in fp16 (1024 + q - (1024 + z) = q - z), the fp16 pairs are dotted with
// x on v_dot2_f32_f16 into fp32, and the group scale is applied once per
// chunk.  The row sum ends with a wavefront butterfly reduction.
#include "awq_internal.h"

namespace awq {
namespace {

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

template <int MT>
__global__ __launch_bounds__(256) void k_gemv_int4(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qweight,
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    _Float16* __restrict__ y, int M, int N, int K) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;                              // the whole wave leaves
    const int G = K / kGroup;
    const int n_chunks = K / 32;
    const uint4* qrow = reinterpret_cast<const uint4*>(qweight + (size_t)n * (K / 8));
    const _Float16* srow = scales + (size_t)n * G;
    const _Float16* zrow = zeros + (size_t)n * G;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

    for (int c = lane; c < n_chunks; c += kWave) {
        const uint4 w = qrow[c];
        const int g = c >> 2;
        const float d = (float)srow[g];
        const _Float16 zb = (_Float16)1024.0f + zrow[g];          // exact
        const half2_t zz = {zb, zb};
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        half2_t hq[16];                                          // pair p = k/2 in the chunk
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t b = ((ws[i] >> (4 * t)) & 0x000F000Fu) | 0x64006400u;
                hq[4 * i + t] = as_half2(b) - zz;
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)m * K + 32 * c);
                float p = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 xv = xr[j];
                    p = __builtin_amdgcn_fdot2(hq[4 * j + 0], as_half2(xv.x), p, false);
                    p = __builtin_amdgcn_fdot2(hq[4 * j + 1], as_half2(xv.y), p, false);
                    p = __builtin_amdgcn_fdot2(hq[4 * j + 2], as_half2(xv.z), p, false);
                    p = __builtin_amdgcn_fdot2(hq[4 * j + 3], as_half2(xv.w), p, false);
                }
                acc[m] = __builtin_fmaf(d, p, acc[m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc[m] += __shfl_xor(acc[m], off);
    }
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < M) y[(size_t)m * N + n] = (_Float16)acc[m];
    }
}

// int3: a chunk is 32 codes = 3 words (96-bit little-endian stream).
template <int MT>
__global__ __launch_bounds__(256) void k_gemv_int3(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qweight,
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    _Float16* __restrict__ y, int M, int N, int K) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const int G = K / kGroup;
    const int n_chunks = K / 32;
    const uint32_t* qrow = qweight + (size_t)n * (3 * (K / 32));
    const _Float16* srow = scales + (size_t)n * G;
    const _Float16* zrow = zeros + (size_t)n * G;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

    for (int c = lane; c < n_chunks; c += kWave) {
        const uint64_t lo = (uint64_t)qrow[3 * c] | ((uint64_t)qrow[3 * c + 1] << 32);
        const uint32_t hi = qrow[3 * c + 2];
        const int g = c >> 2;
        const float d = (float)srow[g];
        const _Float16 zb = (_Float16)1024.0f + zrow[g];
        const half2_t zz = {zb, zb};
        half2_t hq[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            uint32_t q2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int pos = 3 * (2 * p + e);
                uint32_t q;
                if (pos + 3 <= 64) q = (uint32_t)(lo >> pos) & 7u;
                else if (pos >= 64) q = (hi >> (pos - 64)) & 7u;
                else q = ((uint32_t)(lo >> pos) | (hi << (64 - pos))) & 7u;
                q2[e] = q;
            }
            hq[p] = as_half2((q2[0] | (q2[1] << 16)) | 0x64006400u) - zz;
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)m * K + 32 * c);
                float p = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 xv = xr[j];
                    p = __builtin_amdgcn_fdot2(hq[4 * j + 0], as_half2(xv.x), p, false);
                    p = __builtin_amdgcn_fdot2(hq[4 * j + 1], as_half2(xv.y), p, false);
                    p = __builtin_amdgcn_fdot2(hq[4 * j + 2], as_half2(xv.z), p, false);
                    p = __builtin_amdgcn_fdot2(hq[4 * j + 3], as_half2(xv.w), p, false);
                }
                acc[m] = __builtin_fmaf(d, p, acc[m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc[m] += __shfl_xor(acc[m], off);
    }
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < M) y[(size_t)m * N + n] = (_Float16)acc[m];
    }
}

template <int MT>
void launch_gemv_mt(const void* x, const void* qweight, const void* scales, const void* zeros,
                    void* y, int M, int N, int K, int bits, hipStream_t st) {
    const dim3 grid((N + 3) / 4), block(256);
    if (bits == 4) {
        hipLaunchKernelGGL(k_gemv_int4<MT>, grid, block, 0, st, (const _Float16*)x,
                           (const uint32_t*)qweight, (const _Float16*)scales,
                           (const _Float16*)zeros, (_Float16*)y, M, N, K);
    } else {
        hipLaunchKernelGGL(k_gemv_int3<MT>, grid, block, 0, st, (const _Float16*)x,
                           (const uint32_t*)qweight, (const _Float16*)scales,
                           (const _Float16*)zeros, (_Float16*)y, M, N, K);
    }
}

}  // namespace

int launch_gemv(const void* x, const void* qweight, const void* scales, const void* zeros,
                void* y, int M, int N, int K, int bits, hipStream_t st) {
    if (M <= 1) launch_gemv_mt<1>(x, qweight, scales, zeros, y, M, N, K, bits, st);
    else if (M <= 4) launch_gemv_mt<4>(x, qweight, scales, zeros, y, M, N, K, bits, st);
    else if (M <= 8) launch_gemv_mt<8>(x, qweight, scales, zeros, y, M, N, K, bits, st);
    else launch_gemv_mt<16>(x, qweight, scales, zeros, y, M, N, K, bits, st);
    return (int)hipGetLastError();
}

}  // namespace awq
