// Group quantization + packing (format v1) and the activation-side divide.
//
// What is computed: round-to-nearest asymmetric quantization of W*diag(s)
// in groups of 128 input channels, with an fp16 scale and an integer zero
// point per group ("Quantizing a model with AutoAWQ": w_bit, q_group_size,
// zero_point; llm-awq README "Usage" step 3, real INT4 weights).
//
// Layout of the work: W is row-major [N][K] and groups run along K, so the
// groups are contiguous 256-byte runs of W and the whole matrix is a flat
// sequence of groups.  int4: one lane quantizes 8 consecutive weights (one
// 16-byte load, one packed 32-bit word), 16 lanes form a group and reduce
// min/max with cross-lane shuffles.  int3: one lane takes 32 weights (four
// 16-byte loads, three packed words), 4 lanes form a group.  Loads and
// stores of a wave are contiguous; the kernel is HBM-bound (offline).
#include "awq_internal.h"

namespace awq {
namespace {

__device__ __forceinline__ void unpack8(const uint4& raw, float* f) {
    const _Float16* h = reinterpret_cast<const _Float16*>(&raw);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}

template <int WIDTH>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
#pragma unroll
    for (int m = 1; m < WIDTH; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m, WIDTH));
        mx = fmaxf(mx, __shfl_xor(mx, m, WIDTH));
    }
}

// bits = 4: lane t handles flat elements [8t, 8t+8) of W.
__global__ __launch_bounds__(256) void k_quantize_pack_int4(
    const uint4* __restrict__ W, const float* __restrict__ s, int K, long long n_chunks,
    uint32_t* __restrict__ qweight, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
    constexpr int Q = 15;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const bool active = t < n_chunks;   // whole 16-lane groups are active or not
    float v[8];
    if (active) {
        unpack8(W[t], v);
        if (s != nullptr) {
            const int k0 = (int)(t % (K / 8)) * 8;
            const float4 s0 = *reinterpret_cast<const float4*>(s + k0);
            const float4 s1 = *reinterpret_cast<const float4*>(s + k0 + 4);
            v[0] *= s0.x; v[1] *= s0.y; v[2] *= s0.z; v[3] *= s0.w;
            v[4] *= s1.x; v[5] *= s1.y; v[6] *= s1.z; v[7] *= s1.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
    group_minmax<16>(mn, mx);
    const GroupParams p = group_params<Q>(mn, mx);
    uint32_t word = 0;
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2) {
        word |= quant_code<Q>(v[2 * t2], p) << (4 * t2);
        word |= quant_code<Q>(v[2 * t2 + 1], p) << (16 + 4 * t2);
    }
    if (active) {
        qweight[t] = word;
        if ((threadIdx.x & 15) == 0) {
            const long long gidx = t >> 4;
            scales[gidx] = p.dbits;
            zeros[gidx] = half_bits((_Float16)p.zero);
        }
    }
}

// bits = 3: lane t handles flat elements [32t, 32t+32) -> words 3t..3t+2.
__global__ __launch_bounds__(256) void k_quantize_pack_int3(
    const uint4* __restrict__ W, const float* __restrict__ s, int K, long long n_chunks,
    uint32_t* __restrict__ qweight, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
    constexpr int Q = 7;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const bool active = t < n_chunks;
    float v[32];
    if (active) {
#pragma unroll
        for (int j = 0; j < 4; ++j) unpack8(W[4 * t + j], v + 8 * j);
        if (s != nullptr) {
            const int k0 = (int)(t % (K / 32)) * 32;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 sj = *reinterpret_cast<const float4*>(s + k0 + 4 * j);
                v[4 * j] *= sj.x; v[4 * j + 1] *= sj.y; v[4 * j + 2] *= sj.z; v[4 * j + 3] *= sj.w;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
    group_minmax<4>(mn, mx);
    const GroupParams p = group_params<Q>(mn, mx);
    uint64_t lo = 0;
    uint32_t hi = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t q = quant_code<Q>(v[i], p);
        const int pos = 3 * i;
        if (pos + 3 <= 64) {
            lo |= (uint64_t)q << pos;
        } else if (pos >= 64) {
            hi |= q << (pos - 64);
        } else {                       // code straddles stream bit 64
            lo |= (uint64_t)q << pos;
            hi |= q >> (64 - pos);
        }
    }
    if (active) {
        qweight[3 * t] = (uint32_t)lo;
        qweight[3 * t + 1] = (uint32_t)(lo >> 32);
        qweight[3 * t + 2] = hi;
        if ((threadIdx.x & 3) == 0) {
            const long long gidx = t >> 2;
            scales[gidx] = p.dbits;
            zeros[gidx] = half_bits((_Float16)p.zero);
        }
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

}  // namespace

int launch_quantize_pack(const void* W, const float* s, int N, int K, int bits, void* qweight,
                         void* scales, void* zeros, hipStream_t st) {
    const long long elems = (long long)N * K;
    const int per_lane = bits == 4 ? 8 : 32;
    const long long n_chunks = elems / per_lane;
    const int block = 256;
    const long long grid = (n_chunks + block - 1) / block;
    if (bits == 4) {
        hipLaunchKernelGGL(k_quantize_pack_int4, dim3((unsigned)grid), dim3(block), 0, st,
                           (const uint4*)W, s, K, n_chunks, (uint32_t*)qweight,
                           (uint16_t*)scales, (uint16_t*)zeros);
    } else {
        hipLaunchKernelGGL(k_quantize_pack_int3, dim3((unsigned)grid), dim3(block), 0, st,
                           (const uint4*)W, s, K, n_chunks, (uint32_t*)qweight,
                           (uint16_t*)scales, (uint16_t*)zeros);
    }
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

}  // namespace awq
