// Context-stage (prefill) W4A16 GEMM and the dense fp16 loss GEMM of the
// scale search, both on fp16 MFMA with fp32 accumulation.
//
// Y[m][n] = sum_k X[m][k] * B[n][k]   ("NT": both operands K-contiguous)
//   W4A16: B = w_hat = (q - z) * D, dequantized tile by tile into LDS
//          (context kernel of the llm-awq README feature list; version
//          "gemm" of the transformers quantization_config).
//   loss:  B = D_alpha = W - w_hat_alpha / s_alpha (fp16), and the epilogue
//          sums Y^2 per tile instead of storing Y.
//
// Tiling: a 256-thread workgroup owns a 128x128 output tile and walks K in
// steps of 128 (one quantization group, so each B row has one scale and one
// zero per step).  The four waves form a 2x2 grid of 64x64 sub-tiles, each
// 4x4 v_mfma_f32_16x16x32_f16 blocks.  Global loads of step k+1 are issued
// into registers before the MFMAs of step k, then written to LDS.
#include "awq_internal.h"

namespace awq {
namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 8;          // halves; +16 B per row against bank conflicts

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

template <bool B_INT4, bool SQSUM>
__global__ __launch_bounds__(256) void k_gemm(
    const _Float16* __restrict__ A, const void* __restrict__ Bv,
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    _Float16* __restrict__ Y, double* __restrict__ partials, int M, int N, int K,
    long long b_batch_stride) {
    __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int G = K / kGroup;
    const int KT = K / BK;

    const uint32_t* Bq = reinterpret_cast<const uint32_t*>(Bv);
    const _Float16* Bh = reinterpret_cast<const _Float16*>(Bv) + (size_t)blockIdx.z * b_batch_stride;

    // registers for one K-step of global data
    uint4 ra[8];
    uint4 rb[B_INT4 ? 2 : 8];
    _Float16 rs[2], rz[2];

    auto load_step = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = tid + 256 * i, r = id >> 4, c = id & 15, m = m0 + r;
            ra[i] = m < M ? *reinterpret_cast<const uint4*>(A + (size_t)m * K + kt * BK + c * 8)
                          : make_uint4(0, 0, 0, 0);
        }
        if constexpr (B_INT4) {
            // format 2: tile (block, kt) is 64 slots of 16 B; slot s = 16h + j
            // is row 16*block + j, codes 32h..32h+31 of the group
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int id = tid + 256 * i, rb16 = id >> 6, slot = id & 63;
                const int blk = n0 / 16 + rb16;
                if (16 * blk < N) {
                    rb[i] = *reinterpret_cast<const uint4*>(Bq + ((size_t)blk * G + kt) * 256 + slot * 4);
                } else {
                    rb[i] = make_uint4(0, 0, 0, 0);
                }
                // format-2 scales/zeros: [block][g][16], zero on padding rows
                const size_t pidx = ((size_t)blk * G + kt) * 16 + (slot & 15);
                rs[i] = 16 * blk < N ? scales[pidx] : (_Float16)0.0f;
                rz[i] = 16 * blk < N ? zeros[pidx] : (_Float16)0.0f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int id = tid + 256 * i, r = id >> 4, c = id & 15, n = n0 + r;
                rb[i] = n < N ? *reinterpret_cast<const uint4*>(Bh + (size_t)n * K + kt * BK + c * 8)
                              : make_uint4(0, 0, 0, 0);
            }
        }
    };

    auto store_step = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = tid + 256 * i, r = id >> 4, c = id & 15;
            *reinterpret_cast<uint4*>(&As[r * LDS_STRIDE + c * 8]) = ra[i];
        }
        if constexpr (B_INT4) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int id = tid + 256 * i, slot = id & 63;
                const int r = 16 * (id >> 6) + (slot & 15), c = slot >> 4;
                const _Float16 zb = (_Float16)1024.0f + rz[i];
                const half2_t zz = {zb, zb};
                const half2_t dd = {rs[i], rs[i]};
                const uint32_t ws[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint4 out;
                    uint32_t* o = reinterpret_cast<uint32_t*>(&out);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint32_t b = ((ws[d] >> (4 * t)) & 0x000F000Fu) | 0x64006400u;
                        o[t] = as_u32((as_half2(b) - zz) * dd);
                    }
                    *reinterpret_cast<uint4*>(&Bs[r * LDS_STRIDE + c * 32 + d * 8]) = out;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int id = tid + 256 * i, r = id >> 4, c = id & 15;
                *reinterpret_cast<uint4*>(&Bs[r * LDS_STRIDE + c * 8]) = rb[i];
            }
        }
    };

    float4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

    load_step(0);
    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();                       // previous step's reads are done
        store_step();
        __syncthreads();
        if (kt + 1 < KT) load_step(kt + 1);    // in flight during the MFMAs
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            half8_t a[4], b[4];
            const int kk = ks * 32 + (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const half8_t*>(&As[(wm * 64 + i * 16 + (lane & 15)) * LDS_STRIDE + kk]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const half8_t*>(&Bs[(wn * 64 + j * 16 + (lane & 15)) * LDS_STRIDE + kk]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // 16x16 accumulator layout: lane holds column (lane & 15), rows 4*(lane>>4) + r
    if constexpr (SQSUM) {
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) sq = __builtin_fmaf(acc[i][j][r], acc[i][j][r], sq);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
        __shared__ double wsum[4];
        if (lane == 0) wsum[wave] = (double)sq;
        __syncthreads();
        if (tid == 0) {
            const size_t tile = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
            const size_t n_tiles = (size_t)gridDim.x * gridDim.y;
            partials[(size_t)blockIdx.z * n_tiles + tile] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
                    if (m < M && n < N) Y[(size_t)m * N + n] = (_Float16)acc[i][j][r];
                }
            }
        }
    }
}

}  // namespace

int launch_gemm(const void* x, const void* qweight, const void* scales, const void* zeros,
                void* y, int M, int N, int K, hipStream_t st) {
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, 1), block(256);
    hipLaunchKernelGGL((k_gemm<true, false>), grid, block, 0, st, (const _Float16*)x, qweight,
                       (const _Float16*)scales, (const _Float16*)zeros, (_Float16*)y,
                       (double*)nullptr, M, N, K, 0LL);
    return (int)hipGetLastError();
}

size_t loss_gemm_tiles(int T, int N) {
    return (size_t)((N + BN - 1) / BN) * (size_t)((T + BM - 1) / BM);
}

int launch_loss_gemm(const void* X, const void* D, int T, int N, int K, int n_batch,
                     double* partials, hipStream_t st) {
    const dim3 grid((N + BN - 1) / BN, (T + BM - 1) / BM, n_batch), block(256);
    hipLaunchKernelGGL((k_gemm<false, true>), grid, block, 0, st, (const _Float16*)X, D,
                       (const _Float16*)nullptr, (const _Float16*)nullptr, (_Float16*)nullptr,
                       partials, T, N, K, (long long)N * K);
    return (int)hipGetLastError();
}

}  // namespace awq
