// AWQ scale search on the GPU (llm-awq README "Usage" step 1, --run_awq;
// scale from offline activation statistics, section 02.02 "AWQ" of the VPTQ
// blog; saliency from activation magnitude, "Applying AWQ with AutoAWQ").
//
//   1. s_x[k]   = mean_t |X_cal[t][k]|            exact fp64 sums
//   2. s_i[k]   = fp32(pow(max(s_x[k], 1e-4), alpha_i))   fp64 pow
//   3. D_i      = fp16(W - w_hat_i * (1/s_i))     same quantizer (codes) as quantize_pack
//   4. L_i      = sum over tiles of sum (X_cal . D_i^T)^2 / (T N)   MFMA GEMM
//   5. best     = first i with the smallest L_i; s_out = s_best
// All alphas are processed in one launch per stage (the D_i of every alpha
// live side by side in the workspace; W is read once for all of them), so
// the loss GEMM grid has n_alpha x tiles workgroups.  The reductions run in a fixed order, so the
// result does not depend on scheduling.
//
// Several layers that read the same input (q/k/v, gate/up) take one search:
// their rows are treated as the rows of one layer (read in place from each
// layer's own buffer) and the loss averages over all their outputs.
#include "awq_internal.h"

namespace awq {

namespace {

constexpr int kMaxAlpha = 64;
struct AlphaGrid { float a[kMaxAlpha]; };

// the layers searched together: their rows one after the other, layer l's
// 16-byte chunks starting at chunk cstart[l] of the whole (cstart[0] = 0)
struct LayerList {
    const uint4* w[kMaxSearchLayers];
    long long cstart[kMaxSearchLayers];
    int n;
};

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct Layout {
    size_t sx, sall, sinv, D, part, total;
};

Layout layout(int T, int N, int K, int n_alpha) {
    Layout L;
    size_t off = 0;
    L.sx = off;   off += align256((size_t)K * sizeof(float));
    L.sall = off; off += align256((size_t)n_alpha * K * sizeof(float));
    L.sinv = off; off += align256((size_t)n_alpha * K * sizeof(float));
    L.D = off;    off += align256((size_t)n_alpha * N * K * sizeof(_Float16));
    L.part = off; off += align256((size_t)n_alpha * loss_gemm_tiles(T, N) * sizeof(double));
    L.total = off;
    return L;
}

// Block: 64 columns, 1024 threads.  Thread (chunk c = tid % 8, phase r = tid / 8)
// adds |x| of columns 8c..8c+7 over rows r, r + 128, ... with one 16-byte load
// per row (eight threads read a 128-byte row segment), then the 128 phases of
// each column meet in LDS.  Sums of |fp16| in fp64 are exact for T < 2^13, so
// the order of the additions cannot change the result.
__global__ __launch_bounds__(1024) void k_act_stat(const _Float16* __restrict__ X, int T, int K,
                                                  float* __restrict__ s_x) {
    const int c = threadIdx.x & 7, r = threadIdx.x >> 3;
    const int k0 = blockIdx.x * 64 + 8 * c;              // K is a multiple of 128
    double sum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int t = r; t < T; t += 128) {
        const uint4 v = *reinterpret_cast<const uint4*>(X + (size_t)t * K + k0);
        const _Float16* h = reinterpret_cast<const _Float16*>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] += fabs((double)h[e]);
    }
    __shared__ double part[128][64 + 1];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r][8 * c + e] = sum[e];
    __syncthreads();
    if (threadIdx.x < 64) {
        double tot = 0.0;
        for (int q = 0; q < 128; ++q) tot += part[q][threadIdx.x];
        s_x[blockIdx.x * 64 + threadIdx.x] = (float)(tot / (double)T);
    }
}

__global__ __launch_bounds__(256) void k_candidate_scales(const float* __restrict__ s_x, int K,
                                                         AlphaGrid grid, int n_alpha,
                                                         float* __restrict__ s_all,
                                                         float* __restrict__ s_inv) {
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long long)n_alpha * K) return;
    const int i = (int)(t / K), k = (int)(t % K);
    const double base = fmax((double)s_x[k], 1e-4);
    const float sv = (float)pow(base, (double)grid.a[i]);
    s_all[t] = sv;
    s_inv[t] = 1.0f / sv;                         // for the loss only (D = W - w_hat * (1/s))
}

// Quantization error of every alpha: one lane = 8 consecutive weights of one
// row, GS / 8 lanes = one group (16 for 128-groups, 8 for 64-groups; the error
// does not depend on the packed format).  W is read once: each lane keeps its
// 8 weights and walks the alphas, writing D_alpha for each (s_alpha is small
// and stays in L2), so the traffic is one read of W plus the D writes.  The
// codes are rint(fp32(v / Delta)) as in awq_quantize_pack, decided in fixed
// point (quant_codes_b2); w_hat = fma(q, Delta, -z * Delta) is the exact
// (q - z) * Delta.  D multiplies by the reciprocal of s (within 1.5 fp32 ulp
// of w_hat / s before D's own fp16 rounding), which spares this VALU-bound
// loop a division per weight.
template <int Q, bool ZP, int GS>
__global__ __launch_bounds__(256) void k_quant_err(LayerList layers,
                                                  const float* __restrict__ s_all,
                                                  const float* __restrict__ s_inv, int K,
                                                  long long n_chunks, int n_alpha,
                                                  uint4* __restrict__ D) {
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const bool active = t < n_chunks;
    const int k0 = active ? (int)(t % (K / 8)) * 8 : 0;
    // this chunk's layer (rows never straddle layers: a layer holds whole rows)
    const uint4* src = layers.w[0] + t;
#pragma unroll
    for (int l = 1; l < kMaxSearchLayers; ++l)
        if (l < layers.n && t >= layers.cstart[l]) src = layers.w[l] + (t - layers.cstart[l]);
    float w[8];
    {
        const uint4 raw = active ? *src : make_uint4(0, 0, 0, 0);
        const _Float16* h = reinterpret_cast<const _Float16*>(&raw);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = (float)h[i];
    }
    for (int alpha = 0; alpha < n_alpha; ++alpha) {
        const float* s = s_all + (size_t)alpha * K + k0;
        const float* si = s_inv + (size_t)alpha * K + k0;
        float v[8], sv[8], ri[8];
        const float4 s0 = *reinterpret_cast<const float4*>(s);
        const float4 s1 = *reinterpret_cast<const float4*>(s + 4);
        const float4 r0 = *reinterpret_cast<const float4*>(si);
        const float4 r1 = *reinterpret_cast<const float4*>(si + 4);
        sv[0] = s0.x; sv[1] = s0.y; sv[2] = s0.z; sv[3] = s0.w;
        sv[4] = s1.x; sv[5] = s1.y; sv[6] = s1.z; sv[7] = s1.w;
        ri[0] = r0.x; ri[1] = r0.y; ri[2] = r0.z; ri[3] = r0.w;
        ri[4] = r1.x; ri[5] = r1.y; ri[6] = r1.z; ri[7] = r1.w;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = w[i] * sv[i];
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
#pragma unroll
        for (int m = 1; m < GS / 8; m <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, m, GS / 8));
            mx = fmaxf(mx, __shfl_xor(mx, m, GS / 8));
        }
        const GroupParams p = group_params<Q, ZP>(mn, mx);
        uint32_t T[8];
        quant_codes_b2<Q, 8>(v, p, T);                 // = quant_code of each value, << 16
        const float zd = -(p.zero * p.delta);          // exact: z <= 16, Delta an fp16 value
        uint4 out;
        _Float16* o = reinterpret_cast<_Float16*>(&out);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = (float)((T[i] >> 16) & 0xFFu);
            const float w_hat = __builtin_fmaf(q, p.delta, zd);  // (q - z) * Delta, exact
            o[i] = (_Float16)(w[i] - w_hat * ri[i]);
        }
        if (active) D[(size_t)alpha * n_chunks + t] = out;
    }
}

// One workgroup: fixed-order fp64 sums of the loss partials, first argmin.
// Wave w sums the partials of alphas w, w + 4, ...: lane l adds tiles l, l + 64,
// ... and the 64 lane sums meet in a fixed butterfly, so the result does not
// depend on scheduling.
__global__ __launch_bounds__(256) void k_select(const double* __restrict__ partials, int n_tiles,
                                               int n_alpha, double inv_count,
                                               const float* __restrict__ s_all, int K,
                                               float* __restrict__ s_out,
                                               float* __restrict__ loss_out,
                                               int* __restrict__ best_out) {
    __shared__ double loss[kMaxAlpha];
    __shared__ int best_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int a = wave; a < n_alpha; a += 4) {
        double s = 0.0;
        for (int j = lane; j < n_tiles; j += 64) s += partials[(size_t)a * n_tiles + j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
        if (lane == 0) loss[a] = s * inv_count;
    }
    __syncthreads();
    if (tid == 0) {
        int b = 0;
        for (int i = 1; i < n_alpha; ++i)
            if (loss[i] < loss[b]) b = i;
        best_s = b;
        if (best_out) *best_out = b;
    }
    __syncthreads();
    if (loss_out && tid < n_alpha) loss_out[tid] = (float)loss[tid];
    const float* sb = s_all + (size_t)best_s * K;
    for (int k = tid; k < K; k += blockDim.x) s_out[k] = sb[k];
}

}  // namespace

size_t search_workspace_bytes(int T, int N, int K, int n_alpha) {
    return layout(T, N, K, n_alpha).total;
}

template <int GS>
static auto pick_quant_err(int bits, int zero_point) {
    return bits == 4 ? (zero_point ? k_quant_err<15, true, GS> : k_quant_err<15, false, GS>)
                     : (zero_point ? k_quant_err<7, true, GS> : k_quant_err<7, false, GS>);
}

int launch_search(const void* const* Ws, const int* Ns, int n_layers, const void* X_cal, int T, int K,
                  const float* alphas, int n_alpha, int bits, int group_size, int zero_point,
                  float* s_out, float* loss_out, int* best_out, void* workspace, hipStream_t st) {
    LayerList layers{};
    int N = 0;
    for (int l = 0; l < n_layers; ++l) {
        layers.w[l] = static_cast<const uint4*>(Ws[l]);
        layers.cstart[l] = (long long)N * (K / 8);
        N += Ns[l];
    }
    layers.n = n_layers;
    const Layout L = layout(T, N, K, n_alpha);
    char* ws = static_cast<char*>(workspace);
    float* s_x = reinterpret_cast<float*>(ws + L.sx);
    float* s_all = reinterpret_cast<float*>(ws + L.sall);
    float* s_inv = reinterpret_cast<float*>(ws + L.sinv);
    _Float16* D = reinterpret_cast<_Float16*>(ws + L.D);
    double* part = reinterpret_cast<double*>(ws + L.part);

    AlphaGrid grid{};
    for (int i = 0; i < n_alpha; ++i) grid.a[i] = alphas[i];

    hipLaunchKernelGGL(k_act_stat, dim3(K / 64), dim3(1024), 0, st, (const _Float16*)X_cal, T, K, s_x);
    const long long nsk = (long long)n_alpha * K;
    hipLaunchKernelGGL(k_candidate_scales, dim3((unsigned)((nsk + 255) / 256)), dim3(256), 0, st,
                       s_x, K, grid, n_alpha, s_all, s_inv);
    const long long n_chunks = (long long)N * K / 8;
    auto qerr = group_size == 64 ? pick_quant_err<64>(bits, zero_point)
                                 : pick_quant_err<128>(bits, zero_point);
    hipLaunchKernelGGL(qerr, dim3((unsigned)((n_chunks + 255) / 256)), dim3(256), 0, st, layers,
                       s_all, s_inv, K, n_chunks, n_alpha, (uint4*)D);
    int err = (int)hipGetLastError();
    if (err) return err;
    err = launch_loss_gemm(X_cal, D, T, N, K, n_alpha, part, st);
    if (err) return err;
    const int n_tiles = (int)loss_gemm_tiles(T, N);
    hipLaunchKernelGGL(k_select, dim3(1), dim3(256), 0, st, part, n_tiles, n_alpha,
                       1.0 / ((double)T * (double)N), s_all, K, s_out, loss_out, best_out);
    return (int)hipGetLastError();
}

}  // namespace awq
