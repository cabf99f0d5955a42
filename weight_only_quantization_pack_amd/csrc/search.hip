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

// The loss runs one of two ways: a separate error kernel writing D for every
// alpha into the workspace plus a dense loss GEMM (the default: fastest, needs
// one chunk of alphas' D, N rounded up to 16), or one fused kernel forming D
// in registers (a workspace of under a megabyte; MI355X, 4096 x 4096, T = 512,
// 20 alphas: 0.73 ms against 0.65-0.68 ms median, since forming D there does
// not overlap its MFMAs).  The fused kernel's workgroup takes 512 calibration
// rows and one 16-row tile of W per wave, so every D value is formed once per
// alpha (256 rows and two tiles per wave, which forms each D twice at T = 512:
// 0.82 ms; 256 rows and one tile: 0.98 ms)
constexpr int kFusedT = 512;            // calibration rows per workgroup of the fused loss
constexpr int kFusedNT = 1;             // 16-row tiles of W per wave (4 waves)
constexpr int kFusedRows = 64 * kFusedNT;
size_t fused_tiles(int T, int N) {
    return (size_t)((N + kFusedRows - 1) / kFusedRows) * (size_t)((T + kFusedT - 1) / kFusedT);
}

// The default path runs the alpha grid in chunks whose error matrices D fit
// in half of the 256 MB Infinity Cache, so the loss GEMM reads D back from the
// cache rather than from HBM, and the workspace holds one chunk (W is read
// once per chunk).  A D of more than that is one alpha per chunk.
#ifndef AWQ_SEARCH_CHUNK_BYTES
#define AWQ_SEARCH_CHUNK_BYTES ((size_t)128 << 20)
#endif
int alpha_chunk(size_t d_bytes_per_alpha, int n_alpha) {
    const size_t c = AWQ_SEARCH_CHUNK_BYTES / (d_bytes_per_alpha > 0 ? d_bytes_per_alpha : 1);
    return (int)(c < 1 ? 1 : (c > (size_t)n_alpha ? (size_t)n_alpha : c));
}

struct Layout {
    size_t sx, sall, sinv, D, part, total;
    int chunk;                          // alphas per error-kernel + loss-GEMM pass
};

Layout layout(int T, int N, int K, int n_alpha, bool fused) {
    Layout L;
    const size_t d_alpha = loss_rows(N) * K * sizeof(_Float16);
    L.chunk = fused ? n_alpha : alpha_chunk(d_alpha, n_alpha);
    size_t off = 0;
    L.sx = off;   off += align256((size_t)K * sizeof(float));
    L.sall = off; off += align256((size_t)n_alpha * K * sizeof(float));
    L.sinv = off; off += align256((size_t)n_alpha * K * sizeof(float));
    L.D = off;    off += fused ? 0 : align256((size_t)L.chunk * d_alpha);
    L.part = off; off += align256((size_t)n_alpha * (fused ? fused_tiles(T, N) : loss_gemm_tiles(T, N)) * sizeof(double));
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

// Quantization error of every alpha.  One workgroup per 16-row x 128-column
// tile of W (block b, group g of 128 columns), written as one tile of D in
// the loss GEMM's layout: wave q takes the tile's k32 step q, lane 16 hq + j
// the 8 weights of row 16 b + j at columns 128 g + 32 hq + 8 q .. + 7, so each
// wave stores its D step as one contiguous 1 KB run per alpha.  A group's
// min/max is met over the lanes of a row that hold it (all 4 quarters hq for
// 128-groups, hq and hq ^ 1 for 64-groups) and then over the 4 waves through
// LDS, one barrier per alpha.  W is read once: each lane
// keeps its 8 weights and walks the alphas, writing D_alpha for each (s_alpha
// is small and stays in L2).  The codes are rint(fp32(v / Delta)) as in
// awq_quantize_pack, decided in fixed point (quant_codes_b2); w_hat =
// fma(q, Delta, -z * Delta) is the exact (q - z) * Delta.  D multiplies by
// the reciprocal of s (within 1.5 fp32 ulp of w_hat / s before D's own fp16
// rounding), which spares this VALU-bound loop a division per weight.  Rows
// past N (the last block's padding) load nothing and store nothing.
template <int Q, bool ZP, int GS>
__global__ __launch_bounds__(256) void k_quant_err(LayerList layers,
                                                  const float* __restrict__ s_all,
                                                  const float* __restrict__ s_inv, int N, int K,
                                                  int n_alpha, long long d_stride,
                                                  uint4* __restrict__ D) {
    __shared__ float red[2][2][4][4][16];              // [alpha parity][min, max][step q][quarter hq][row j]
    const int G = K / kGroup;
    const int b = (int)(blockIdx.x / (unsigned)G), g = (int)(blockIdx.x % (unsigned)G);
    const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane & 15, hq = lane >> 4;
    const int n = 16 * b + j;
    const bool active = n < N;
    const int k0 = kGroup * g + 32 * hq + 8 * q;
    // this chunk's layer (rows never straddle layers: a layer holds whole rows)
    const long long t = (long long)n * (K / 8) + k0 / 8;
    const uint4* src = layers.w[0] + t;
#pragma unroll
    for (int l = 1; l < kMaxSearchLayers; ++l)
        if (l < layers.n && t >= layers.cstart[l]) src = layers.w[l] + (t - layers.cstart[l]);
    const size_t dpos = ((size_t)blockIdx.x * 4 + q) * 64 + lane;
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
        // the row's lanes of this step in the group (lanes j + 16 hq: hq ^ 1 for
        // 64-groups, all four for 128-groups)
        mn = fminf(mn, __shfl_xor(mn, 16)); mx = fmaxf(mx, __shfl_xor(mx, 16));
        if constexpr (GS == 128) {
            mn = fminf(mn, __shfl_xor(mn, 32)); mx = fmaxf(mx, __shfl_xor(mx, 32));
        }
        // the group's other steps (the 4 waves): min and max are exact, so the
        // order is free
        const int par = alpha & 1;
        red[par][0][q][hq][j] = mn; red[par][1][q][hq][j] = mx;
        __syncthreads();
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            mn = fminf(mn, red[par][0][o][hq][j]); mx = fmaxf(mx, red[par][1][o][hq][j]);
        }
        const GroupParams p = group_params<Q, ZP>(mn, mx);
        uint32_t T[8];
        quant_codes_b2<Q, 8>(v, p, T);                 // = quant_code of each value, << 16
        const float zd = -(p.zero * p.delta);          // exact: z <= 16, Delta an fp16 value
        uint4 out;
        _Float16* o = reinterpret_cast<_Float16*>(&out);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float qf = (float)((T[i] >> 16) & 0xFFu);
            const float w_hat = __builtin_fmaf(qf, p.delta, zd);  // (q - z) * Delta, exact
            o[i] = (_Float16)(w[i] - w_hat * ri[i]);
        }
        if (active) D[(size_t)alpha * d_stride + dpos] = out;
    }
}

// Fused loss (the error matrix D_alpha = W - w_hat_alpha / s_alpha never goes
// to memory): L_alpha * T * N = sum over (t, n) of (X D_alpha^T)[t][n]^2.  A
// workgroup owns 64 rows of W (one 16-row MFMA B tile per wave) and up to 512
// calibration rows for one alpha, so every D value is formed once per alpha:
// each wave builds its D fragments in registers in the B-operand layout of
// v_mfma_f32_16x16x32_f16 (lane (j, q) holds row j's k = 32 s + 8 q + e of
// substep s), quantizing the group from W, s and 1/s with the codes of
// quant_codes_b2, exactly as the separate error kernel does.  X streams
// through LDS in 64-k steps (512 rows x 128 B, two buffers, direct-to-LDS
// loads, chunk p of row r holding global chunk p ^ (r & 7), which the
// A-fragment reads see free of bank conflicts on MI355X); W of the next group
// is loaded into registers one group ahead, its s and 1/s into LDS.  The 32
// MFMA accumulators of a lane (128 fp32) live in AGPRs.  The epilogue squares
// and sums the outputs of rows < T and columns < N in fp32 per lane, then in
// fp64 in a fixed order, into one partial per workgroup.
namespace lf {
constexpr int kT = kFusedT;             // calibration rows per workgroup
constexpr int kFR = kT / 16;            // X fragments per substep
constexpr int kStepK = 64;              // k per LDS step (half a group)
constexpr int kRow = kStepK * 2;        // bytes of one X row in LDS
constexpr int kBuf = kT * kRow;         // 64 KB per buffer
constexpr int kXLoads = kBuf / 1024 / 4;   // direct-to-LDS loads per wave and step (16)
constexpr int kWLoads = kFusedNT * 4;      // W loads per wave and group
}

struct RowList {                        // rows of the layers searched together
    const _Float16* w[kMaxSearchLayers];
    int nstart[kMaxSearchLayers];
    int n;
};

template <int Q, bool ZP, int GS>
__global__ __launch_bounds__(256, 1) void k_loss_fused(RowList layers, const _Float16* __restrict__ X,
                                                       int T, int N, int K,
                                                       const float* __restrict__ s_all,
                                                       const float* __restrict__ s_inv,
                                                       double* __restrict__ partials) {
    static_assert(GS == 128 || GS == 64, "128- or 64-wide groups");
    extern __shared__ __attribute__((aligned(16))) unsigned char Xs[];   // 2 x lf::kBuf, then the s slots
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, hq = lane >> 4;
    const int alpha = blockIdx.z;
    const int t0 = blockIdx.y * lf::kT;
    const int G = K / kGroup;
    constexpr int NT = kFusedNT;
    const int n_base = blockIdx.x * kFusedRows + wave * 16 * NT;

    // this lane's W row in each of its two tiles (rows past N: row N - 1, never summed)
    const _Float16* wrow[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int n = min(n_base + 16 * c + j, N - 1);
        int l = 0;
#pragma unroll
        for (int m = 1; m < kMaxSearchLayers; ++m)
            if (m < layers.n && n >= layers.nstart[m]) l = m;
        wrow[c] = layers.w[l] + (size_t)(n - layers.nstart[l]) * K;
    }

    // X: load q (0..kXLoads-1) of this wave writes rows 8 (kXLoads wave + q) .. + 7
    // of the tile, lane l row + (l >> 3), LDS chunk l & 7; rows past T read row T - 1
    uint32_t x_off[lf::kXLoads];
#pragma unroll
    for (int q = 0; q < lf::kXLoads; ++q) {
        const int rr = 8 * (lf::kXLoads * wave + q) + (lane >> 3);
        const int row = min(t0 + rr, T - 1);
        const int kc = (lane & 7) ^ (rr & 7);
        x_off[q] = (uint32_t)row * (uint32_t)K + 8u * (uint32_t)kc;
    }
    auto issue_x = [&](int step, int buf) {
        const uint32_t k0 = (uint32_t)min(step, 2 * G - 1) * lf::kStepK;
#pragma unroll
        for (int q = 0; q < lf::kXLoads; ++q)
            __builtin_amdgcn_global_load_lds((global_void_t*)(X + x_off[q] + k0),
                                             (lds_void_t*)(Xs + buf * lf::kBuf + (lf::kXLoads * wave + q) * 1024),
                                             16, 0, 0);
    };

    // the next group's W rows, loaded one group ahead (its s and 1/s go to
    // LDS during the second half of the group before): value i = 8 sub + e
    // of a lane is k = 32 sub + 8 q + e of the group
    struct PreW { uint4 w[NT][4]; };
    // s and 1/s of a group go to LDS (two slots: the group being quantized and
    // the next), written by wave 0 with one direct-to-LDS load (lanes 0..31
    // the 128 s values, lanes 32..63 the 128 reciprocals) and read by every
    // wave while it forms D; registers would hold them for a whole group
    float* const Ss = reinterpret_cast<float*>(Xs + 2 * lf::kBuf);   // [2 slots][s 128, 1/s 128]
    auto issue_w = [&](int g, PreW& p) {
        const int k0 = kGroup * min(g, G - 1);
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int sub = 0; sub < 4; ++sub)
                p.w[c][sub] = *reinterpret_cast<const uint4*>(wrow[c] + k0 + 32 * sub + 8 * hq);
    };
    auto issue_s = [&](int g, int slot) {
        if (wave != 0) return;                       // wave-uniform
        const int k0 = kGroup * min(g, G - 1);
        const float* src = (lane < 32 ? s_all : s_inv) + (size_t)alpha * K + k0 + 4 * (lane & 31);
        __builtin_amdgcn_global_load_lds((global_void_t*)src, (lds_void_t*)(Ss + slot * 256), 16, 0, 0);
    };
    auto f4 = [](const float4& q, int e) { return e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w; };
    auto wval = [](const uint4& raw, int e) {
        return (float)reinterpret_cast<const _Float16*>(&raw)[e];
    };

    half8_t dfr[NT][4];                  // D fragments of the current group: [tile][substep]
    auto make_d = [&](const PreW& pw, int slot) {
        // value i = 8 sub + e of this lane is column 32 sub + 8 hq + e of the group
        struct { float4 s[8], r[8]; } ps;
        const float* sl = Ss + slot * 256 + 8 * hq;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            ps.s[2 * sub] = *reinterpret_cast<const float4*>(sl + 32 * sub);
            ps.s[2 * sub + 1] = *reinterpret_cast<const float4*>(sl + 32 * sub + 4);
            ps.r[2 * sub] = *reinterpret_cast<const float4*>(sl + 128 + 32 * sub);
            ps.r[2 * sub + 1] = *reinterpret_cast<const float4*>(sl + 128 + 32 * sub + 4);
        }
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            float v[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = wval(pw.w[c][i / 8], i % 8) * f4(ps.s[i / 4], i % 4);
            constexpr int NV = GS / 4;       // values of one group in a lane
#pragma unroll
            for (int gg = 0; gg < 32 / NV; ++gg) {
                float mn = v[NV * gg], mx = v[NV * gg];
#pragma unroll
                for (int i = 1; i < NV; ++i) { mn = fminf(mn, v[NV * gg + i]); mx = fmaxf(mx, v[NV * gg + i]); }
                // the group's other values sit in the lanes of the same row j
                mn = fminf(mn, __shfl_xor(mn, 16)); mx = fmaxf(mx, __shfl_xor(mx, 16));
                mn = fminf(mn, __shfl_xor(mn, 32)); mx = fmaxf(mx, __shfl_xor(mx, 32));
                const GroupParams gp = group_params<Q, ZP>(mn, mx);
                uint32_t Tc[NV];
                quant_codes_b2<Q, NV>(v + NV * gg, gp, Tc);
                const float zd = -(gp.zero * gp.delta);     // exact: z <= 16, Delta an fp16 value
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const int idx = NV * gg + i;
                    const float q = (float)((Tc[i] >> 16) & 0xFFu);
                    const float w_hat = __builtin_fmaf(q, gp.delta, zd);   // (q - z) * Delta, exact
                    const float w = wval(pw.w[c][idx / 8], idx % 8);
                    dfr[c][idx / 8][idx % 8] = (_Float16)(w - w_hat * f4(ps.r[idx / 4], idx % 4));
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // one tile's temporaries at a time
        }
    };

    float4_t acc[lf::kFR][NT];         // [X fragment][tile]
#pragma unroll
    for (int i = 0; i < lf::kFR; ++i)
#pragma unroll
        for (int c = 0; c < NT; ++c) acc[i][c] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // the two substeps of one LDS step (half h of the group): X fragments in
    // batches of 8, batch b + 1 read under batch b's 16 MFMAs (a scheduling
    // barrier per batch keeps the compiler from hoisting every read)
    constexpr int kB = 8, kNB = 2 * lf::kFR / kB;          // batches per LDS step
    auto read_batch = [&](const unsigned char* buf, int b, half8_t* xf) {
        const int sub = b / (lf::kFR / kB), i0 = (b % (lf::kFR / kB)) * kB;
        const int kc = 4 * sub + hq;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int r = 16 * (i0 + u) + j;
            xf[u] = *reinterpret_cast<const half8_t*>(buf + r * lf::kRow + ((kc ^ (r & 7)) << 4));
        }
    };
    auto compute_half = [&](int h, const unsigned char* buf) {
        half8_t xa[kB], xb[kB];
        read_batch(buf, 0, xa);
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            half8_t* cur = (b & 1) ? xb : xa;
            half8_t* nxt = (b & 1) ? xa : xb;
            if (b + 1 < kNB) read_batch(buf, b + 1, nxt);
            const int sub = b / (lf::kFR / kB), i0 = (b % (lf::kFR / kB)) * kB;
#pragma unroll
            for (int u = 0; u < kB; ++u)
#pragma unroll
                for (int c = 0; c < NT; ++c)
                    acc[i0 + u][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dfr[c][2 * h + sub], cur[u], acc[i0 + u][c], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    PreW pw;
    issue_x(0, 0);
    issue_w(0, pw);
    issue_s(0, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int g = 0; g < G; ++g) {
        // step 2g, buffer 0: X(2g) and the group's W, s, 1/s have landed
        __builtin_amdgcn_sched_barrier(0);
        issue_x(2 * g + 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        make_d(pw, g & 1);
        __builtin_amdgcn_sched_barrier(0);
        issue_w(g + 1, pw);                  // clamped past the last group: a uniform load stream
        __builtin_amdgcn_sched_barrier(0);
        compute_half(0, Xs);
        // step 2g + 1, buffer 1: X(2g + 1) has landed once at most the next
        // group's W loads are outstanding; every wave is done with buffer 0
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(lf::kWLoads));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        issue_x(2 * g + 2, 0);
        issue_s(g + 1, (g + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(1, Xs + lf::kBuf);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    float sq = 0.0f;
#pragma unroll
    for (int i = 0; i < lf::kFR; ++i) {
        const bool t_ok = t0 + 16 * i + j < T;
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = t_ok && n_base + 16 * c + 4 * hq + r < N;
                sq = __builtin_fmaf(ok ? acc[i][c][r] : 0.0f, ok ? acc[i][c][r] : 0.0f, sq);
            }
    }
    double dsq = (double)sq;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dsq += __shfl_xor(dsq, off);
    __shared__ double wsum[4];
    if (lane == 0) wsum[wave] = dsq;
    __syncthreads();
    if (tid == 0) {
        const size_t tile = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
        const size_t n_tiles = (size_t)gridDim.x * gridDim.y;
        partials[(size_t)alpha * n_tiles + tile] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
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

// Rows of the layers in `layers` (fp16, row-major, the N rows one layer after
// the other) rewritten in the loss GEMM's tiled layout, as k_quant_err writes
// D: one workgroup per 16-row x 128-column tile, wave q its k32 step, lane
// 16 hq + j the 8 values of row 16 b + j at columns 128 g + 32 hq + 8 q.
// Padding rows of the last block are written as zeros.
__global__ __launch_bounds__(256) void k_tile_rows(LayerList layers, int N, int K, uint4* __restrict__ out) {
    const int G = K / kGroup;
    const int b = (int)(blockIdx.x / (unsigned)G), g = (int)(blockIdx.x % (unsigned)G);
    const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane & 15, hq = lane >> 4;
    const int n = 16 * b + j;
    const int k0 = kGroup * g + 32 * hq + 8 * q;
    const long long t = (long long)n * (K / 8) + k0 / 8;
    const uint4* src = layers.w[0] + t;
#pragma unroll
    for (int l = 1; l < kMaxSearchLayers; ++l)
        if (l < layers.n && t >= layers.cstart[l]) src = layers.w[l] + (t - layers.cstart[l]);
    out[((size_t)blockIdx.x * 4 + q) * 64 + lane] = n < N ? *src : make_uint4(0, 0, 0, 0);
}

}  // namespace

size_t search_workspace_bytes(int T, int N, int K, int n_alpha, bool fused) {
    return layout(T, N, K, n_alpha, fused).total;
}

template <int GS>
static auto pick_loss_fused(int bits, int zero_point) {
    return bits == 4 ? (zero_point ? k_loss_fused<15, true, GS> : k_loss_fused<15, false, GS>)
                     : (zero_point ? k_loss_fused<7, true, GS> : k_loss_fused<7, false, GS>);
}

template <int GS>
static auto pick_quant_err(int bits, int zero_point) {
    return bits == 4 ? (zero_point ? k_quant_err<15, true, GS> : k_quant_err<15, false, GS>)
                     : (zero_point ? k_quant_err<7, true, GS> : k_quant_err<7, false, GS>);
}

int launch_search(const void* const* Ws, const int* Ns, int n_layers, const void* X_cal, int T, int K,
                  const float* alphas, int n_alpha, int bits, int group_size, int zero_point,
                  float* s_out, float* loss_out, int* best_out, void* workspace, bool fused,
                  hipStream_t st) {
    LayerList layers{};
    int N = 0;
    for (int l = 0; l < n_layers; ++l) {
        layers.w[l] = static_cast<const uint4*>(Ws[l]);
        layers.cstart[l] = (long long)N * (K / 8);
        N += Ns[l];
    }
    layers.n = n_layers;
    const Layout L = layout(T, N, K, n_alpha, fused);
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
    int n_tiles;
    if (fused) {
        RowList rows{};
        int n0 = 0;
        for (int l = 0; l < n_layers; ++l) {
            rows.w[l] = static_cast<const _Float16*>(Ws[l]);
            rows.nstart[l] = n0;
            n0 += Ns[l];
        }
        rows.n = n_layers;
        auto kern = group_size == 64 ? pick_loss_fused<64>(bits, zero_point)
                                     : pick_loss_fused<128>(bits, zero_point);
        const int lds = 2 * lf::kBuf + 2 * 256 * (int)sizeof(float);
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return (int)e;
        const dim3 grid_f((N + kFusedRows - 1) / kFusedRows, (T + lf::kT - 1) / lf::kT, n_alpha);
        hipLaunchKernelGGL(kern, grid_f, dim3(256), lds, st, rows, (const _Float16*)X_cal, T, N, K,
                           (const float*)s_all, (const float*)s_inv, part);
        const int err = (int)hipGetLastError();
        if (err) return err;
        n_tiles = (int)fused_tiles(T, N);
    } else {
        auto qerr = group_size == 64 ? pick_quant_err<64>(bits, zero_point)
                                     : pick_quant_err<128>(bits, zero_point);
        const size_t n_tiles16 = loss_rows(N) / 16 * (size_t)(K / kGroup);
        n_tiles = (int)loss_gemm_tiles(T, N);
        for (int a0 = 0; a0 < n_alpha; a0 += L.chunk) {
            const int na = min(L.chunk, n_alpha - a0);
            hipLaunchKernelGGL(qerr, dim3((unsigned)n_tiles16), dim3(256), 0, st, layers,
                               (const float*)s_all + (size_t)a0 * K, (const float*)s_inv + (size_t)a0 * K,
                               N, K, na, (long long)loss_rows(N) * K / 8, (uint4*)D);
            int err = (int)hipGetLastError();
            if (err) return err;
            err = launch_loss_gemm(X_cal, 0, D, (long long)loss_rows(N) * K, T, N, K, na,
                                   part + (size_t)a0 * n_tiles, st);
            if (err) return err;
        }
    }
    hipLaunchKernelGGL(k_select, dim3(1), dim3(256), 0, st, part, n_tiles, n_alpha,
                       1.0 / ((double)T * (double)N), s_all, K, s_out, loss_out, best_out);
    return (int)hipGetLastError();
}

namespace {
// workspace of the block-output search
struct MlpLayout {
    size_t sx, sall, sinv, D, wt, wdt, ref, dh, part, total;
    int chunk;                          // alphas per pass, as in the single-layer search
};

// alphas per pass of the block search: the cache budget's count, but at
// least enough that the down projection's loss GEMM (its tiles times the
// pass's alphas) gives every CU two workgroups
#ifndef AWQ_MLP_MIN_CHUNK
#define AWQ_MLP_MIN_CHUNK 0
#endif
int mlp_chunk(int T, int K, int I, int K_out, int n_alpha) {
    const int budget = alpha_chunk((size_t)2 * I * K * sizeof(_Float16), n_alpha);
    const int tiles = (int)loss_gemm_tiles(T, K_out);
    int fill = (2 * device_cu_count() + tiles - 1) / tiles;
    if (AWQ_MLP_MIN_CHUNK > 0) fill = AWQ_MLP_MIN_CHUNK;
    return min(n_alpha, max(budget, fill));
}

MlpLayout mlp_layout(int T, int K, int I, int K_out, int n_alpha) {
    MlpLayout L;
    const size_t d_alpha = (size_t)2 * I * K * sizeof(_Float16);
    L.chunk = mlp_chunk(T, K, I, K_out, n_alpha);
    size_t off = 0;
    L.sx = off;   off += align256((size_t)K * sizeof(float));
    L.sall = off; off += align256((size_t)n_alpha * K * sizeof(float));
    L.sinv = off; off += align256((size_t)n_alpha * K * sizeof(float));
    L.D = off;    off += align256((size_t)L.chunk * d_alpha);
    L.wt = off;   off += align256((size_t)2 * I * K * sizeof(_Float16));
    L.wdt = off;  off += align256(loss_rows(K_out) * (size_t)I * sizeof(_Float16));
    L.ref = off;  off += align256((size_t)3 * T * I * sizeof(float));
    L.dh = off;   off += align256((size_t)L.chunk * T * I * sizeof(_Float16));
    L.part = off; off += align256((size_t)n_alpha * loss_gemm_tiles(T, K_out) * sizeof(double));
    L.total = off;
    return L;
}
}  // namespace

size_t search_mlp_workspace_bytes(int T, int K, int I, int K_out, int n_alpha) {
    return mlp_layout(T, K, I, K_out, n_alpha).total;
}

// The gate/up pair's shared scale searched on the MLP block's output:
//   D_a      = [Wg; Wu] - w_hat_a / s_a            (k_quant_err, both layers)
//   g, u, h  = X Wg^T, X Wu^T, SiLU(g) u            (once, fp32)
//   dh_a     = fp16(SiLU(g - X Dg_a^T) (u - X Du_a^T) - h)
//   L_a      = sum (dh_a Wd^T)^2 / (T K_out)          (the loss GEMM on dh_a, Wd)
// The change of the block's output is formed from the fp32 quantization error
// of g and u (a difference of fp16-rounded block outputs would lose it).
int launch_search_mlp(const void* Wg, const void* Wu, const void* Wd, int K_out, const void* X_cal, int T,
                      int K, int I, const float* alphas, int n_alpha, int bits, int group_size,
                      int zero_point, float* s_out, float* loss_out, int* best_out, void* workspace,
                      hipStream_t st) {
    const MlpLayout L = mlp_layout(T, K, I, K_out, n_alpha);
    char* ws = static_cast<char*>(workspace);
    float* s_x = reinterpret_cast<float*>(ws + L.sx);
    float* s_all = reinterpret_cast<float*>(ws + L.sall);
    float* s_inv = reinterpret_cast<float*>(ws + L.sinv);
    _Float16* D = reinterpret_cast<_Float16*>(ws + L.D);
    _Float16* wt = reinterpret_cast<_Float16*>(ws + L.wt);
    _Float16* wdt = reinterpret_cast<_Float16*>(ws + L.wdt);
    float* ref = reinterpret_cast<float*>(ws + L.ref);
    _Float16* dh = reinterpret_cast<_Float16*>(ws + L.dh);
    double* part = reinterpret_cast<double*>(ws + L.part);
    const int N = 2 * I;

    AlphaGrid grid{};
    for (int i = 0; i < n_alpha; ++i) grid.a[i] = alphas[i];
    hipLaunchKernelGGL(k_act_stat, dim3(K / 64), dim3(1024), 0, st, (const _Float16*)X_cal, T, K, s_x);
    const long long nsk = (long long)n_alpha * K;
    hipLaunchKernelGGL(k_candidate_scales, dim3((unsigned)((nsk + 255) / 256)), dim3(256), 0, st,
                       s_x, K, grid, n_alpha, s_all, s_inv);

    LayerList pair{};
    pair.w[0] = static_cast<const uint4*>(Wg);
    pair.w[1] = static_cast<const uint4*>(Wu);
    pair.cstart[0] = 0;
    pair.cstart[1] = (long long)I * (K / 8);
    pair.n = 2;
    auto qerr = group_size == 64 ? pick_quant_err<64>(bits, zero_point) : pick_quant_err<128>(bits, zero_point);
    hipLaunchKernelGGL(k_tile_rows, dim3((unsigned)((size_t)N / 16 * (K / kGroup))), dim3(256), 0, st, pair, N,
                       K, (uint4*)wt);
    LayerList down{};
    down.w[0] = static_cast<const uint4*>(Wd);
    down.n = 1;
    hipLaunchKernelGGL(k_tile_rows, dim3((unsigned)(loss_rows(K_out) / 16 * (I / kGroup))), dim3(256), 0, st,
                       down, K_out, I, (uint4*)wdt);
    int err = (int)hipGetLastError();
    if (err) return err;
    if ((err = launch_mlp_gemm(X_cal, wt, 0, T, I, K, 1, true, ref, nullptr, st))) return err;
    const size_t n_tiles = loss_gemm_tiles(T, K_out);
    for (int a0 = 0; a0 < n_alpha; a0 += L.chunk) {
        const int na = min(L.chunk, n_alpha - a0);
        hipLaunchKernelGGL(qerr, dim3((unsigned)((size_t)N / 16 * (K / kGroup))), dim3(256), 0, st, pair,
                           (const float*)s_all + (size_t)a0 * K, (const float*)s_inv + (size_t)a0 * K, N, K, na,
                           (long long)N * K / 8, (uint4*)D);
        if ((err = (int)hipGetLastError())) return err;
        if ((err = launch_mlp_gemm(X_cal, D, (long long)N * K, T, I, K, na, false, ref, dh, st))) return err;
        if ((err = launch_loss_gemm(dh, (long long)T * I, wdt, 0, T, K_out, I, na, part + (size_t)a0 * n_tiles,
                                    st)))
            return err;
    }
    hipLaunchKernelGGL(k_select, dim3(1), dim3(256), 0, st, part, (int)loss_gemm_tiles(T, K_out), n_alpha,
                       1.0 / ((double)T * (double)K_out), s_all, K, s_out, loss_out, best_out);
    return (int)hipGetLastError();
}

}  // namespace awq
