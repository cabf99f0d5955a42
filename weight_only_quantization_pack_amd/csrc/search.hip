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
#include <type_traits>

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
// alpha into the workspace plus a dense loss GEMM (needs one chunk of alphas'
// D, N rounded up to 16), or one fused kernel forming D in registers (a
// workspace of under a megabyte).  MI355X, 4096 x 4096, T = 512, 20 alphas:
// 0.52-0.54 ms and 0.65-0.66 ms.  The fused kernel's workgroup takes 512
// calibration rows and 64 rows of W, so every D value is formed once per
// alpha, by two waves of one SIMD that each form half of it while the other's
// MFMAs run.
constexpr int kFusedT = 512;            // calibration rows per workgroup of the fused loss
constexpr int kFusedNT = 1;             // 16-row tiles of W per wave
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
    // four rows' loads in flight before their sums (rows past T load nothing)
    for (int t0 = r; t0 < T; t0 += 4 * 128) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = t0 + 128 * u;
            v[u] = t < T ? *reinterpret_cast<const uint4*>(X + (size_t)t * K + k0) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const _Float16* h = reinterpret_cast<const _Float16*>(&v[u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) sum[e] += fabs((double)h[e]);
        }
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
// workgroup of 8 waves owns 64 rows of W (four 16-row MFMA B tiles) and up to
// 512 calibration rows for one alpha.  Wave w takes tile w & 3 against
// calibration rows 256 (w >> 2) .. + 255; the two waves of a tile (w and
// w + 4, on one SIMD when the CU deals a workgroup's waves to its SIMDs
// round-robin; correctness does not depend on it) each form the D fragments
// of half the group's columns (k 64 (w >> 2)
// .. + 63) in registers in the B-operand layout of v_mfma_f32_16x16x32_f16
// (lane (j, q) holds row j's k = 32 s + 8 q + e of substep s), meeting its
// partner through LDS for the group's min and max (128-wide groups) and for the
// other half of the fragments.  The codes are those of quant_codes_b2, exactly
// as the separate error kernel forms them.  The kernel is software-pipelined
// by one group: while a wave runs the 64 MFMAs of group g it forms its half of
// D for group g + 1, in slices of VALU work placed behind each 4 MFMAs, and the
// other wave of the SIMD fills the issue slots that one wave leaves.  X streams
// through LDS in 64-k steps (512 rows x 128 B, two buffers, direct-to-LDS
// buffer loads with the step's offset in the scalar operand, chunk p of row r
// holding global chunk p ^ (r & 7), which the A-fragment reads see free of bank
// conflicts on MI355X); W rows are loaded two groups ahead into registers, s
// and 1/s one group ahead into an LDS slot.  The epilogue squares and sums the
// outputs of rows < T and columns < N in fp32 per lane, then in fp64 in a
// fixed order, into one partial per workgroup.
namespace lf {
constexpr int kT = kFusedT;             // calibration rows per workgroup
constexpr int kWaves = 8;
constexpr int kFR = kT / 2 / 16;        // X fragments per wave and substep (16)
constexpr int kStepK = 64;              // k per LDS step (half a group)
constexpr int kRow = kStepK * 2;        // bytes of one X row in LDS
constexpr int kBuf = kT * kRow;         // 64 KB per buffer
constexpr int kNBuf = 2;
constexpr int kXLoads = kBuf / 1024 / kWaves;   // direct-to-LDS loads per wave and step (8)
constexpr int kWLoads = 2;              // W loads per wave and group
constexpr int kUnits = 2 * kFR / 4;     // units of 4 MFMAs per LDS step (8)
constexpr int kSBytes = 2 * 256 * 4;    // two slots of s and 1/s
constexpr int kRedBytes = kWaves * 16 * 2 * 4;      // [wave][row][min, max]
constexpr int kDxBytes = kWaves * 2 * 64 * 16;      // [wave][substep][lane] half8
constexpr int kLds = kSBytes + kRedBytes + kDxBytes + kNBuf * kBuf;
static_assert(kFusedNT == 1 && kFusedRows == 64, "four 16-row tiles per workgroup");
}

struct RowList {                        // rows of the layers searched together
    const _Float16* w[kMaxSearchLayers];
    int nstart[kMaxSearchLayers];
    int n;
};

template <int Q, bool ZP, int GS>
__global__ __launch_bounds__(512, 1) void k_loss_fused(RowList layers, const _Float16* __restrict__ X,
                                                       int T, int N, int K,
                                                       const float* __restrict__ s_all,
                                                       const float* __restrict__ s_inv,
                                                       double* __restrict__ partials) {
    static_assert(GS == 128 || GS == 64, "128- or 64-wide groups");
    // the small arrays first (within reach of a DS instruction's 16-bit offset
    // from one base), then the X buffers
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    float* const Ss = reinterpret_cast<float*>(lds);                               // [2 slots][s 128, 1/s 128]
    float* const Red = reinterpret_cast<float*>(lds + lf::kSBytes);                 // [wave][row][2]
    unsigned char* const Dx = lds + lf::kSBytes + lf::kRedBytes;                    // [wave][substep][lane]
    unsigned char* const Xs = lds + lf::kSBytes + lf::kRedBytes + lf::kDxBytes;     // kNBuf x lf::kBuf
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = wave & 3;                      // W tile
    const int j = lane & 15, hq = lane >> 4;
    // Workgroup L -> (unit, alpha), unit = calibration block * row blocks + row
    // block.  Workgroups go to the XCDs round-robin (L mod 8), so each run of
    // 8 A consecutive workgroups gives XCD x all A alphas of unit 8 c + x: the
    // workgroups that run together on one XCD share their W rows in its L2.
    // Units past the last whole run of 8 take the alphas in the plain order.
    const int nblk = (N + kFusedRows - 1) / kFusedRows;
    const int U = nblk * ((T + lf::kT - 1) / lf::kT);
    const int A = (int)gridDim.x / U;
    const int full = U / 8 * 8;
    const int L = blockIdx.x;
    int unit, alpha;
    if (L < full * A) {
        const int r = L % (8 * A);
        unit = L / (8 * A) * 8 + r % 8;
        alpha = r / 8;
    } else {
        const int Lt = L - full * A, rem = U - full;
        unit = full + Lt % rem;
        alpha = Lt / rem;
    }
    const int t0 = unit / nblk * lf::kT;
    const int G = K / kGroup;
    const int n_base = unit % nblk * kFusedRows + tile * 16;
    // X: load q (0..kXLoads-1) of wave w fills rows 8 (kXLoads w + q) .. + 7 of
    // the buffer, lane l row + (l >> 3) at position l & 7, which holds chunk
    // (l & 7) ^ (l >> 3) of the row (chunk p of row r at position p ^ (r & 7),
    // which the A-fragment reads see free of bank conflicts).  Byte offsets
    // within X (T K < 2^31 halves, checked by the caller): the lane's part in
    // the vector operand, the load's rows and the step's k in the scalar one.
    // Rows past T fall outside the buffer (zero, no memory access) and their
    // outputs are never summed.
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(X), (short)0, (int)((uint32_t)T * (uint32_t)K * 2u), 0x00020000);
    const uint32_t x_voff = 2u * (uint32_t)K * (uint32_t)(t0 + 8 * lf::kXLoads * wave + (lane >> 3))
                          + 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
    // (past the last step it loads the last step again into the buffer the
    // step would take, which nothing reads: a uniform load stream)
    auto issue_x = [&](int step) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)min(step, 2 * G - 1) * (uint32_t)lf::kRow;
        unsigned char* const buf = Xs + (step & (lf::kNBuf - 1)) * lf::kBuf;
#pragma unroll
        for (int q = 0; q < lf::kXLoads; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(buf + (lf::kXLoads * wave + q) * 1024),
                                                     16, x_voff, soff + (uint32_t)q * 16u * (uint32_t)K, 0, 0);
    };
    // s and 1/s of a group go to LDS (two slots), written by wave 0 with one
    // direct-to-LDS load (lanes 0..31 the 128 s values, lanes 32..63 the 128
    // reciprocals) and read by every wave while it forms D
    auto issue_s = [&](int g, int slot) __attribute__((always_inline)) {
        if (wave != 0) return;                       // wave-uniform
        const int k0 = kGroup * min(g, G - 1);
        const float* src = (lane < 32 ? s_all : s_inv) + (size_t)alpha * K + k0 + 4 * (lane & 31);
        __builtin_amdgcn_global_load_lds((global_void_t*)src, (lds_void_t*)(Ss + slot * 256), 16, 0, 0);
    };
    // weight e of a lane's 8 (the packed words stay 32-bit registers)
    auto wword = [](const uint4& raw, int e) __attribute__((always_inline)) {
        return e / 2 == 0 ? raw.x : e / 2 == 1 ? raw.y : e / 2 == 2 ? raw.z : raw.w;
    };
    auto whalf = [](uint32_t word, int e) __attribute__((always_inline)) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)((e & 1) ? (word >> 16) : (word & 0xFFFFu)));
    };
    auto wval = [&](const uint4& raw, int e) __attribute__((always_inline)) { return whalf(wword(raw, e), e); };

    // this wave's half of W of a group in registers: value i = 8 ls + e of a
    // lane is k = 64 th + 32 ls + 8 q + e
    struct PreW { uint4 w[2]; };
    // This wave's half of one group's D, formed in slices: 16 values per lane,
    // value i = 8 ls + e (one 64-group for 64-wide groups; half of one
    // 128-group, whose min and max meet the partner wave's through LDS).
    struct MakeD {
        float v[16];
        float mn, mx;
        GroupParams gp;
        uint32_t Tc[16];
        uint32_t fmin;
        float4 r0, r1;
        half8_t d[2];
    };
    float4_t acc[lf::kFR];
#pragma unroll
    for (int i = 0; i < lf::kFR; ++i) acc[i] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // The rest depends on the wave's calibration half th = wave >> 2 (also the
    // half of D's columns it forms), a compile-time constant in each copy.
    auto run = [&](auto th_c) __attribute__((always_inline)) {
        constexpr int TH = decltype(th_c)::value;
        // this lane's W row (rows past N: row N - 1, never summed), from its half of the group
        const _Float16* wrow;
        {
            const int n = min(n_base + j, N - 1);
            int l = 0;
#pragma unroll
            for (int m = 1; m < kMaxSearchLayers; ++m)
                if (m < layers.n && n >= layers.nstart[m]) l = m;
            wrow = layers.w[l] + (size_t)(n - layers.nstart[l]) * K + 64 * TH + 8 * hq;
        }
        auto issue_w = [&](int g, PreW& p) __attribute__((always_inline)) {
            const int k0 = kGroup * min(g, G - 1);
#pragma unroll
            for (int ls = 0; ls < 2; ++ls)
                p.w[ls] = *reinterpret_cast<const uint4*>(wrow + k0 + 32 * ls);
        };
        // s (or 1/s, at +128) of value i of this lane in slot `slot`
        const float* const s_lane = Ss + 64 * TH + 8 * hq;
        auto s_at = [&](int slot, int i) __attribute__((always_inline)) {
            return s_lane + slot * 256 + 32 * (i / 8) + (i % 8);
        };
        // v = w * s for the 8 values of local substep ls; running min and max
        auto slice_scale = [&](MakeD& st, const PreW& pw, int slot, int ls) __attribute__((always_inline)) {
            const float4 s0 = *reinterpret_cast<const float4*>(s_at(slot, 8 * ls));
            const float4 s1 = *reinterpret_cast<const float4*>(s_at(slot, 8 * ls + 4));
            const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            float mn = 0.0f, mx = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = wval(pw.w[ls], e) * sv[e];
                st.v[8 * ls + e] = v;
                mn = e == 0 ? v : fminf(mn, v);
                mx = e == 0 ? v : fmaxf(mx, v);
            }
            if (ls == 0) { st.mn = mn; st.mx = mx; }
            else { st.mn = fminf(st.mn, mn); st.mx = fmaxf(st.mx, mx); }
        };
        // the row's other values of this half sit in the lanes of the same row j
        auto slice_rowminmax = [&](MakeD& st) __attribute__((always_inline)) {
            st.mn = fminf(st.mn, __shfl_xor(st.mn, 16)); st.mx = fmaxf(st.mx, __shfl_xor(st.mx, 16));
            st.mn = fminf(st.mn, __shfl_xor(st.mn, 32)); st.mx = fmaxf(st.mx, __shfl_xor(st.mx, 32));
        };
        auto slice_params = [&](MakeD& st) __attribute__((always_inline)) {
            st.gp = group_params<Q, ZP>(st.mn, st.mx);
            st.fmin = 0xFFFFu;
        };
        // fixed-point codes of values 4c .. 4c + 3 (quant_codes_b2's fast path)
        auto slice_codes = [&](MakeD& st, int c) __attribute__((always_inline)) {
            const float zb = st.gp.zero + (128.5f + 0x3p-16f);   // exact: z <= 15
#pragma unroll
            for (int i = 4 * c; i < 4 * c + 4; ++i) {
                const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(st.v[i], st.gp.rd, zb), 128.25f, 128.5f + Q);
                st.Tc[i] = __builtin_bit_cast(uint32_t, t);
                st.fmin = min(st.fmin, st.Tc[i] & 0xFFFFu);
            }
        };
        // a group whose fraction came too close to a rounding boundary takes
        // quant_code's division (quant_codes_b2's fallback), on v = w * s formed
        // again exactly as slice_scale formed it
        auto slice_fallback = [&](MakeD& st, const PreW& pw, int slot) __attribute__((always_inline)) {
            const bool near = st.fmin <= 5u;
            if (__builtin_amdgcn_ballot_w64(near)) {
                if (near) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        st.Tc[i] = quant_code<Q>(wval(pw.w[i / 8], i % 8) * *s_at(slot, i), st.gp) << 16;
                }
            }
        };
        // D of values 4c .. 4c + 3: w - w_hat * (1/s)
        auto slice_d = [&](MakeD& st, const PreW& pw, int slot, int c) __attribute__((always_inline)) {
            const int ls = c / 2;
            if (c % 2 == 0) {
                st.r0 = *reinterpret_cast<const float4*>(s_at(slot, 8 * ls) + 128);
                st.r1 = *reinterpret_cast<const float4*>(s_at(slot, 8 * ls + 4) + 128);
            }
            const float zd = -(st.gp.zero * st.gp.delta);   // exact: z <= 16, Delta an fp16 value
#pragma unroll
            for (int i = 4 * c; i < 4 * c + 4; ++i) {
                const int e = i % 8;
                const float qf = (float)((st.Tc[i] >> 16) & 0xFFu);
                const float w_hat = __builtin_fmaf(qf, st.gp.delta, zd);   // (q - z) * Delta, exact
                const float r = e == 0 ? st.r0.x : e == 1 ? st.r0.y : e == 2 ? st.r0.z : e == 3 ? st.r0.w
                              : e == 4 ? st.r1.x : e == 5 ? st.r1.y : e == 6 ? st.r1.z : st.r1.w;
                // w converted again here (an opaque copy of its packed pair keeps
                // the compiler from holding the fp32 weights across the group)
                uint32_t pair = wword(pw.w[ls], e);
                asm volatile("" : "+v"(pair));
                st.d[ls][e] = (_Float16)(whalf(pair, e) - w_hat * r);
            }
        };
        // the partner wave's half of the min and max (128-wide groups)
        auto put_red = [&](const MakeD& st) __attribute__((always_inline)) {
            if (hq == 0) {
                Red[(wave * 16 + j) * 2] = st.mn;
                Red[(wave * 16 + j) * 2 + 1] = st.mx;
            }
        };
        auto get_red = [&](MakeD& st) __attribute__((always_inline)) {
            const float2 o = *reinterpret_cast<const float2*>(Red + ((wave ^ 4) * 16 + j) * 2);
            st.mn = fminf(st.mn, o.x);
            st.mx = fmaxf(st.mx, o.y);
        };
        auto put_d = [&](const MakeD& st) __attribute__((always_inline)) {
#pragma unroll
            for (int ls = 0; ls < 2; ++ls)
                *reinterpret_cast<half8_t*>(Dx + ((wave * 2 + ls) * 64 + lane) * 16) = st.d[ls];
        };
        // slice u (0..15) of one group's D, behind unit u of the group; the
        // group's middle barrier separates units 7 and 8
        auto slice = [&](MakeD& st, const PreW& pw, int slot, int u) __attribute__((always_inline)) {
            if constexpr (GS == 128) {
                if (u < 2) slice_scale(st, pw, slot, u);
                else if (u == 2) { slice_rowminmax(st); put_red(st); }
                else if (u == 8) { get_red(st); slice_params(st); }
                else if (u >= 9 && u < 13) slice_codes(st, u - 9);
                else if (u == 13) { slice_fallback(st, pw, slot); slice_d(st, pw, slot, 0); }
                else if (u == 14) { slice_d(st, pw, slot, 1); slice_d(st, pw, slot, 2); }
                else if (u == 15) { slice_d(st, pw, slot, 3); put_d(st); }
            } else {
                if (u < 2) slice_scale(st, pw, slot, u);
                else if (u == 2) { slice_rowminmax(st); slice_params(st); }
                else if (u >= 3 && u < 7) slice_codes(st, u - 3);
                else if (u == 7) slice_fallback(st, pw, slot);
                else if (u >= 8 && u < 12) slice_d(st, pw, slot, u - 8);
                else if (u == 15) put_d(st);
            }
        };
        // the complete D fragments of a group: this wave's half from its own
        // registers, the partner's from LDS
        auto take_d = [&](const MakeD& st, half8_t* dcur) __attribute__((always_inline)) {
#pragma unroll
            for (int ls = 0; ls < 2; ++ls) {
                dcur[2 * TH + ls] = st.d[ls];
                dcur[2 * (TH ^ 1) + ls] = *reinterpret_cast<const half8_t*>(Dx + (((wave ^ 4) * 2 + ls) * 64 + lane) * 16);
            }
        };

        // A-fragment reads: lane (j, q) takes chunk 4 sub + q of row 256 TH + 16 i + j
        // (substep sub of the LDS step), at position (4 sub + q) ^ (j & 7)
        const uint32_t x_lane0 = (uint32_t)(256 * TH + j) * lf::kRow + 16u * (uint32_t)(hq ^ (j & 7));
        const uint32_t x_lane1 = (uint32_t)(256 * TH + j) * lf::kRow + 16u * (uint32_t)((4 + hq) ^ (j & 7));
        auto read_unit = [&](const unsigned char* buf, int u, half8_t* xf) __attribute__((always_inline)) {
            const int sub = u / (lf::kFR / 4), i0 = 4 * (u % (lf::kFR / 4));
            const unsigned char* const b = buf + (sub ? x_lane1 : x_lane0);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                xf[v] = *reinterpret_cast<const half8_t*>(b + (i0 + v) * 16 * lf::kRow);
        };
        // one LDS step (half h of a group): 8 units of 4 X fragments and 4
        // MFMAs, the fragments of unit u + 1 read under unit u's MFMAs, one
        // slice of the next group's D behind each unit
        auto step = [&](int h, const half8_t* dcur, MakeD& st, const PreW& pwn, int slot_n) __attribute__((always_inline)) {
            const unsigned char* const buf = Xs + h * lf::kBuf;      // step 2 g + h uses buffer h
            half8_t xa[4], xb[4];
            read_unit(buf, 0, xa);
#pragma unroll
            for (int u = 0; u < lf::kUnits; ++u) {
                half8_t* cur = (u & 1) ? xb : xa;
                half8_t* nxt = (u & 1) ? xa : xb;
                if (u + 1 < lf::kUnits) read_unit(buf, u + 1, nxt);
                const int sub = u / (lf::kFR / 4), i0 = 4 * (u % (lf::kFR / 4));
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[i0 + v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dcur[2 * h + sub], cur[v], acc[i0 + v], 0, 0, 0);
                slice(st, pwn, slot_n, lf::kUnits * h + u);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        PreW pw[2];
        half8_t dcur[4];                // D fragments of the group whose MFMAs run: [substep]
        MakeD st;

        // prologue: X(0), W(0), W(1), s(0), s(1) land; D(0) formed in full
        issue_x(0);
        issue_w(0, pw[0]);
        issue_w(1, pw[1]);
        issue_s(0, 0);
        issue_s(1, 1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int u = 8 * m; u < 8 * m + 8; ++u) slice(st, pw[0], 0, u);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        take_d(st, dcur);
        __builtin_amdgcn_sched_barrier(0);

        // group g: MFMAs on D(g) (dcur) while this wave's half of D(g + 1) is
        // formed from W(g + 1) (pw[1]) and s(g + 1) (slot (g + 1) & 1); W(g + 2)
        // loads into pw[0], s(g + 2) into slot g & 1
        for (int g = 0; g < G; ++g) {
            const int slot_n = (g + 1) & 1;
            // step 2g, buffer 0: X(2g) has landed, as have W(g + 1) and s(g + 1)
            issue_x(2 * g + 1);
            issue_w(g + 2, pw[0]);               // clamped past the last group: a uniform load stream
            __builtin_amdgcn_sched_barrier(0);
            step(0, dcur, st, pw[1], slot_n);
            // step 2g + 1, buffer 1: X(2g + 1) has landed once at most the W
            // loads are outstanding; every wave is done with buffer 0 and slot
            // g & 1, and the min and max of the partner's half are in LDS
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(lf::kWLoads));
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            issue_x(2 * g + 2);
            issue_s(g + 2, g & 1);
            __builtin_amdgcn_sched_barrier(0);
            step(1, dcur, st, pw[1], slot_n);
            // every wave's half of D(g + 1) is in LDS, X(2g + 2) has landed
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            take_d(st, dcur);
            pw[1] = pw[0];
        }

        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < lf::kFR; ++i) {
            const bool t_ok = t0 + 256 * TH + 16 * i + j < T;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = t_ok && n_base + 4 * hq + r < N;
                sq = __builtin_fmaf(ok ? acc[i][r] : 0.0f, ok ? acc[i][r] : 0.0f, sq);
            }
        }
        return sq;
    };
    const float sq = (wave >> 2) == 0 ? run(std::integral_constant<int, 0>{}) : run(std::integral_constant<int, 1>{});

    double dsq = (double)sq;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dsq += __shfl_xor(dsq, off);
    __shared__ double wsum[lf::kWaves];
    if (lane == 0) wsum[wave] = dsq;
    __syncthreads();
    if (tid == 0) {
        double tot = wsum[0];
#pragma unroll
        for (int w = 1; w < lf::kWaves; ++w) tot += wsum[w];
        partials[(size_t)alpha * U + unit] = tot;
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
    // wave w sums alphas w, w + 4, ..., four of them at a time so that their
    // loads are in flight together (each alpha's order as one at a time)
    for (int a0 = wave; a0 < n_alpha; a0 += 16) {
        double s[4] = {0.0, 0.0, 0.0, 0.0};
        for (int j = lane; j < n_tiles; j += 64) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int a = a0 + 4 * u;
                if (a < n_alpha) s[u] += partials[(size_t)a * n_tiles + j];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) s[u] += __shfl_xor(s[u], off);
            if (lane == 0 && a0 + 4 * u < n_alpha) loss[a0 + 4 * u] = s[u] * inv_count;
        }
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
    for (int k0 = tid; k0 < K; k0 += 8 * (int)blockDim.x) {     // eight loads in flight
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = k0 + u * (int)blockDim.x;
            v[u] = k < K ? sb[k] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = k0 + u * (int)blockDim.x;
            if (k < K) s_out[k] = v[u];
        }
    }
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
        const int lds = lf::kLds;
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return (int)e;
        const dim3 grid_f((unsigned)(fused_tiles(T, N) * (size_t)n_alpha));
        hipLaunchKernelGGL(kern, grid_f, dim3(64 * lf::kWaves), lds, st, rows, (const _Float16*)X_cal, T, N, K,
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
