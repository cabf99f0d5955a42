// C ABI of libawq: argument validation on the host, then dispatch to the
// kernel launchers.  Nothing here touches the GPU before every argument has
// been checked, so invalid calls never launch and never write an output.
#include "awq_internal.h"

#include <mutex>

namespace {

constexpr int kMaxGemvM = 16;
constexpr int kMaxT = 8192;        // exact fp64 |x| sums need T < 2^13
constexpr int kMaxAlpha = 64;

int check_ptr(const void* p) {
    if (p == nullptr) return AWQ_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(p) & 15u) return AWQ_ERR_ALIGN;
    return AWQ_OK;
}

// First non-OK status of a list of required pointers; NULL errors are
// reported before alignment errors.
int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps) if (p == nullptr) return AWQ_ERR_NULL;
    for (const void* p : ps) if (check_ptr(p) != AWQ_OK) return AWQ_ERR_ALIGN;
    return AWQ_OK;
}

int check_quant_params(int bits, int group_size, int zero_point) {
    if (bits != 3 && bits != 4) return AWQ_ERR_UNSUPPORTED;
    if (group_size != 128 && group_size != 64) return AWQ_ERR_UNSUPPORTED;
    if (zero_point != 0 && zero_point != 1) return AWQ_ERR_UNSUPPORTED;
    return AWQ_OK;
}

int check_nk(int N, int K) {
    if (N < 0 || K <= 0) return AWQ_ERR_SHAPE;
    if (K % awq::kGroup != 0) return AWQ_ERR_SHAPE;
    return AWQ_OK;
}

awq_status hip_status(int err) { return err == 0 ? AWQ_OK : AWQ_ERR_HIP; }

// the checks above return awq_status values as int
awq_status as_status(int st) { return static_cast<awq_status>(st); }
static_assert(sizeof(awq_status) == sizeof(int), "awq_status is passed as a C int");

}  // namespace

extern "C" {

const char* awq_status_str(awq_status status) {
    switch (status) {
        case AWQ_OK: return "AWQ_OK";
        case AWQ_ERR_NULL: return "AWQ_ERR_NULL";
        case AWQ_ERR_SHAPE: return "AWQ_ERR_SHAPE";
        case AWQ_ERR_UNSUPPORTED: return "AWQ_ERR_UNSUPPORTED";
        case AWQ_ERR_ALIGN: return "AWQ_ERR_ALIGN";
        case AWQ_ERR_WORKSPACE: return "AWQ_ERR_WORKSPACE";
        case AWQ_ERR_HIP: return "AWQ_ERR_HIP";
        default: return "AWQ_ERR_UNKNOWN";
    }
}

int awq_pack_format_version(void) { return 3; }

size_t awq_packed_words_per_row(int K, int bits) {
    if (K <= 0) return 0;
    if (bits == 4) return (size_t)K / 8;
    if (bits == 3) return 3 * ((size_t)K / 32);
    return 0;
}

size_t awq_packed_words(int N, int K, int bits) {
    if (N < 0) return 0;
    return 16 * (((size_t)N + 15) / 16) * awq_packed_words_per_row(K, bits);
}

awq_status awq_quantize_pack(const void* W, const float* s, int N, int K, int bits, int group_size,
                      int zero_point, void* qweight, void* scales, void* zeros, hipStream_t stream) {
    int st = check_quant_params(bits, group_size, zero_point);
    if (st) return as_status(st);
    if ((st = check_nk(N, K))) return as_status(st);
    if (N == 0) return AWQ_OK;
    if ((st = check_ptrs({W, qweight, scales, zeros}))) return as_status(st);
    if (s != nullptr && (st = check_ptr(s))) return as_status(st);
    return hip_status(awq::launch_quantize_pack(W, s, N, K, bits, group_size, zero_point, qweight, scales, zeros,
                                                stream));
}

awq_status awq_dequantize(const void* qweight, const void* scales, const void* zeros, void* W_hat, int N,
                   int K, int bits, int group_size, hipStream_t stream) {
    int st = check_quant_params(bits, group_size, 1);
    if (st) return as_status(st);
    if ((st = check_nk(N, K))) return as_status(st);
    if ((long long)N * K >= (1LL << 40)) return AWQ_ERR_SHAPE;
    if (N == 0) return AWQ_OK;
    if ((st = check_ptrs({qweight, scales, zeros, W_hat}))) return as_status(st);
    return hip_status(awq::launch_dequantize(qweight, scales, zeros, W_hat, N, K, bits, group_size,
                                             stream));
}

awq_status awq_scale_activations(const void* x, const float* s, void* x_out, int M, int K, hipStream_t stream) {
    if (M < 0 || K <= 0 || K % awq::kGroup != 0) return AWQ_ERR_SHAPE;
    if (M == 0) return AWQ_OK;
    int st = check_ptrs({x, s, x_out});
    if (st) return as_status(st);
    return hip_status(awq::launch_scale_activations(x, s, x_out, M, K, stream));
}

size_t awq_search_workspace_bytes(int T, int N, int K, int n_alpha) {
    if (T <= 0 || N <= 0 || K <= 0 || n_alpha <= 0) return 0;
    return awq::search_workspace_bytes(T, N, K, n_alpha, false);
}

size_t awq_search_workspace_bytes_fused(int T, int N, int K, int n_alpha) {
    if (T <= 0 || N <= 0 || K <= 0 || n_alpha <= 0) return 0;
    return awq::search_workspace_bytes(T, N, K, n_alpha, true);
}

namespace {
// the search path a workspace of this size takes: 0 = D buffered (the
// default), 1 = fused loss, -1 = too small for either
int search_path(int T, int N, int K, int n_alpha, size_t workspace_bytes) {
    if (workspace_bytes >= awq::search_workspace_bytes(T, N, K, n_alpha, false)) return 0;
    if (workspace_bytes >= awq::search_workspace_bytes(T, N, K, n_alpha, true)) return 1;
    return -1;
}
}  // namespace

awq_status awq_search_scale(const void* W, const void* X_cal, int T, int N, int K, const float* alphas,
                     int n_alpha, int bits, int group_size, int zero_point, float* s_out,
                     float* loss_out, int* best_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    int st = check_quant_params(bits, group_size, zero_point);
    if (st) return as_status(st);
    if (n_alpha < 1 || n_alpha > kMaxAlpha) return AWQ_ERR_UNSUPPORTED;
    if (T > kMaxT) return AWQ_ERR_UNSUPPORTED;
    if (T <= 0 || N <= 0) return AWQ_ERR_SHAPE;
    if ((st = check_nk(N, K))) return as_status(st);
    if ((long long)T * K >= (1LL << 31)) return AWQ_ERR_SHAPE;   // 32-bit offsets into X_cal
    if (alphas == nullptr) return AWQ_ERR_NULL;
    if ((st = check_ptrs({W, X_cal, s_out, workspace}))) return as_status(st);
    if (loss_out != nullptr && (st = check_ptr(loss_out))) return as_status(st);
    if (best_out != nullptr && (st = check_ptr(best_out))) return as_status(st);
    const int path = search_path(T, N, K, n_alpha, workspace_bytes);
    if (path < 0) return AWQ_ERR_WORKSPACE;
    return hip_status(awq::launch_search(&W, &N, 1, X_cal, T, K, alphas, n_alpha, bits, group_size,
                                         zero_point, s_out, loss_out, best_out, workspace,
                                         path == 1, stream));
}

awq_status awq_search_scale_shared(const void* const* Ws, const int* Ns, int n_layers, const void* X_cal,
                            int T, int K, const float* alphas, int n_alpha, int bits, int group_size,
                            int zero_point, float* s_out, float* loss_out, int* best_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_quant_params(bits, group_size, zero_point);
    if (st) return as_status(st);
    if (n_alpha < 1 || n_alpha > kMaxAlpha) return AWQ_ERR_UNSUPPORTED;
    if (n_layers < 1 || n_layers > awq::kMaxSearchLayers) return AWQ_ERR_UNSUPPORTED;
    if (T > kMaxT) return AWQ_ERR_UNSUPPORTED;
    if (Ws == nullptr || Ns == nullptr || alphas == nullptr) return AWQ_ERR_NULL;
    long long N = 0;
    for (int l = 0; l < n_layers; ++l) {
        if (Ns[l] <= 0) return AWQ_ERR_SHAPE;
        N += Ns[l];
    }
    if (T <= 0 || N > (1LL << 30)) return AWQ_ERR_SHAPE;
    if ((st = check_nk((int)N, K))) return as_status(st);
    if ((long long)T * K >= (1LL << 31)) return AWQ_ERR_SHAPE;   // 32-bit offsets into X_cal
    for (int l = 0; l < n_layers; ++l)
        if (Ws[l] == nullptr) return AWQ_ERR_NULL;
    if ((st = check_ptrs({X_cal, s_out, workspace}))) return as_status(st);
    for (int l = 0; l < n_layers; ++l)
        if ((st = check_ptr(Ws[l]))) return as_status(st);
    if (loss_out != nullptr && (st = check_ptr(loss_out))) return as_status(st);
    if (best_out != nullptr && (st = check_ptr(best_out))) return as_status(st);
    const int path = search_path(T, (int)N, K, n_alpha, workspace_bytes);
    if (path < 0) return AWQ_ERR_WORKSPACE;
    return hip_status(awq::launch_search(Ws, Ns, n_layers, X_cal, T, K, alphas, n_alpha, bits,
                                         group_size, zero_point, s_out, loss_out, best_out,
                                         workspace, path == 1, stream));
}

size_t awq_search_mlp_workspace_bytes(int T, int K, int I, int K_out, int n_alpha) {
    if (T <= 0 || K <= 0 || I <= 0 || K_out <= 0 || n_alpha <= 0) return 0;
    if (K % awq::kGroup != 0 || I % awq::kGroup != 0) return 0;
    return awq::search_mlp_workspace_bytes(T, K, I, K_out, n_alpha);
}

awq_status awq_search_scale_mlp(const void* W_gate, const void* W_up, const void* W_down,
                                const void* X_cal, int T, int K, int I, int K_out,
                                const float* alphas, int n_alpha, int bits, int group_size,
                                int zero_point, float* s_out, float* loss_out, int* best_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_quant_params(bits, group_size, zero_point);
    if (st) return as_status(st);
    if (n_alpha < 1 || n_alpha > kMaxAlpha) return AWQ_ERR_UNSUPPORTED;
    if (T > kMaxT) return AWQ_ERR_UNSUPPORTED;
    if (T <= 0 || I <= 0 || K_out <= 0) return AWQ_ERR_SHAPE;
    if ((st = check_nk(I, K))) return as_status(st);
    if (I % awq::kGroup != 0) return AWQ_ERR_SHAPE;            // I is the down projection's K
    // 32-bit offsets into X_cal and into the intermediate activations
    if ((long long)T * K >= (1LL << 31) || (long long)T * I >= (1LL << 31)) return AWQ_ERR_SHAPE;
    if ((long long)K_out * I >= (1LL << 40) || (long long)I * K >= (1LL << 40)) return AWQ_ERR_SHAPE;
    if (alphas == nullptr) return AWQ_ERR_NULL;
    if ((st = check_ptrs({W_gate, W_up, W_down, X_cal, s_out, workspace}))) return as_status(st);
    if (loss_out != nullptr && (st = check_ptr(loss_out))) return as_status(st);
    if (best_out != nullptr && (st = check_ptr(best_out))) return as_status(st);
    if (workspace_bytes < awq::search_mlp_workspace_bytes(T, K, I, K_out, n_alpha)) return AWQ_ERR_WORKSPACE;
    return hip_status(awq::launch_search_mlp(W_gate, W_up, W_down, K_out, X_cal, T, K, I, alphas, n_alpha,
                                             bits, group_size, zero_point, s_out, loss_out, best_out,
                                             workspace, stream));
}

namespace {
// shared checks of the decode entry points; 1 = nothing to do (M or N is 0)
int check_gemv(int M, int N, int K, int bits, int group_size) {
    int st = check_quant_params(bits, group_size, 1);
    if (st) return as_status(st);
    if (M > kMaxGemvM) return AWQ_ERR_UNSUPPORTED;
    if (M < 0) return AWQ_ERR_SHAPE;
    if ((st = check_nk(N, K))) return as_status(st);
    // the decode kernels address x and the packed tiles with 32-bit offsets
    if ((long long)M * K * 2 >= (1LL << 31) ||
        16LL * ((N + 15) / 16) * K / 8 * bits >= (1LL << 31))
        return AWQ_ERR_SHAPE;
    return (M == 0 || N == 0) ? -1 : AWQ_OK;
}
}  // namespace

awq_status awq_gemv(const void* x, const void* qweight, const void* scales, const void* zeros, void* y,
             int M, int N, int K, int bits, int group_size, hipStream_t stream) {
    int st = check_gemv(M, N, K, bits, group_size);
    if (st) return st < 0 ? AWQ_OK : as_status(st);
    if ((st = check_ptrs({x, qweight, scales, zeros, y}))) return as_status(st);
    return hip_status(awq::launch_gemv(x, nullptr, qweight, scales, zeros, nullptr, nullptr, nullptr,
                                       y, M, N, K, bits, group_size, stream));
}

awq_status awq_gemv_scaled(const void* x, const float* inv_s, const void* qweight, const void* scales,
                    const void* zeros, void* y, int M, int N, int K, int bits, int group_size,
                    hipStream_t stream) {
    int st = check_gemv(M, N, K, bits, group_size);
    if (st) return st < 0 ? AWQ_OK : as_status(st);
    if ((st = check_ptrs({x, inv_s, qweight, scales, zeros, y}))) return as_status(st);
    return hip_status(awq::launch_gemv(x, inv_s, qweight, scales, zeros, nullptr, nullptr, nullptr,
                                       y, M, N, K, bits, group_size, stream));
}

awq_status awq_gemv_gate_up(const void* x, const float* inv_s, const void* gate_qweight,
                     const void* gate_scales, const void* gate_zeros, const void* up_qweight,
                     const void* up_scales, const void* up_zeros, void* h, int M, int N, int K,
                     int bits, int group_size, hipStream_t stream) {
    int st = check_gemv(M, N, K, bits, group_size);
    if (st) return st < 0 ? AWQ_OK : as_status(st);
    if ((st = check_ptrs({x, gate_qweight, gate_scales, gate_zeros, up_qweight, up_scales, up_zeros, h})))
        return as_status(st);
    if (inv_s && (st = check_ptr(inv_s))) return as_status(st);
    return hip_status(awq::launch_gemv(x, inv_s, gate_qweight, gate_scales, gate_zeros, up_qweight,
                                       up_scales, up_zeros, h, M, N, K, bits, group_size,
                                       stream));
}

awq_status awq_gemm(const void* x, const void* qweight, const void* scales, const void* zeros, void* y,
             int M, int N, int K, int bits, int group_size, hipStream_t stream) {
    int st = check_quant_params(bits, group_size, 1);
    if (st) return as_status(st);
    if (M < 0) return AWQ_ERR_SHAPE;
    if ((st = check_nk(N, K))) return as_status(st);
    // the prefill kernel addresses x and the packed tiles with 32-bit offsets
    if ((long long)M * K >= (1LL << 31) || (long long)N * K / 8 >= (1LL << 31)) return AWQ_ERR_SHAPE;
    if (M == 0 || N == 0) return AWQ_OK;
    if ((st = check_ptrs({x, qweight, scales, zeros, y}))) return as_status(st);
    return hip_status(awq::launch_gemm(x, nullptr, qweight, scales, zeros, y, M, N, K, bits, group_size,
                                       stream));
}

size_t awq_gemm_splitk_workspace_bytes(int M, int N, int K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % awq::kGroup != 0) return 0;
    return awq::gemm_splitk_workspace_bytes(M, N, K);
}

awq_status awq_gemm_splitk(const void* x, const void* qweight, const void* scales, const void* zeros,
                    void* y, int M, int N, int K, int bits, int group_size, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
    int st = check_quant_params(bits, group_size, 1);
    if (st) return as_status(st);
    if (M < 0) return AWQ_ERR_SHAPE;
    if ((st = check_nk(N, K))) return as_status(st);
    if ((long long)M * K >= (1LL << 31) || (long long)N * K / 8 >= (1LL << 31)) return AWQ_ERR_SHAPE;
    if (M == 0 || N == 0) return AWQ_OK;
    if ((st = check_ptrs({x, qweight, scales, zeros, y}))) return as_status(st);
    const size_t need = awq::gemm_splitk_workspace_bytes(M, N, K);
    if (need > 0) {
        if (workspace == nullptr) return AWQ_ERR_NULL;
        if ((st = check_ptr(workspace))) return as_status(st);
        if (workspace_bytes < need) return AWQ_ERR_WORKSPACE;
    }
    return hip_status(awq::launch_gemm_splitk(x, nullptr, qweight, scales, zeros, y, M, N, K, bits,
                                              group_size, workspace, stream));
}

awq_status awq_gemm_scaled(const void* x, const float* inv_s, const void* qweight,
                           const void* scales, const void* zeros, void* y, int M, int N, int K,
                           int bits, int group_size, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    int st = check_quant_params(bits, group_size, 1);
    if (st) return as_status(st);
    if (M < 0) return AWQ_ERR_SHAPE;
    if ((st = check_nk(N, K))) return as_status(st);
    if ((long long)M * K >= (1LL << 31) || (long long)N * K / 8 >= (1LL << 31)) return AWQ_ERR_SHAPE;
    if (M == 0 || N == 0) return AWQ_OK;
    if ((st = check_ptrs({x, inv_s, qweight, scales, zeros, y}))) return as_status(st);
    if (workspace == nullptr || workspace_bytes == 0)
        return hip_status(awq::launch_gemm(x, inv_s, qweight, scales, zeros, y, M, N, K, bits,
                                           group_size, stream));
    if ((st = check_ptr(workspace))) return as_status(st);
    if (workspace_bytes < awq::gemm_splitk_workspace_bytes(M, N, K)) return AWQ_ERR_WORKSPACE;
    return hip_status(awq::launch_gemm_splitk(x, inv_s, qweight, scales, zeros, y, M, N, K, bits,
                                              group_size, workspace, stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// awq_gemm_splitk_noalloc: awq_gemm_splitk with the fp32 partial sums in a
// fixed device array instead of a caller workspace.  Split K runs only while
// the output tiles (at most 128 x 256) occupy at most half the CUs, so the
// partials take at most CUs x 128 x 256 x 4 bytes: 32 MiB on a 256-CU MI355X.
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address of each
// GPU's copy is asked of the runtime once, with that device current, and kept.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// the current device's copy of `scratch` (nullptr if the runtime cannot say)
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

size_t awq_gemm_splitk_noalloc_max_bytes(void) { return kScratchBytes; }

awq_status awq_gemm_splitk_noalloc(const void* x, const void* qweight, const void* scales,
                                   const void* zeros, void* y, int M, int N, int K, int bits,
                                   int group_size, hipStream_t stream) {
    int st = check_quant_params(bits, group_size, 1);
    if (st) return as_status(st);
    if (M < 0) return AWQ_ERR_SHAPE;
    if ((st = check_nk(N, K))) return as_status(st);
    if ((long long)M * K >= (1LL << 31) || (long long)N * K / 8 >= (1LL << 31)) return AWQ_ERR_SHAPE;
    if (M == 0 || N == 0) return AWQ_OK;
    if ((st = check_ptrs({x, qweight, scales, zeros, y}))) return as_status(st);
    const size_t need = awq::gemm_splitk_workspace_bytes(M, N, K);
    if (need > kScratchBytes) return AWQ_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0 && (ws = device_scratch()) == nullptr) return AWQ_ERR_HIP;
    // every split writes all M x N entries of its partial tile, so nothing in
    // the array needs clearing between calls
    return hip_status(awq::launch_gemm_splitk(x, nullptr, qweight, scales, zeros, y, M, N, K, bits,
                                              group_size, ws, stream));
}

}  // extern "C"
