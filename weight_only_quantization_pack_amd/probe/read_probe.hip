// Plain streaming-read kernel: the achievable HBM read rate at a given byte
// count on this GPU, measured the way the decode GEMV is (cold buffers, one
// launch per buffer, graph replay).  It is a measuring stick for the GEMV's
// roofline, not part of the quantized matmul path; only the benchmark loads
// this library.
//
// Each workgroup reads chunks of WT * 16 * U bytes (chunk c, c + gridDim.x,
// ...): lane t issues U 16-byte non-temporal buffer loads per chunk, all in
// flight before the first is used, and folds them into an XOR.  Loads past
// `bytes` are out-of-range buffer loads (zero, no memory access), so the
// kernel never touches memory outside the buffer.  Each workgroup writes one
// word (its XOR) to out[blockIdx.x], which keeps the loads alive.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <int WT, int U>
__global__ __launch_bounds__(WT) void k_read(const void* buf, uint32_t bytes, uint32_t* out) {
    const __amdgpu_buffer_rsrc_t r = rsrc(buf, bytes);
    constexpr uint32_t CH = (uint32_t)WT * 16u * U;
    const uint32_t nch = (bytes + CH - 1) / CH;
    uint32_t acc = 0;
    for (uint32_t c = blockIdx.x; c < nch; c += gridDim.x) {
        uint32_t v[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t off = c * CH + ((uint32_t)u * WT + threadIdx.x) * 16u;
            const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
            v[u][0] = w[0]; v[u][1] = w[1]; v[u][2] = w[2]; v[u][3] = w[3];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    __shared__ uint32_t red[WT / 64];
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < WT / 64; ++w) t ^= red[w];
        out[blockIdx.x] = t;
    }
}

using ReadFn = void (*)(const void*, uint32_t, uint32_t*);

ReadFn pick(int threads, int unroll) {
    if (threads == 256) return unroll == 4 ? k_read<256, 4> : unroll == 8 ? k_read<256, 8> : k_read<256, 16>;
    if (threads == 512) return unroll == 4 ? k_read<512, 4> : unroll == 8 ? k_read<512, 8> : k_read<512, 16>;
    return unroll == 4 ? k_read<1024, 4> : unroll == 8 ? k_read<1024, 8> : nullptr;
}

}  // namespace

extern "C" {

// Workgroups a launch of this configuration uses for `bytes` (at most
// `max_groups`, never more than the chunks); `out` needs that many words.
int awq_probe_read_groups(size_t bytes, int threads, int unroll, int max_groups) {
    if (bytes == 0 || max_groups <= 0) return 0;
    const size_t ch = (size_t)threads * 16 * unroll;
    const size_t nch = (bytes + ch - 1) / ch;
    return (int)(nch < (size_t)max_groups ? nch : (size_t)max_groups);
}

// Read `bytes` (< 2^31, 16-byte aligned device buffer) once with workgroups
// of `threads` (256, 512 or 1024) lanes, `unroll` (4, 8 or 16; 4 or 8 for
// 1024) loads in flight per lane, on at most `max_groups` workgroups.
// Returns 0, or a hipError_t value (invalid configuration: hipErrorInvalidValue).
int awq_probe_read(const void* buf, size_t bytes, int threads, int unroll, int max_groups,
                   uint32_t* out, hipStream_t stream) {
    if (buf == nullptr || out == nullptr || bytes >= ((size_t)1 << 31)) return (int)hipErrorInvalidValue;
    if ((threads != 256 && threads != 512 && threads != 1024) || (unroll != 4 && unroll != 8 && unroll != 16))
        return (int)hipErrorInvalidValue;
    ReadFn f = pick(threads, unroll);
    if (f == nullptr) return (int)hipErrorInvalidValue;
    const int g = awq_probe_read_groups(bytes, threads, unroll, max_groups);
    if (g == 0) return 0;
    hipLaunchKernelGGL(f, dim3(g), dim3(threads), 0, stream, buf, (uint32_t)bytes, out);
    return (int)hipGetLastError();
}

}  // extern "C"
