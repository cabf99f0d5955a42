/*
 * awq.h -- C ABI of the AWQ W4A16 g128 hot path for MI355X (gfx950)
 * (also W3A16, and 64-wide groups).
 *
 * What the calls compute is set by these web pages (cited by title and
 * section; no code is taken from them):
 *   "AWQ: Activation-aware Weight Quantization for LLM Compression and
 *    Acceleration" (llm-awq README): feature list (AWQ search, a 4-bit
 *    linear layer, kernels for the context and decode stages), AWQ model zoo
 *    table (INT4-g128 and INT3-g128), "Usage" (--w_bit 4 --q_group_size 128;
 *    search, fake quantization, real INT4 quantization).
 *   "transformers - AWQ": the quantization_config block (bits 4,
 *    group_size 128, zero_point true, version "gemm").
 *   "AWQ (Activation-Aware Weight Quantization) and how it differs from
 *    GPTQ": "Applying AWQ with AutoAWQ" (saliency from activation magnitude
 *    on calibration data), "Quantizing a model with AutoAWQ" (w_bit,
 *    q_group_size, zero_point).
 *   "LLM quantization's revolutionary breakthrough (VPTQ)", section 02.02
 *    "AWQ": salient input channels are scaled up through an equivalent
 *    transform; the scale comes from offline activation statistics.
 *
 * Conventions shared by every call
 *   - Math: y = x . W^T.  W is fp16 [N][K] (output x input, row-major),
 *     x is fp16 [M][K], y is fp16 [M][N].  Groups of group_size = 128
 *     (or 64: "Quantizing a model with AutoAWQ" gives 64 and 128 as typical
 *     q_group_size values) consecutive k share one fp16 scale D and one
 *     integer zero point z; G = K / group_size.  Q = 2^bits - 1.  K must be
 *     a multiple of 128 for either group size (a packed tile spans 128 k).
 *   - Pointers are DEVICE pointers (HBM) allocated by the caller, 16-byte
 *     aligned, unless a comment says HOST.  The library never allocates or
 *     frees and keeps nothing after a call returns; scratch memory comes only
 *     from the caller's workspace.  Calls are asynchronous on `stream`
 *     (a hipStream_t; NULL = the default stream); outputs are ready when the
 *     stream is synchronized.  Calls on different streams are re-entrant.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error nothing is launched and no output is touched.  No C++
 *     exception crosses this interface.  Inputs must be finite (not checked).
 *   - M == 0 or N == 0 is a valid empty call: it returns AWQ_OK and
 *     launches nothing.
 *
 * Packed weight format, version 3 (chosen for gfx950 MFMA operand loads):
 *   Row words.  bits = 4: word j of row n holds the codes of k = 8j..8j+7;
 *     code 8j+2t is at bits 4t..4t+3 and code 8j+2t+1 at bits 16+4t..19+4t
 *     (t = 0..3), so ((w >> 4t) & 0x000F000F) | 0x64006400 is the fp16 pair
 *     (1024 + q[8j+2t], 1024 + q[8j+2t+1]).  bits = 3: each run of 32 codes
 *     c[i] = q[32r + i] fills 3 words; pair P = (c[2P], c[2P+1]), P < 15, sits
 *     in word P / 5 with c[2P] at bits 3t..3t+2 and c[2P+1] at bits
 *     16+3t..18+3t (t = P % 5), so ((w >> 3t) & 0x00070007) | 0x64006400 is
 *     its fp16 pair; bit b of c[30] and of c[31] is bit 15 and bit 31 of word
 *     b.  (Version 2 held the int3 run as a 96-bit bit stream; int4 and the
 *     tiling are unchanged.)
 *   Tiles.  Rows are taken 16 at a time (row block b = rows 16b..16b+15,
 *     padded with zero rows past N).  Tile (b, t) holds k = 128t .. 128t+127
 *     of the 16 rows of block b as 64 lane slots; slot s = 16h + j holds the
 *     row words of row 16b + j that cover k = 128t + 32h .. 128t + 32h + 31
 *     (4 words for bits 4, 3 for bits 3).  The codes' layout does not depend
 *     on the group size.  qweight is the array of tiles
 *     [ceil(N/16)][K/128][64][4 or 3] uint32: one tile is one
 *     contiguous 1 KB (768 B for bits 3) wave load whose slots are the
 *     v_mfma_f32_16x16x32_f16 operand layout.
 *   scales, zeros: fp16 [ceil(N/16)][G][16], the same tiling: the group
 *     scale D[n][g] and the integer zero point z[n][g] (0..Q, stored
 *     exactly) of row n sit at [n / 16][g][n % 16]; padding rows hold 0.
 *     One group's 16 scales are one 32-byte load next to their tile (with
 *     64-wide groups a tile's two groups are g = 2t, 2t + 1).
 *   Dequantized weight: w_hat[n][k] = (q[n][k] - z[n][g]) * D[n][g].
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream handle, declared as HIP declares it so that this header
 * needs no HIP include (the same type as hip_runtime_api.h's hipStream_t).
 * Every call is asynchronous on the stream it is given; NULL is the default
 * stream. */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    AWQ_OK = 0,
    AWQ_ERR_NULL = 1,         /* a required pointer is NULL                 */
    AWQ_ERR_SHAPE = 2,        /* negative size, K == 0, K % group_size != 0 */
    AWQ_ERR_UNSUPPORTED = 3,  /* bits, group_size, zero_point or M not supported */
    AWQ_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned           */
    AWQ_ERR_WORKSPACE = 5,    /* workspace smaller than required            */
    AWQ_ERR_HIP = 6           /* a HIP launch or runtime call failed        */
} awq_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* awq_status_str(awq_status status);

/* Version of the packed weight format described above (3). */
int awq_pack_format_version(void);

/* uint32 words per packed row: K/8 for bits 4, 3K/32 for bits 3
 * (0 for unsupported bits or K <= 0). */
size_t awq_packed_words_per_row(int K, int bits);

/* uint32 words of a whole packed matrix: 16 * ceil(N/16) * words_per_row
 * (0 for invalid arguments). */
size_t awq_packed_words(int N, int K, int bits);

/*
 * awq_quantize_pack -- round-to-nearest group quantization of W*diag(s),
 * then packing ("Usage" step 3 of the llm-awq README: real INT4 weights;
 * "Quantizing a model with AutoAWQ": w_bit, q_group_size, zero_point).
 *
 *   W        fp16 [N][K]   weights, row-major (nn.Linear layout)
 *   s        fp32 [K]      per-input-channel scale, or NULL for s == 1
 *   qweight  uint32 [awq_packed_words(N, K, bits)]  out, format above
 *            (padding rows of the last block are written as zeros)
 *   scales   fp16 [ceil(N/16)][G][16]  out, D (below)
 *   zeros    fp16 [ceil(N/16)][G][16]  out, z (below)
 * with, per (n, g), v = fp32(W) * s and q = clamp(rint(v / D) + z, 0, Q),
 * Q = 2^bits - 1:
 *   zero_point = 1 (asymmetric): lo = min(0, min v), hi = max(0, max v),
 *     D = largest fp16 <= max(hi - lo, 1e-5) / Q, z = clamp(rint(-lo / D), 0, Q)
 *   zero_point = 0 (symmetric): D = largest fp16 <= max(max |v|, 1e-5) /
 *     (2^(bits-1) - 1), z = 2^(bits-1) (codes z - 7..z + 7 for int4)
 * all fp32 IEEE, round-half-even, correctly rounded division.  Either way
 * w_hat = (q - z) * D, so awq_gemv and awq_gemm serve both.
 * bits in {3, 4}; group_size 128 or 64; zero_point 0 or 1.
 */
awq_status awq_quantize_pack(const void* W, const float* s, int N, int K, int bits,
                      int group_size, int zero_point, void* qweight,
                      void* scales, void* zeros, hipStream_t stream);

/*
 * awq_dequantize -- fake quantization ("Usage" step 2 of the llm-awq README,
 * --q_backend fake: the quantized weights kept as dequantized fp16 values):
 *   W_hat[n][k] = fp16_rne((q[n][k] - z[n][g]) * D[n][g])
 *   (the product is exact in fp32; one rounding to fp16)
 *   qweight, scales, zeros as produced by awq_quantize_pack (same bits and
 *   group_size); W_hat fp16 [N][K] out.  Errors as awq_quantize_pack.
 */
awq_status awq_dequantize(const void* qweight, const void* scales, const void* zeros,
                   void* W_hat, int N, int K, int bits, int group_size,
                   hipStream_t stream);

/*
 * awq_scale_activations -- the activation side of the equivalent transform
 * (section 02.02 "AWQ" of the VPTQ blog): x_out[m][k] = fp16_rne(fp32(x[m][k]) / s[k]).
 *   x      fp16 [M][K] in;  s fp32 [K] in;  x_out fp16 [M][K] out (may equal x).
 */
awq_status awq_scale_activations(const void* x, const float* s, void* x_out, int M,
                          int K, hipStream_t stream);

/*
 * awq_search_workspace_bytes -- device workspace of awq_search_scale's
 * buffered path for T calibration tokens, an N x K layer and n_alpha grid
 * points: it holds W - w_hat_i / s_i for one chunk of alphas (as many as fit
 * in 128 MB, at least one: N rounded up to a multiple of 16 x K fp16 each, in
 * the loss GEMM's tiled layout; the grid is run chunk by chunk).  0 when an
 * argument is <= 0.
 */
size_t awq_search_workspace_bytes(int T, int N, int K, int n_alpha);

/*
 * awq_search_workspace_bytes_fused -- the smaller workspace (the scales and
 * one loss partial per tile and alpha: 0.7 MB for a 4096 x 4096 layer, T =
 * 512, 20 alphas) with which awq_search_scale and awq_search_scale_shared take
 * their fused path: one loss kernel forms W - w_hat_i / s_i in registers
 * instead of writing it out (the same codes and the same fp16 differences).
 * MI355X, T = 512, 20 alphas: 0.63-0.68 ms against 0.51-0.54 ms buffered on
 * 4096 x 4096, where four alphas' differences fit the cache; 8.0 against 9.0
 * ms and 8.0 against 11.6 ms on the Llama-70B MLP layers, where one alpha's
 * do not.  A workspace of at least awq_search_workspace_bytes selects the
 * buffered path, one of at least this size the fused one, anything smaller is
 * AWQ_ERR_WORKSPACE.
 */
size_t awq_search_workspace_bytes_fused(int T, int N, int K, int n_alpha);

/*
 * awq_search_scale -- the AWQ scale search ("Usage" step 1, --run_awq, of
 * the llm-awq README; scale from offline activation statistics, section
 * 02.02 of the VPTQ blog; saliency from activation magnitude, "Applying AWQ
 * with AutoAWQ").
 *   s_x[k]   = mean_t |X_cal[t][k]|                         (exact fp64 sum)
 *   s_i[k]   = fp32(pow(max(s_x[k], 1e-4), alphas[i]))        (fp64 pow)
 *   L_i      = mean_{t,n} (sum_k X_cal[t][k] (W[n][k] - w_hat_i[n][k] / s_i[k]))^2
 *              with w_hat_i the dequantized weights of awq_quantize_pack(W, s_i)
 *              (same bits and zero_point)
 *   best     = smallest i with L_i == min L
 *   W        fp16 [N][K] in;  X_cal fp16 [T][K] in, 1 <= T <= 8192, T * K < 2^31
 *   alphas   HOST fp32 [n_alpha], 1 <= n_alpha <= 64
 *   s_out    fp32 [K] out: s_best
 *   loss_out fp32 [n_alpha] out, or NULL
 *   best_out int32 [1] out (device), or NULL
 *   workspace / workspace_bytes: device scratch of at least
 *            awq_search_workspace_bytes(T, N, K, n_alpha) bytes (default
 *            path), or of awq_search_workspace_bytes_fused bytes (fused path).
 * The loss is one fp16 MFMA kernel with fp32 accumulation that forms the fp16
 * differences W - w_hat_i * (1/s_i) in registers (the codes are those of
 * awq_quantize_pack), so L_i carries a relative error of order 1e-4 and
 * near-ties may pick a neighbouring alpha.
 */
awq_status awq_search_scale(const void* W, const void* X_cal, int T, int N, int K,
                     const float* alphas, int n_alpha, int bits, int group_size,
                     int zero_point, float* s_out, float* loss_out, int* best_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_search_scale_shared -- one scale search for several layers that read
 * the same input (q/k/v after one norm, gate/up after another): the
 * activations are divided by s once (section 02.02 "AWQ" of the VPTQ blog), so
 * every layer fed by that input carries the same s.
 *   The layers' rows, in order, are searched as the rows of one layer of
 *   N = sum Ns[l] rows: L_i is the mean over t and every row of every layer,
 *   i.e. the row-weighted mean of the layers' own losses; everything else as
 *   awq_search_scale.  Each layer is read in place (no copy).
 *   Ws       HOST array of n_layers device pointers, layer l fp16 [Ns[l]][K]
 *   Ns       HOST int array [n_layers], each >= 1;  1 <= n_layers <= 8
 *   workspace: awq_search_workspace_bytes(T, sum Ns, K, n_alpha) bytes, or
 *            the _fused size for the fused path.
 *   Errors as awq_search_scale; n_layers out of range is AWQ_ERR_UNSUPPORTED,
 *   a NULL Ws / Ns / layer pointer AWQ_ERR_NULL, a row count <= 0 AWQ_ERR_SHAPE.
 */
awq_status awq_search_scale_shared(const void* const* Ws, const int* Ns, int n_layers,
                            const void* X_cal, int T, int K, const float* alphas,
                            int n_alpha, int bits, int group_size, int zero_point,
                            float* s_out, float* loss_out, int* best_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_search_mlp_workspace_bytes -- device workspace of awq_search_scale_mlp:
 * the quantization errors of both layers for one chunk of alphas (chunk x 2I
 * x K fp16; the chunk is as many alphas as fit in 128 MB, but at least enough
 * to fill the GPU), the tiled weights, the reference activations (3 x T x I
 * fp32), the change of the intermediate activation per alpha of the chunk
 * (chunk x T x I fp16) and the loss partials.  0 for invalid sizes (K or I
 * not a multiple of 128).
 */
size_t awq_search_mlp_workspace_bytes(int T, int K, int I, int K_out, int n_alpha);

/*
 * awq_search_scale_mlp -- the AWQ scale search ("Usage" step 1 of the llm-awq
 * README) of the gate and up projections of an MLP block, which read one
 * input and so share one s (section 02.02 "AWQ" of the VPTQ blog), with the
 * error measured on the block's output ("transformers - AWQ", "Fused
 * modules": the MLP as gate, up and down):
 *   y      = (SiLU(X W_gate^T) * (X W_up^T)) W_down^T
 *   y_i    = the same with gate and up replaced by their fake-quantized
 *            weights w_hat_i / s_i (awq_quantize_pack with s_i), W_down kept
 *   L_i    = mean over t and the K_out outputs of (y_i - y)^2
 *   best   = smallest i with L_i == min L;  s_i as in awq_search_scale
 *   W_gate, W_up  fp16 [I][K];  W_down fp16 [K_out][I];  X_cal fp16 [T][K]
 *   K and I multiples of 128; 1 <= T <= 8192, T * K and T * I < 2^31
 *   alphas HOST fp32 [n_alpha], 1 <= n_alpha <= 64
 *   s_out fp32 [K] out; loss_out fp32 [n_alpha] out or NULL; best_out int32
 *   [1] out (device) or NULL; workspace of at least
 *   awq_search_mlp_workspace_bytes(T, K, I, K_out, n_alpha) bytes.
 * The change of the intermediate activation SiLU(g) u is formed in fp32 from
 * the fp16-MFMA products of X with the weights and with their quantization
 * errors, rounded to fp16 and multiplied by W_down on fp16 MFMA with fp32
 * accumulation, so L_i carries a relative error of order 1e-3 and near-ties
 * may pick a neighbouring alpha.  Errors as awq_search_scale (an I or K that
 * is not a multiple of 128 is AWQ_ERR_SHAPE).
 */
awq_status awq_search_scale_mlp(const void* W_gate, const void* W_up, const void* W_down,
                                const void* X_cal, int T, int K, int I, int K_out,
                                const float* alphas, int n_alpha, int bits, int group_size,
                                int zero_point, float* s_out, float* loss_out, int* best_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_gemv -- decode-stage W4A16 (or W3A16) product for small batches (the
 * decode kernel of the llm-awq README feature list):
 *   y[m][n] = sum_g D[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
 *   x fp16 [M][K] in; qweight, scales, zeros as produced by
 *   awq_quantize_pack; y fp16 [M][N] out (round to nearest from fp32).
 *   1 <= M <= 16; bits in {3, 4}; group_size 128 or 64 (as packed).  With
 *   64-wide groups each weight is dequantized to fp16 (q - z) * D before the
 *   product (one rounding); with 128 the group sums are scaled in fp32.
 *   The packed weight must
 *   be < 2^31 bytes (16 * ceil(N/16) * K * bits / 8) and x < 2^31 bytes
 *   (M * K * 2), else AWQ_ERR_SHAPE.
 */
awq_status awq_gemv(const void* x, const void* qweight, const void* scales,
             const void* zeros, void* y, int M, int N, int K, int bits,
             int group_size, hipStream_t stream);

/*
 * awq_gemv_scaled -- awq_gemv with the activation side of the equivalent
 * transform (section 02.02 "AWQ" of the VPTQ blog: x / s against weights
 * quantized as W * s) folded into the activation load, so no separate pass
 * over x is needed (the fused modules of "transformers - AWQ" fold it into
 * the layer before):
 *   x'[m][k] = fp16_rne(fp32(x[m][k]) * inv_s[k]);  y = awq_gemv(x', ...)
 *   inv_s  fp32 [K] in, device, 16-byte aligned: the caller's 1 / s (NULL is
 *          AWQ_ERR_NULL).  With inv_s = fp32(1 / s), x' equals
 *          awq_scale_activations(x, s) except where x / s lies within one fp32
 *          ulp of an fp16 rounding boundary (then one fp16 ulp apart).
 *   Other arguments, limits and errors as awq_gemv.
 */
awq_status awq_gemv_scaled(const void* x, const float* inv_s, const void* qweight,
                    const void* scales, const void* zeros, void* y, int M, int N,
                    int K, int bits, int group_size, hipStream_t stream);

/*
 * awq_gemv_gate_up -- the gate and up projections of a fused MLP ("transformers
 * - AWQ", "Fused modules": the gate, up and down layers of the MLP fused into
 * one module; Llama and Mistral use SiLU on the gate output) in one launch:
 *   g = x' . w_hat_gate^T,  u = x' . w_hat_up^T   (fp32 sums, as awq_gemv)
 *   h[m][n] = fp16_rne(SiLU(g[m][n]) * u[m][n]),  SiLU(t) = t / (1 + e^-t) in fp32
 *   x' = x * inv_s as in awq_gemv_scaled, or x when inv_s is NULL (gate and up
 *   read the same input, so they share one activation scale).
 *   gate_* / up_*: two layers of the same N x K shape, bits and group_size,
 *   packed by awq_quantize_pack.  h fp16 [M][N] out.  The down projection is
 *   a plain awq_gemv / awq_gemv_scaled on h.
 *   Limits and errors as awq_gemv; every pointer but inv_s is required.
 */
awq_status awq_gemv_gate_up(const void* x, const float* inv_s, const void* gate_qweight,
                     const void* gate_scales, const void* gate_zeros,
                     const void* up_qweight, const void* up_scales,
                     const void* up_zeros, void* h, int M, int N, int K, int bits,
                     int group_size, hipStream_t stream);

/*
 * awq_gemm -- context-stage (prefill) W4A16 product, same formula as
 * awq_gemv for any M >= 1 (the context kernel of the llm-awq README
 * feature list; version "gemm" in the transformers quantization_config).
 * Dequantized fp16 tiles feed fp16 MFMA with fp32 accumulation.
 *   bits in {3, 4}; group_size 128 or 64; M*K < 2^31 and N*K/8 < 2^31 (else
 *   AWQ_ERR_SHAPE).
 */
awq_status awq_gemm(const void* x, const void* qweight, const void* scales,
             const void* zeros, void* y, int M, int N, int K, int bits,
             int group_size, hipStream_t stream);

/*
 * awq_gemm_splitk_workspace_bytes -- device workspace awq_gemm_splitk needs
 * for an M x N x K product on the current device: 0 when the output tiles
 * already occupy at least half the workgroup slots (one per compute unit,
 * two for M <= 16; no split), else splits * M * N * 4 bytes of fp32 partial
 * sums.  0 for invalid shapes.
 */
size_t awq_gemm_splitk_workspace_bytes(int M, int N, int K);

/*
 * awq_gemm_splitk -- the awq_gemm product for small M (few output tiles),
 * with K split across workgroups: each split writes an fp32 partial tile to
 * the workspace and a second kernel adds the splits in a fixed order and
 * rounds to fp16 (deterministic).  The split count is chosen per shape and
 * device (each split keeps >= 8 groups, at most 16 splits); with one split
 * this is awq_gemm.  Same arguments and limits as awq_gemm, plus
 *   workspace / workspace_bytes: device scratch of at least
 *   awq_gemm_splitk_workspace_bytes(M, N, K) bytes (ignored, may be NULL,
 *   when that is 0), 16-byte aligned; too small -> AWQ_ERR_WORKSPACE.
 * Callers that need no workspace use awq_gemm.  (The split-K / stream-K
 * prefill item of the decode/prefill split in "transformers - AWQ".)
 */
awq_status awq_gemm_splitk(const void* x, const void* qweight, const void* scales,
                    const void* zeros, void* y, int M, int N, int K, int bits,
                    int group_size, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * awq_gemm_scaled -- awq_gemm (and, given a workspace, awq_gemm_splitk) with
 * the activation side of the equivalent transform (section 02.02 "AWQ" of the
 * VPTQ blog: x / s against weights quantized as W * s) folded into the
 * activation tiles, so a prefill needs no separate pass over x (the fused
 * modules of "transformers - AWQ" fold it into the layer before):
 *   x'[m][k] = fp16_rne(fp32(x[m][k]) * inv_s[k]);  y = awq_gemm(x', ...)
 *   the same x' as awq_gemv_scaled, bit for bit.
 *   inv_s    fp32 [K] in, device, 16-byte aligned: the caller's 1 / s.
 *   workspace / workspace_bytes: NULL or 0 runs without a K split (as
 *            awq_gemm); otherwise at least awq_gemm_splitk_workspace_bytes(M,
 *            N, K) bytes (else AWQ_ERR_WORKSPACE), and the shape splits K as
 *            awq_gemm_splitk does.
 *   Other arguments, limits and errors as awq_gemm.
 */
awq_status awq_gemm_scaled(const void* x, const float* inv_s, const void* qweight,
                           const void* scales, const void* zeros, void* y, int M, int N, int K,
                           int bits, int group_size, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * awq_gemm_splitk_noalloc -- awq_gemm_splitk for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels, split count and
 * results (bit for bit), with the fp32 partial sums in a fixed device array
 * of awq_gemm_splitk_noalloc_max_bytes() bytes (32 MiB) that the library
 * holds on each GPU it runs on until the process ends.  The call allocates
 * nothing and frees nothing.
 *   Arguments, limits and errors as awq_gemm_splitk without the workspace;
 *   a shape whose split needs more than the array holds
 *   (awq_gemm_splitk_workspace_bytes(M, N, K) > the maximum) is
 *   AWQ_ERR_WORKSPACE, and AWQ_ERR_HIP if the runtime cannot give the
 *   array's address on the current device.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (other streams or host threads) race and must be serialized by the
 *   caller.  Each call writes every partial it reads, so nothing carries over
 *   from a previous call.
 */
size_t awq_gemm_splitk_noalloc_max_bytes(void);
awq_status awq_gemm_splitk_noalloc(const void* x, const void* qweight, const void* scales,
                                   const void* zeros, void* y, int M, int N, int K, int bits,
                                   int group_size, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_H */
