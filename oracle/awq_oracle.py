"""CPU oracle for the AWQ W4A16 g128 hot path -- TEST INFRASTRUCTURE ONLY.

This module is the slow, plain, obviously-correct definition that the HIP
library is checked against.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  The product path (``weight_only_quantization_pack_amd``) never imports
it, and it imports nothing from the product: the two share no arithmetic.

Sources (web pages, cited by title and section):
  [P1] "AWQ: Activation-aware Weight Quantization for LLM Compression and
       Acceleration" (llm-awq README, Chinese translation) -- feature list,
       "AWQ model zoo" table (INT4-g128 / INT3-g128), "Usage" (search, fake
       and real quantization with --w_bit 4 --q_group_size 128).
  [P3] "transformers - AWQ" -- the quantization_config block
       (bits 4, group_size 128, zero_point true, version "gemm").
  [P4] "AWQ (Activation-Aware Weight Quantization) and how it differs from
       GPTQ" -- "Applying AWQ with AutoAWQ" (salient weights are found from
       the magnitude of the matching activations on calibration data) and
       "Quantizing a model with AutoAWQ" (w_bit, q_group_size, zero_point).
  [P5] "LLM quantization's revolutionary breakthrough (VPTQ)" -- section
       02.02 "AWQ": scale salient input channels up through a
       mathematically equivalent transform; the scale comes from offline
       activation statistics; no backprop or reconstruction.

The pages give the mechanism in words only.  The operational recipe taken
here: s = s_x ** alpha with s_x the per-input-channel mean |activation|,
alpha chosen from a grid by the smallest output MSE of the layer,
round-to-nearest group quantization of W*diag(s) with an fp16 group scale and
an integer zero point, bits 4 (or 3), group 128.  Every point the pages leave
open is a stated reading (listed in the design notes of the repository and
repeated at the function that takes it).

Precision.  Where a float decides an integer (the codes, the zero point, the
stored fp16 scale) the oracle works in IEEE fp32 with correctly rounded
division and round-half-even, which is also the kernel's precision.  Every
other quantity (statistics, dequantized weights, matmul, loss) is fp64.

Parity status: every function here is pinned by tests/test_oracle_*.py
against brute force, closed forms, invariants or the textbook definition.
"""
from __future__ import annotations

import numpy as np

# Parameters named as on the pages ([P4] quant_config, [P3] quantization_config).
GROUP_SIZE = 128                   # default group; also the K width of a packed tile
SUPPORTED_GROUP_SIZES = (64, 128)  # [P4] "Quantizing a model with AutoAWQ": typical 64, 128
SUPPORTED_BITS = (3, 4)
SPAN_FLOOR = np.float32(1e-5)      # reading: (hi - lo), or max |v|, floored before the divide
STAT_FLOOR = 1e-4                  # reading: s_x floored before the power

PACK_FORMAT_VERSION = 3


def levels(bits: int) -> int:
    """Q = 2**bits - 1, the largest code."""
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be 3 or 4, got {bits}")
    return (1 << bits) - 1


# ---------------------------------------------------------------------------
# fp16 helpers
# ---------------------------------------------------------------------------
def f16_round_down(v32) -> np.ndarray:
    """Largest fp16 value <= v for positive finite fp32 v.

    Reading: the stored group scale is rounded toward -inf (not to nearest),
    so that the group's extreme values still reach codes 0 and Q and a second
    quantize of the dequantized weights reproduces the same codes.
    """
    v32 = np.asarray(v32, dtype=np.float32)
    h = v32.astype(np.float16)                      # round to nearest even
    went_up = h.astype(np.float32) > v32
    lower = np.nextafter(h, np.float16(-np.inf))
    return np.where(went_up, lower, h).astype(np.float16)


# ---------------------------------------------------------------------------
# a1 / a2: activation statistics and candidate scales
# ---------------------------------------------------------------------------
def act_stat(X_cal: np.ndarray) -> np.ndarray:
    """s_x[k] = mean over calibration tokens of |X_cal[t, k]|  (fp32 result).

    [P4] "Applying AWQ with AutoAWQ": salient weights are identified by the
    magnitude of their activations on calibration data; [P5] 02.02: the scale
    comes from offline activation statistics.  Reading: the statistic is the
    mean absolute value per input channel, summed in fp64 (exact for fp16
    inputs and T < 8192), divided by T in fp64, rounded once to fp32.
    """
    X = np.asarray(X_cal)
    if X.dtype != np.float16 or X.ndim != 2:
        raise ValueError("X_cal must be a 2-D float16 array [T][K]")
    T = X.shape[0]
    total = np.abs(X.astype(np.float64)).sum(axis=0)
    return (total / np.float64(T)).astype(np.float32)


def candidate_scale(s_x: np.ndarray, alpha: float) -> np.ndarray:
    """s[k] = max(s_x[k], 1e-4) ** alpha, evaluated in fp64, rounded to fp32.

    [P5] 02.02: salient channels are scaled up; the exponent form
    s = s_x ** alpha and the floor 1e-4 are the readings taken.  alpha = 0
    gives s == 1 exactly (plain round-to-nearest).
    """
    s64 = np.maximum(np.asarray(s_x, dtype=np.float64), STAT_FLOOR)
    return np.power(s64, np.float64(alpha)).astype(np.float32)


# ---------------------------------------------------------------------------
# a3: group quantization
# ---------------------------------------------------------------------------
def quantize(W: np.ndarray, s: np.ndarray | None = None, bits: int = 4,
             group_size: int = GROUP_SIZE, zero_point: bool = True):
    """Round-to-nearest group quantization of W * diag(s).

    [P4] "Quantizing a model with AutoAWQ": q_group_size weights share one
    scale and one zero point; zero_point=True means asymmetric quantization,
    False symmetric; [P1] "Usage": --w_bit 4 --q_group_size 128.
    v = W[n, k] * s[k] is one fp32 multiply (s = None means s == 1); the
    groups of v are then quantized by ``quantize_values``.
    Returns (q uint8 [N][K], scales fp16 [N][G], zeros fp16 [N][G]).
    """
    W = np.asarray(W)
    if W.dtype != np.float16 or W.ndim != 2:
        raise ValueError("W must be a 2-D float16 array [N][K]")
    K = W.shape[1]
    v = W.astype(np.float32)
    if s is not None:
        s32 = np.asarray(s, dtype=np.float32)
        if s32.shape != (K,):
            raise ValueError("s must have shape [K]")
        v = v * s32[None, :]                        # one fp32 multiply
    return quantize_values(v, bits, group_size, zero_point)


def quantize_values(v: np.ndarray, bits: int = 4, group_size: int = GROUP_SIZE,
                    zero_point: bool = True):
    """Group quantizer on already-scaled fp32 values v [N][K].

    Per (row n, group g of group_size (128 or 64) consecutive k), all in
    IEEE fp32, with zero_point (asymmetric):
        lo  = min(0, min v),  hi = max(0, max v)
        D32 = max(hi - lo, 1e-5) / Q ;  Dh = largest fp16 <= D32 ;  D = Dh
        z   = clamp(rint(-lo / D), 0, Q)
    without (symmetric, zero centred; Qs = 2**(bits-1) - 1):
        D32 = max(max |v|, 1e-5) / Qs ;  Dh = largest fp16 <= D32 ;  D = Dh
        z   = 2**(bits-1)       (a fixed offset, so the codes stay unsigned)
    and in both cases
        q   = clamp(rint(v / D) + z, 0, Q)
    rint rounds half to even.  Readings: the asymmetric range is widened to
    contain 0; the floor 1e-5 keeps an all-zero group finite; Dh is rounded
    down; the code is computed with the stored fp16 scale; the symmetric
    grid is the textbook one, codes -Qs..Qs around the offset.
    """
    Q = levels(bits)
    v = np.asarray(v)
    if v.dtype != np.float32 or v.ndim != 2:
        raise ValueError("v must be a 2-D float32 array [N][K]")
    N, K = v.shape
    if group_size not in SUPPORTED_GROUP_SIZES or K % group_size != 0:
        raise ValueError("group_size must be 64 or 128 and divide K")
    G = K // group_size
    g = v.reshape(N, G, group_size)

    if zero_point:
        lo = np.minimum(g.min(axis=2), np.float32(0.0))
        hi = np.maximum(g.max(axis=2), np.float32(0.0))
        span = np.maximum(hi - lo, SPAN_FLOOR)
        delta16 = f16_round_down(span / np.float32(Q))
        delta = delta16.astype(np.float32)
        z = np.clip(np.rint(-lo / delta), 0, Q).astype(np.int32)
    else:
        amax = np.maximum(np.abs(g).max(axis=2), SPAN_FLOOR)
        delta16 = f16_round_down(amax / np.float32(2 ** (bits - 1) - 1))
        delta = delta16.astype(np.float32)
        z = np.full(delta.shape, 2 ** (bits - 1), dtype=np.int32)
    code = np.rint(g / delta[:, :, None]) + z[:, :, None].astype(np.float32)
    q = np.clip(code, 0, Q).astype(np.uint8)
    return q.reshape(N, K), delta16, z.astype(np.float16)


def dequantize(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               group_size: int = GROUP_SIZE) -> np.ndarray:
    """w_hat[n, k] = (q[n, k] - z[n, g]) * D[n, g] in fp64 (exact).

    This is the "fake quantization" weight of [P1] "Usage" step 2.
    """
    N, K = q.shape
    G = K // group_size
    qq = q.astype(np.float64).reshape(N, G, group_size)
    zz = zeros.astype(np.float64)[:, :, None]
    dd = scales.astype(np.float64)[:, :, None]
    return ((qq - zz) * dd).reshape(N, K)


# ---------------------------------------------------------------------------
# a6: packing (format version 3, chosen for gfx950)
# ---------------------------------------------------------------------------
ROW_BLOCK = 16          # rows of one packed tile
QUARTER = 32            # codes of one lane slot in a tile


def words_per_quarter(bits: int) -> int:
    return 4 if bits == 4 else 3


def pack_rows(q: np.ndarray, bits: int) -> np.ndarray:
    """Bit-pack each row of codes q uint8 [N][K] into uint32 words [N][W].

    bits=4 (W = K/8): word j of a row holds codes k = 8j..8j+7; code 8j+2t
    is at bits 4t..4t+3 and code 8j+2t+1 at bits 16+4t..19+4t (t = 0..3),
    so (word >> 4t) & 0x000F000F holds the pair (q[8j+2t], q[8j+2t+1]) in
    its two 16-bit halves.
    bits=3 (W = 3K/32): each run of 32 codes c_0..c_31 (k = 32r + i) fills 3
    words.  Pair P = (c_2P, c_2P+1), P = 0..14, sits in word P // 5 with c_2P
    at bits 3t..3t+2 and c_2P+1 at bits 16+3t..18+3t (t = P % 5), so that
    (word >> 3t) & 0x00070007 holds the pair in its two 16-bit halves, like
    the int4 nibble pairs; the last pair spreads over the spare bits: bit b of
    c_30 is bit 15 of word b, bit b of c_31 is bit 31 of word b.
    """
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    Q = levels(bits)
    if q.max(initial=0) > Q:
        raise ValueError("code out of range")
    if bits == 4:
        c = q.reshape(N, K // 8, 8).astype(np.uint32)
        word = np.zeros((N, K // 8), dtype=np.uint32)
        for t in range(4):
            word |= c[:, :, 2 * t] << np.uint32(4 * t)
            word |= c[:, :, 2 * t + 1] << np.uint32(16 + 4 * t)
        return word
    c = q.reshape(N, K // 32, 32).astype(np.uint32)
    out = np.zeros((N, K // 32, 3), dtype=np.uint32)
    for P in range(15):
        w, t = divmod(P, 5)
        out[:, :, w] |= c[:, :, 2 * P] << np.uint32(3 * t)
        out[:, :, w] |= c[:, :, 2 * P + 1] << np.uint32(16 + 3 * t)
    for b in range(3):
        out[:, :, b] |= ((c[:, :, 30] >> np.uint32(b)) & np.uint32(1)) << np.uint32(15)
        out[:, :, b] |= ((c[:, :, 31] >> np.uint32(b)) & np.uint32(1)) << np.uint32(31)
    return out.reshape(N, 3 * (K // 32))


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Packed weights, format 3: tiles of 16 rows x 128 codes (one 128-group or
    two 64-groups; the codes' layout does not depend on the group size).
    Format 3 is format 2 with the int3 pair layout of ``pack_rows`` (int4 as
    before).

    The row words of ``pack_rows`` are regrouped so that the 16 rows of
    block b and the group g form one contiguous tile of 64 lane slots:
    slot s = 16h + j holds the words of row n = 16b + j that cover codes
    k = 128g + 32h .. 128g + 32h + 31 (4 words for bits 4, 3 for bits 3).
    Result shape [ceil(N/16)][G][64][4 or 3]; rows past N are zero.
    Reading: the pages say only that the packing is chosen per platform
    ("platform-aware weight packing"); this order makes one tile one
    contiguous 1 KB load whose lane slots are the MFMA operand layout.
    """
    rows = pack_rows(q, bits)
    N, K = np.asarray(q).shape
    W = words_per_quarter(bits)
    NB, G = -(-N // ROW_BLOCK), K // GROUP_SIZE
    padded = np.zeros((NB * ROW_BLOCK, rows.shape[1]), dtype=np.uint32)
    padded[:N] = rows
    t = padded.reshape(NB, ROW_BLOCK, G, 4, W)          # [b][j][g][h][i]
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1, 4)).reshape(NB, G, 64, W)


def tile_params(p: np.ndarray) -> np.ndarray:
    """Scales or zeros [N][G] -> format-2 layout [ceil(N/16)][G][16] (zero padded).

    Element (n, g) moves to [n // 16][g][n % 16]: the 16 rows of a row block
    sit side by side for each group, next to the tile they scale.
    """
    p = np.asarray(p)
    N, G = p.shape
    NB = -(-N // ROW_BLOCK)
    out = np.zeros((NB * ROW_BLOCK, G), dtype=p.dtype)
    out[:N] = p
    return np.ascontiguousarray(out.reshape(NB, ROW_BLOCK, G).transpose(0, 2, 1))


def untile_params(t: np.ndarray, N: int) -> np.ndarray:
    """Inverse of ``tile_params`` ([ceil(N/16)][G][16] -> [N][G])."""
    t = np.asarray(t)
    NB, G = t.shape[0], t.shape[1]
    return np.ascontiguousarray(t.reshape(NB, G, ROW_BLOCK).transpose(0, 2, 1)).reshape(NB * ROW_BLOCK, G)[:N]


def packed_words(N: int, K: int, bits: int) -> int:
    """uint32 words of a packed weight matrix (rows padded to 16)."""
    return -(-N // ROW_BLOCK) * ROW_BLOCK * packed_words_per_row(K, bits)


def unpack(words: np.ndarray, bits: int, K: int, N: int | None = None) -> np.ndarray:
    """Inverse of ``pack``: locate every code's bits one by one."""
    W = words_per_quarter(bits)
    words = np.asarray(words, dtype=np.uint32)
    NB = words.size // ((K // GROUP_SIZE) * 64 * W)
    t = words.reshape(NB, K // GROUP_SIZE, 64, W)
    N = NB * ROW_BLOCK if N is None else N
    q = np.zeros((N, K), dtype=np.uint8)
    for k in range(K):
        g, r = divmod(k, GROUP_SIZE)
        h, kk = divmod(r, QUARTER)                 # quarter and code within it
        for b in range(bits):
            if bits == 4:
                i, e = divmod(kk, 8)
                pos = 4 * (e // 2) + 16 * (e % 2) + b
            else:
                P, odd = divmod(kk, 2)
                if P < 15:
                    i, tp = divmod(P, 5)
                    pos = 3 * tp + 16 * odd + b
                else:
                    i, pos = b, 15 + 16 * odd
            for n in range(N):
                blk, j = divmod(n, ROW_BLOCK)
                w = t[blk, g, 16 * h + j, i]
                q[n, k] |= np.uint8(((int(w) >> pos) & 1) << b)
    return q


def packed_words_per_row(K: int, bits: int) -> int:
    return K // 8 if bits == 4 else 3 * (K // 32)


def fake_quantize(qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                  bits: int, K: int) -> np.ndarray:
    """w_hat as fp16 [N][K] from the packed layer: fp16_rne((q - z) * D).

    [P1] "Usage" step 2 (--q_backend fake): the quantized weights are kept as
    dequantized fp16 values for evaluation.  (q - z) * D is exact in fp64 (a
    small integer times an fp16 value), so this is its single rounding to fp16.
    The group size comes from the [N][G] parameters.
    """
    N, G = np.asarray(scales).shape
    q = unpack_fast(qweight, bits, K, N)
    return dequantize(q, scales, zeros, K // G).astype(np.float16)


# ---------------------------------------------------------------------------
# a7: activation-side half of the equivalent transform
# ---------------------------------------------------------------------------
def scale_activations(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x'[m, k] = fp16_rne(fp32(x[m, k]) / s[k]).

    [P5] 02.02: (x / s) . (s w) = x . w; the weights carry s inside the
    quantizer, the activations are divided by it.
    """
    x32 = np.asarray(x, dtype=np.float16).astype(np.float32)
    return (x32 / np.asarray(s, dtype=np.float32)[None, :]).astype(np.float16)


def apply_inv_scale(x: np.ndarray, inv_s: np.ndarray) -> np.ndarray:
    """x'[m, k] = fp16_rne(fp32(x[m, k]) * inv_s[k]).

    The same activation side of the [P5] 02.02 transform as
    ``scale_activations``, with the caller's reciprocal 1/s instead of s
    (reading: the matmul entry points that fold the scale into their
    activation load take inv_s, as the fused modules of "transformers - AWQ"
    fold it into the layer before).  With inv_s = fp32(1/s) the result equals
    fp16_rne(x / s) except where x/s lies within an fp32 ulp of an fp16
    rounding boundary, and then differs by one fp16 ulp.
    """
    x32 = np.asarray(x, dtype=np.float16).astype(np.float32)
    with np.errstate(over="ignore"):
        return (x32 * np.asarray(inv_s, dtype=np.float32)[None, :]).astype(np.float16)


# ---------------------------------------------------------------------------
# a8 / a9 / a10: the W4A16 (W3A16) matmul
# ---------------------------------------------------------------------------
def matmul(x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
           zeros: np.ndarray, bits: int, K: int) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * w_hat[n, k], fp64, from the packed weights.

    [P1] feature list: the 4-bit linear layer and its context (GEMM) and
    decode (GEMV) kernels compute this one product.
    """
    N, G = np.asarray(scales).shape
    q = unpack_fast(qweight, bits, K, N)
    w_hat = dequantize(q, scales, zeros, K // G)        # group size from the [N][G] parameters
    return np.asarray(x, dtype=np.float16).astype(np.float64) @ w_hat.T


def tiles_to_rows(words: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Row words [ceil(N/16)*16][W] of a format-2 array (inverse regrouping)."""
    W = words_per_quarter(bits)
    t = np.asarray(words, dtype=np.uint32).reshape(-1, K // GROUP_SIZE, 4, ROW_BLOCK, W)
    NB = t.shape[0]                                            # [b][g][h][j][i]
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2, 4)).reshape(NB * ROW_BLOCK, -1)


def unpack_fast(words: np.ndarray, bits: int, K: int, N: int | None = None) -> np.ndarray:
    """Vectorised inverse of ``pack`` (same format; checked against ``unpack``)."""
    rows = tiles_to_rows(words, bits, K)
    N = rows.shape[0] if N is None else N
    rows = rows[:N]
    if bits == 4:
        w = rows.reshape(N, K // 8, 1)
        r = np.arange(8, dtype=np.uint32)
        shift = 4 * (r // 2) + 16 * (r % 2)
        return ((w >> shift[None, None, :]) & np.uint32(15)).astype(np.uint8).reshape(N, K)
    w = rows.reshape(N, K // 32, 3)
    q = np.zeros((N, K // 32, 32), dtype=np.uint8)
    for P in range(15):
        wi, t = divmod(P, 5)
        q[:, :, 2 * P] = ((w[:, :, wi] >> np.uint32(3 * t)) & np.uint32(7)).astype(np.uint8)
        q[:, :, 2 * P + 1] = ((w[:, :, wi] >> np.uint32(16 + 3 * t)) & np.uint32(7)).astype(np.uint8)
    for b in range(3):
        q[:, :, 30] |= (((w[:, :, b] >> np.uint32(15)) & np.uint32(1)) << np.uint32(b)).astype(np.uint8)
        q[:, :, 31] |= (((w[:, :, b] >> np.uint32(31)) & np.uint32(1)) << np.uint32(b)).astype(np.uint8)
    return q.reshape(N, K)


def matmul_rows(x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                zeros: np.ndarray, bits: int, K: int, rows) -> np.ndarray:
    """Output columns y[:, rows] only (for sampled checks at full size)."""
    rows = np.asarray(rows)
    W = words_per_quarter(bits)
    t = np.asarray(qweight, dtype=np.uint32).reshape(-1, K // GROUP_SIZE, 4, ROW_BLOCK, W)
    blk, j = rows // ROW_BLOCK, rows % ROW_BLOCK
    sel = t[blk, :, :, j, :]                                   # [len(rows)][G][h][i]
    q = unpack_fast(sel[:, :, :, None, :].repeat(ROW_BLOCK, axis=3), bits, K)
    q = q.reshape(len(rows), ROW_BLOCK, K)[:, 0, :]
    w_hat = dequantize(q, scales[rows], zeros[rows], K // np.asarray(scales).shape[1])
    return np.asarray(x, dtype=np.float16).astype(np.float64) @ w_hat.T


# ---------------------------------------------------------------------------
# f4: the gate/up half of the fused MLP ("transformers - AWQ", "Fused modules")
# ---------------------------------------------------------------------------
def silu(t) -> np.ndarray:
    """SiLU(t) = t * sigmoid(t) = t / (1 + exp(-t)), fp64.

    Reading: the pages fuse an MLP of gate, up and down layers for the Llama
    and Mistral architectures without naming its activation; those
    architectures use SiLU on the gate output, times the up output.
    """
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def gate_up(x: np.ndarray, inv_s, gate, up, bits: int, K: int) -> np.ndarray:
    """h[m, n] = SiLU(g[m, n]) * u[m, n], fp64, with g = x' . w_hat_gate^T and
    u = x' . w_hat_up^T from the packed layers gate = (qweight, scales, zeros)
    and up likewise; x' = apply_inv_scale(x, inv_s), or x when inv_s is None
    (gate and up read the same input, so they share one scale).

    "transformers - AWQ", "Fused modules": the MLP's gate, up and down layers
    fused into one module; this is the part ahead of the down projection.
    """
    xs = np.asarray(x, dtype=np.float16) if inv_s is None else apply_inv_scale(x, inv_s)
    g = matmul(xs, *gate, bits, K)
    u = matmul(xs, *up, bits, K)
    return silu(g) * u


def gate_up_rows(x: np.ndarray, inv_s, gate, up, bits: int, K: int, rows) -> np.ndarray:
    """Output columns h[:, rows] of ``gate_up`` only (sampled checks at full size)."""
    xs = np.asarray(x, dtype=np.float16) if inv_s is None else apply_inv_scale(x, inv_s)
    g = matmul_rows(xs, *gate, bits, K, rows)
    u = matmul_rows(xs, *up, bits, K, rows)
    return silu(g) * u


# ---------------------------------------------------------------------------
# a4 / a5: output-MSE loss and the alpha grid search
# ---------------------------------------------------------------------------
def output_mse(X_cal: np.ndarray, W: np.ndarray, w_hat: np.ndarray,
               s: np.ndarray) -> float:
    """L = mean over (t, n) of (sum_k X[t,k] (W[n,k] - w_hat[n,k] / s[k]))^2.

    The layer's own fp16 output X.W^T against the output of the deployed
    pair (X / s).(w_hat)^T, in exact arithmetic; fp64.  Reading: the MSE is
    of this single linear layer, averaged over calibration tokens and output
    channels.
    """
    X = np.asarray(X_cal, dtype=np.float16).astype(np.float64)
    D = np.asarray(W, dtype=np.float16).astype(np.float64) - w_hat / np.asarray(s, np.float32).astype(np.float64)[None, :]
    E = X @ D.T
    return float(np.mean(E * E))


def search_scale(W: np.ndarray, X_cal: np.ndarray, alphas, bits: int = 4,
                 group_size: int = GROUP_SIZE, zero_point: bool = True):
    """Grid search of alpha minimising the layer's output MSE.

    [P1] "Usage" step 1 (--run_awq: search and save the per-channel scales),
    [P5] 02.02 (scale from offline activation statistics, no backprop).
    For each alpha_i: s_i = candidate_scale(s_x, alpha_i), quantize W with
    s_i, L_i = output_mse.  The smallest i attaining min L_i is chosen.
    Returns (s_best fp32 [K], losses fp64 [n_alpha], best index).
    """
    s_x = act_stat(X_cal)
    losses = []
    for a in alphas:
        s = candidate_scale(s_x, a)
        q, d, z = quantize(W, s, bits, group_size, zero_point)
        losses.append(output_mse(X_cal, W, dequantize(q, d, z, group_size), s))
    losses = np.asarray(losses, dtype=np.float64)
    best = int(np.argmin(losses))                   # first minimum
    return candidate_scale(s_x, alphas[best]), losses, best


def search_scale_shared(Ws, X_cal: np.ndarray, alphas, bits: int = 4,
                        group_size: int = GROUP_SIZE, zero_point: bool = True):
    """One alpha (one s) for several layers that read the same input.

    [P5] 02.02: the activations are divided by s once, before the layers that
    read them, so every layer fed by that input must carry the same s
    (reading: q/k/v after one norm, gate/up after another); [P1] "Usage"
    step 1 searches per model.  Reading: the loss is the output MSE over all
    the layers' outputs together, i.e. the search of the layer whose rows are
    the layers' rows one after the other -- so it is that search, written out.
    Returns (s_best fp32 [K], losses fp64 [n_alpha], best index).
    """
    W = np.concatenate([np.asarray(w, dtype=np.float16) for w in Ws], axis=0)
    return search_scale(W, X_cal, alphas, bits, group_size, zero_point)


# ---------------------------------------------------------------------------
# f2: the gate/up scale searched on the MLP block's output
# ---------------------------------------------------------------------------
def mlp_block_loss(X_cal: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
                   s: np.ndarray, bits: int = 4, group_size: int = GROUP_SIZE,
                   zero_point: bool = True) -> float:
    """L = mean over tokens t and block outputs o of (y_q[t, o] - y[t, o])^2 for
    the MLP block y = (SiLU(X Wg^T) * (X Wu^T)) Wd^T, where y_q has the gate and
    up weights quantized with the activation scale s (the deployed pair
    (X / s).w_hat^T, i.e. X.(w_hat / s)^T) and the down projection Wd kept as it
    is; fp64 throughout.

    Reading: "Usage" step 1 of the llm-awq README searches the scales per
    model; gate and up read one input, so they share one s (section 02.02 of
    the VPTQ blog: the activations are divided by s once), and the error that
    matters is that of the block those two layers feed -- the MLP's output
    after SiLU(gate) * up and the down projection ("transformers - AWQ", "Fused
    modules": the MLP as gate, up and down).  Wg, Wu fp16 [I][K]; Wd fp16
    [K_out][I]; X_cal fp16 [T][K].
    """
    X = np.asarray(X_cal, dtype=np.float16).astype(np.float64)
    s64 = np.asarray(s, np.float32).astype(np.float64)
    hats = []
    for W in (Wg, Wu):
        q, d, z = quantize(W, s, bits, group_size, zero_point)
        hats.append(dequantize(q, d, z, group_size) / s64[None, :])
    Wg64, Wu64 = (np.asarray(w, np.float16).astype(np.float64) for w in (Wg, Wu))
    h_q = silu(X @ hats[0].T) * (X @ hats[1].T)
    h = silu(X @ Wg64.T) * (X @ Wu64.T)
    E = (h_q - h) @ np.asarray(Wd, np.float16).astype(np.float64).T
    return float(np.mean(E * E))


def search_scale_mlp(X_cal: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, alphas,
                     bits: int = 4, group_size: int = GROUP_SIZE, zero_point: bool = True):
    """The alpha grid search of the gate/up pair's shared scale on the MLP
    block's output error (``mlp_block_loss``): s_i = candidate_scale(s_x,
    alpha_i), the first index of the smallest loss is chosen.  Returns
    (s_best fp32 [K], losses fp64 [n_alpha], best index)."""
    s_x = act_stat(X_cal)
    losses = np.asarray([mlp_block_loss(X_cal, Wg, Wu, Wd, candidate_scale(s_x, a), bits, group_size,
                                        zero_point) for a in alphas], dtype=np.float64)
    best = int(np.argmin(losses))
    return candidate_scale(s_x, alphas[best]), losses, best
