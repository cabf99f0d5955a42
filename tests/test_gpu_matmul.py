"""GPU parity: awq_gemv and awq_gemm vs the oracle's fp64 product.

Bar: max|y - y_ref| / max|y_ref| <= 2e-3 over the compared outputs, with the
weights packed by the oracle (so the matmul is checked on its own).
"""
import numpy as np
import pytest

import oracle as O
import weight_only_quantization_pack_amd as awq
from weight_only_quantization_pack_amd import workloads as WL

from gpu_util import TOL, announce, dev, guarded_empty, host, rel_err, sentinel_intact

pytestmark = pytest.mark.gpu


def packed(W, bits, s=None, chunk=2048, group_size=128):
    """Oracle quantize + pack, in row chunks to bound host memory."""
    parts = []
    for r in range(0, W.shape[0], chunk):
        q, d, z = O.quantize(W[r:r + chunk], s, bits, group_size)
        parts.append((O.pack(q, bits), d, z))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


_CACHE = {}


def workload_layer(w, shape_index, bits=4):
    """(W, qweight, scales, zeros) of a workload layer, packed by the oracle once."""
    key = (w, shape_index, bits)
    if key not in _CACHE:
        _CACHE.clear()
        W = WL.workload(w).weights(shape_index)
        _CACHE[key] = (W,) + packed(W, bits)
    return _CACHE[key]


def run(fn, x, qw, d, z, N, bits, group_size=128):
    import torch
    y = getattr(awq, fn)(dev(x), dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)),
                         N=N, bits=bits, group_size=group_size)
    torch.cuda.synchronize()
    return host(y).astype(np.float64)


def check(fn, M, N, K, bits, seed, sigma=1.0, rows=None, layer=None, x=None, group_size=128):
    announce(fn, f"M={M} N={N} K={K} bits={bits} group_size={group_size} seed={seed}")
    if layer is None:
        qw, d, z = packed(WL.random_weights(N, K, seed=seed), bits, group_size=group_size)
    else:
        _, qw, d, z = layer
    x = WL.random_activations(M, K, seed=seed + 1, sigma=sigma) if x is None else x
    y = run(fn, x, qw, d, z, N, bits, group_size)
    if rows is None:
        y_ref = O.matmul(x, qw, d, z, bits, K)
        err = rel_err(y, y_ref)
    else:
        y_ref = O.matmul_rows(x, qw, d, z, bits, K, rows)
        err = rel_err(y[:, rows], y_ref)
    assert err <= TOL, f"{fn} M={M} N={N} K={K} bits={bits}: rel err {err:.3e}"
    return y


# ----------------------------------------------------------------------------- GEMV
@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M", [1, 2, 4, 5, 8, 16])
# (8300, 1408) and (9000, 384): more 16-row blocks than persistent workgroups
# (some take two) while the waves' group counts are ragged (11 and 3 groups)
@pytest.mark.parametrize("N,K", [(512, 512), (37, 384), (1, 128), (130, 11008), (8300, 1408), (9000, 384)])
def test_gemv_small(gpu, bits, M, N, K):
    check("gemv", M, N, K, bits, seed=100 + M + N + K)


@pytest.mark.parametrize("shape_index", [0, 1, 2])
def test_gemv_workload2_full(gpu, shape_index):
    wl = WL.workload(2)
    K, N = wl.shapes[shape_index]
    check("gemv", 1, N, K, 4, seed=0, layer=workload_layer(2, shape_index),
          x=wl.activations(1, shape_index))


@pytest.mark.parametrize("shape_index", [0, 1])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_workload3_full(gpu, M, shape_index):
    """Llama-70B MLP shapes, whole output tensor.  8192x28672 (1792 row blocks)
    takes the 4-wave sliced kernel at M = 4 and 16; 28672x8192 at M = 16 the
    sliced kernel with two row blocks per workgroup (rows >= 16384, M >= 8)."""
    wl = WL.workload(3)
    K, N = wl.shapes[shape_index]
    check("gemv", M, N, K, 4, seed=0, layer=workload_layer(3, shape_index),
          x=wl.activations(M, shape_index))


@pytest.mark.parametrize("M", [5, 16])
def test_gemv_sliced_two_blocks_per_workgroup(gpu, M):
    """x too large to stage at once (K sliced) with 1019 row blocks over at most
    512 persistent workgroups: each owns two blocks, some only one valid."""
    N, K = 16300, 4096
    check("gemv", M, N, K, 4, seed=31 + M)


@pytest.mark.parametrize("M,bits,group_size", [(5, 4, 128), (16, 3, 128), (8, 4, 64)])
def test_gemv_sliced_wide_layer(gpu, M, bits, group_size):
    """K sliced on a layer of 1025 row blocks (the 4-wave workgroup form, slices
    of 8 groups): K = 4736 leaves a ragged last slice of 5 groups, and N = 16393
    a last block with one valid row."""
    N, K = 16393, 4736
    check("gemv", M, N, K, bits, seed=37 + M, group_size=group_size)


@pytest.mark.parametrize("M", [8, 13])
def test_gemv_sliced_long_rows_two_blocks(gpu, M):
    """K >= 16384 at M >= 8 with at least two blocks per CU: two row blocks per
    workgroup.  N = 8200 gives 513 blocks (the last workgroup holds one valid
    block) and K = 16512 a ragged last slice of one group."""
    N, K = 8200, 16512
    key = ("long_rows", N, K)
    if key not in _CACHE:
        _CACHE.clear()
        W = WL.random_weights(N, K, seed=91)
        _CACHE[key] = (W,) + packed(W, 4)
    check("gemv", M, N, K, 4, seed=92 + M, layer=_CACHE[key])


# x staged once with 12 16-byte x loads per lane (the largest staging of the
# one-pass kernel: M * (K + 8) * 2 <= 64 KB with 33-48 (group, row) pairs per
# wave): M = 3 with K = 10368 (81 groups, 11 per wave), M = 5 with K = 6400,
# M = 7 with K = 4480, M = 15 with K = 2176 (17 groups: 3 per wave, 45 pairs)
X1_XL12 = [(3, 1000, 10368), (5, 300, 6400), (7, 130, 4480), (15, 600, 2176)]


@pytest.mark.parametrize("group_size", [128, 64])
@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M,N,K", X1_XL12)
def test_gemv_x1_twelve_loads(gpu, M, N, K, bits, group_size):
    assert M * (K + 8) * 2 <= 65536 and ((-(-K // 128 // 8)) * M + 3) // 4 > 8
    check("gemv", M, N, K, bits, seed=500 + M + K, group_size=group_size)


# ----------------------------------------------------------------------------- 64-wide groups
@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("fn,M,N,K", [
    ("gemv", 1, 300, 4096),        # x staged once, short rows (ring of 2)
    ("gemv", 4, 130, 11008),       # 4 x 11008 > 32K halves: K in slices, ragged last slice
    ("gemv", 16, 1000, 2048),      # K slices, one 16-group slice
    ("gemm", 5, 302, 2048),        # split K, 16-row tiles
    ("gemm", 20, 302, 2048),       # split K, 32-row tiles
    ("gemm", 257, 200, 1152),      # several M tiles, no split
])
def test_group64_matmuls(gpu, fn, M, N, K, bits):
    check(fn, M, N, K, bits, seed=400 + M + N, group_size=64)


# ----------------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M", [1, 5, 64, 128, 130, 257])
@pytest.mark.parametrize("N,K", [(512, 512), (37, 384), (200, 1152)])
def test_gemm_small(gpu, M, N, K, bits):
    check("gemm", M, N, K, bits, seed=200 + M + N + K)


@pytest.mark.parametrize("M", [256, 2048])
def test_gemm_int3_many_tiles(gpu, M):
    """int3 with more tiles than CUs (the pipelined kernel in rounds)."""
    N, K = 4096, 1024
    check("gemm", M, N, K, 3, seed=7)


@pytest.mark.parametrize("bits,group_size", [(4, 128), (3, 128), (4, 64)])
@pytest.mark.parametrize("N,width", [(14296, 448), (6100, 384)])
@pytest.mark.parametrize("M", [2048, 1999])
def test_gemm_wide_tiles(gpu, M, N, width, bits, group_size):
    """M = 2048 or 1999 (16 row tiles, the last one ragged) on 256 CUs: N =
    14296 takes 128 x 448 tiles (7 column blocks per wave; 512 tiles, two
    rounds) and N = 6100 128 x 384 tiles (6 per wave; 256 tiles).  Both end in
    a ragged tile whose last waves' columns lie past N; the whole output is
    compared."""
    K = 1024
    check("gemm", M, N, K, bits, seed=31 + bits, group_size=group_size)


def test_gemm_two_workgroups_per_cu(gpu):
    """M = 2048, N = 8192 on 256 CUs: 512 tiles of 128 x 256 columns, run by the
    double-buffered kernel at two workgroups per CU (one round of 512 slots)."""
    M, N, K = 2048, 8192, 1024
    check("gemm", M, N, K, 4, seed=41)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M,N,K", [(5, 302, 2048), (130, 200, 4736), (64, 1000, 8192)])
def test_gemm_split_k(gpu, M, N, K, bits):
    """Few output tiles: K split over workgroups (fp32 partials + ordered sum).
    (130, 200, 4736): 37 groups in splits of 10, 10, 10, 7; N = 302: the
    scalar tails of the partial store and of the reduction."""
    import torch
    assert awq.gemm_splitk_workspace_bytes(M, N, K) > 0
    qw, d, z = packed(WL.random_weights(N, K, seed=N + K), bits)
    x = WL.random_activations(M, K, seed=M + 1, sigma=1.0)
    announce("gemm split-K", f"M={M} N={N} K={K} bits={bits}")
    y_ref = O.matmul(x, qw, d, z, bits, K)
    args = (dev(x), dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)))
    for split in (True, False):
        y = awq.gemm(*args, N=N, bits=bits, split_k=split)
        torch.cuda.synchronize()
        err = rel_err(host(y).astype(np.float64), y_ref)
        assert err <= TOL, f"split_k={split}: rel err {err:.3e}"


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M", [16, 17, 24, 32, 33, 48, 64])
@pytest.mark.parametrize("N,K", [(302, 2048), (1000, 1152)])
def test_gemm_row_tile_heights(gpu, M, N, K, bits):
    """The pipelined kernel's 16-, 32- and 64-row tiles around their limits
    (M = 16 | 17, 32 | 33; M = 24 and 48 leave padding rows in a 32- and a
    64-row tile; 16-row tiles are 64 columns wide, 32- and 64-row ones 128, so
    N = 302 and 1000 end in a partial column tile), with and without the K
    split, whole output."""
    import torch
    qw, d, z = packed(WL.random_weights(N, K, seed=N + K + M), bits)
    x = WL.random_activations(M, K, seed=M + 11, sigma=1.0)
    announce("gemm row tiles", f"M={M} N={N} K={K} bits={bits}")
    y_ref = O.matmul(x, qw, d, z, bits, K)
    args = (dev(x), dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)))
    for split in (True, False):
        y = awq.gemm(*args, N=N, bits=bits, split_k=split)
        torch.cuda.synchronize()
        err = rel_err(host(y).astype(np.float64), y_ref)
        assert err <= TOL, f"split_k={split}: rel err {err:.3e}"


@pytest.mark.parametrize("shape_index", [0, 1, 2])
@pytest.mark.parametrize("M", [512, 2048])
def test_gemm_workload4_full(gpu, M, shape_index):
    """Mistral-7B prefill shapes at M = 512 (split K) and 2048 (the tiles the
    benchmark times), whole output tensor."""
    wl = WL.workload(4)
    K, N = wl.shapes[shape_index]
    check("gemm", M, N, K, 4, seed=0, layer=workload_layer(4, shape_index),
          x=wl.activations(M, shape_index))


@pytest.mark.parametrize("shape_index", [0, 1])
@pytest.mark.parametrize("M", [64, 16])
def test_gemm_workload3_full(gpu, M, shape_index):
    """Llama-70B MLP shapes at M = 64 and 16 (64- and 16-row tiles, split
    K), whole tensor."""
    wl = WL.workload(3)
    K, N = wl.shapes[shape_index]
    check("gemm", M, N, K, 4, seed=0, layer=workload_layer(3, shape_index),
          x=wl.activations(M, shape_index))


# ----------------------------------------------------------------------------- exact cases
@pytest.mark.parametrize("fn,bits", [("gemv", 4), ("gemv", 3), ("gemm", 4), ("gemm", 3)])
def test_one_hot_rows_are_exact(gpu, fn, bits):
    """x = e_k picks column k of w_hat; with D = 2^-4 every value is an exact fp16."""
    K, N = 256, 48
    rng = np.random.default_rng(77)
    Q = (1 << bits) - 1
    q = rng.integers(0, Q + 1, (N, K)).astype(np.uint8)
    d = np.full((N, K // 128), 2.0 ** -4, np.float16)
    z = rng.integers(0, Q + 1, (N, K // 128)).astype(np.float16)
    qw = O.pack(q, bits)
    ks = [0, 1, 2, 7, 8, 31, 32, 127, 128, 200, 255]
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    w_hat = O.dequantize(q, d, z)
    announce(fn, "one-hot", bits)
    if fn == "gemv":
        ys = np.concatenate([run(fn, x[i:i + 1], qw, d, z, N, bits) for i in range(len(ks))])
    else:
        ys = run(fn, x, qw, d, z, N, bits)
    for i, k in enumerate(ks):
        assert np.array_equal(ys[i], w_hat[:, k]), f"column {k}"


def test_gemv_equals_gemm_at_m1(gpu):
    W = WL.random_weights(300, 2048, seed=8)
    x = WL.random_activations(1, 2048, seed=9)
    qw, d, z = packed(W, 4)
    a = run("gemv", x, qw, d, z, 300, 4)
    b = run("gemm", x, qw, d, z, 300, 4)
    assert rel_err(a, b) <= TOL


@pytest.mark.parametrize("fn,K", [("gemv", 384), ("gemm", 384), ("gemm", 2048)])
def test_no_write_past_output_and_repeatable(gpu, fn, K):
    """K = 2048 with 3 rows: the GEMM splits K (fp32 partials + reduction)."""
    import torch
    M, N = 3, 37
    W = WL.random_weights(N, K, seed=12)
    x = WL.random_activations(M, K, seed=13)
    qw, d, z = packed(W, 4)
    y, raw, n = guarded_empty((M, N), torch.float16)
    args = (dev(x), dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)))
    announce(fn, "guarded", M, N, K)
    getattr(awq, fn)(*args, N=N, bits=4, out=y)
    first = host(y).copy()
    getattr(awq, fn)(*args, N=N, bits=4, out=y)
    torch.cuda.synchronize()
    assert np.array_equal(first.view(np.uint16), host(y).view(np.uint16))
    assert sentinel_intact(raw, n)


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
def test_empty_calls(gpu, fn):
    import torch
    qw, d, z = packed(WL.random_weights(8, 128, seed=1), 4)
    x = torch.empty((0, 128), dtype=torch.float16, device="cuda:0")
    y = getattr(awq, fn)(x, dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)),
                         N=8, bits=4)
    assert tuple(y.shape) == (0, 8)


# ----------------------------------------------------------------------------- folded scale (prefill)
# (M, N, K): every tile form of the pipelined kernel with the scale folded into
# its activation tiles -- 16-, 32- and 64-row tiles with split K (M = 5, 17,
# 32, 64), 128-row 8 x 2
# tiles with a ragged split (130 x 200 x 4736: 37 groups in splits of 10, 10,
# 10, 7), several row tiles, 4 x 7 (N = 14296) and 8 x 3 (N = 6100) wide tiles
# with ragged edges, and N = 8192 at M = 2048, where awq_gemm takes the
# two-workgroups-per-CU kernel but the scaled product the 8 x 2 tiles
SCALED_GEMM = [(5, 302, 2048), (17, 302, 2048), (32, 1000, 4736), (64, 1000, 8192), (130, 200, 4736),
               (257, 600, 1152),
               (2048, 14296, 1024), (1999, 6100, 1024), (2048, 8192, 1024)]


def _inv_scale(K, seed):
    s = np.random.default_rng(seed).lognormal(0, 1, K).astype(np.float32)
    return (np.float32(1) / s).astype(np.float32)


@pytest.mark.parametrize("bits,group_size", [(4, 128), (3, 128), (4, 64)])
@pytest.mark.parametrize("M,N,K", SCALED_GEMM)
def test_gemm_scaled(gpu, M, N, K, bits, group_size):
    """awq_gemm_scaled within the matmul bar of the oracle's product of
    x' = fp16(fp32(x) * inv_s), and bit-identical to awq_gemm on the oracle's
    x' wherever both take the same kernel (the scale is applied exactly in LDS
    before any MFMA reads the tile)."""
    import torch
    announce("gemm_scaled", f"M={M} N={N} K={K} bits={bits} gs={group_size}")
    qw, d, z = packed(WL.random_weights(N, K, seed=N + K), bits, group_size=group_size)
    x = WL.random_activations(M, K, seed=M + 3, sigma=1.5)
    inv_s = _inv_scale(K, K + 5)
    xs = O.apply_inv_scale(x, inv_s)
    args = (dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)))
    y = awq.gemm(dev(x), *args, N=N, bits=bits, group_size=group_size, inv_s=dev(inv_s))
    y_plain = awq.gemm(dev(xs), *args, N=N, bits=bits, group_size=group_size)
    torch.cuda.synchronize()
    err = rel_err(host(y).astype(np.float64), O.matmul(xs, qw, d, z, bits, K))
    assert err <= TOL, f"rel err {err:.3e}"
    if not (M, N, K) == (2048, 8192, 1024) or (bits, group_size) != (4, 128):
        assert np.array_equal(host(y).view(np.uint16), host(y_plain).view(np.uint16))


@pytest.mark.parametrize("M", [5, 130])
def test_gemm_scaled_without_split(gpu, M):
    """No workspace: the scaled product runs without a K split (one launch)."""
    import torch
    N, K = 302, 4736
    qw, d, z = packed(WL.random_weights(N, K, seed=3), 4)
    x = WL.random_activations(M, K, seed=4, sigma=1.5)
    inv_s = _inv_scale(K, 6)
    announce("gemm_scaled no split", M, N, K)
    y = awq.gemm(dev(x), dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)), N=N,
                 bits=4, inv_s=dev(inv_s), split_k=False)
    torch.cuda.synchronize()
    err = rel_err(host(y).astype(np.float64), O.matmul(O.apply_inv_scale(x, inv_s), qw, d, z, 4, K))
    assert err <= TOL, f"rel err {err:.3e}"


@pytest.mark.parametrize("shape_index", [0, 1, 2])
def test_gemm_scaled_workload4_full(gpu, shape_index):
    """Mistral-7B prefill shapes at M = 2048 with the folded scale, whole tensor."""
    import torch
    wl = WL.workload(4)
    K, N = wl.shapes[shape_index]
    _, qw, d, z = workload_layer(4, shape_index)
    x = wl.activations(2048, shape_index)
    inv_s = _inv_scale(K, 11)
    announce("gemm_scaled workload 4", K, N)
    y = awq.gemm(dev(x), dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)), N=N,
                 bits=4, inv_s=dev(inv_s))
    torch.cuda.synchronize()
    err = rel_err(host(y).astype(np.float64), O.matmul(O.apply_inv_scale(x, inv_s), qw, d, z, 4, K))
    assert err <= TOL, f"rel err {err:.3e}"
