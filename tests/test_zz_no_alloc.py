"""awq_gemm_splitk_noalloc (split-K partials in the library's fixed per-GPU
array, no allocation) against awq_gemm_splitk with a caller workspace: the
same kernels and split count, so the outputs must agree bit for bit, and both
within the matmul bar of the oracle's fp64 product.  Two calls in a row, the
second on a smaller problem (the array keeps the first call's partials, which
the second must not read)."""
import numpy as np
import pytest

import oracle as O
import weight_only_quantization_pack_amd as awq
from weight_only_quantization_pack_amd import workloads as WL

from gpu_util import TOL, announce, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _layer(M, N, K, bits, seed):
    q, d, z = O.quantize(WL.random_weights(N, K, seed=seed), None, bits)
    qw = O.pack(q, bits)
    x = WL.random_activations(M, K, seed=seed + 1, sigma=1.0)
    return x, qw, d, z


def test_noalloc_matches_workspace_entry_twice(gpu):
    import torch
    cap = awq.gemm_splitk_noalloc_max_bytes()
    assert cap == 32 << 20
    # 64 x 4096 x 14336: 32 tiles of 128 columns, 8 splits (8.4 MB of partials); then
    # 5 x 302 x 2048: 2 splits over a few kB of the same array
    for M, N, K, bits in [(64, 4096, 14336, 4), (5, 302, 2048, 3)]:
        need = awq.gemm_splitk_workspace_bytes(M, N, K)
        assert 0 < need <= cap, need
        announce("gemm_splitk_noalloc", f"M={M} N={N} K={K} bits={bits} partials={need}")
        x, qw, d, z = _layer(M, N, K, bits, seed=M + N)
        args = (dev(x), dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        y_ws = awq.gemm(*args, N=N, bits=bits, split_k=True, workspace=ws)
        y_na = awq.gemm_splitk_noalloc(*args, N=N, bits=bits)
        torch.cuda.synchronize()
        a, b = host(y_ws), host(y_na)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "differs from awq_gemm_splitk"
        err = rel_err(b.astype(np.float64), O.matmul(x, qw, d, z, bits, K))
        assert err <= TOL, f"rel err {err:.3e}"


def test_noalloc_without_split_is_the_plain_gemm(gpu):
    """A shape whose tiles fill the CUs takes no split: the plain awq_gemm."""
    import torch
    M, N, K = 1024, 8192, 1024
    assert awq.gemm_splitk_workspace_bytes(M, N, K) == 0
    x, qw, d, z = _layer(M, N, K, 4, seed=7)
    args = (dev(x), dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z)))
    announce("gemm_splitk_noalloc", f"M={M} N={N} K={K} no split")
    a = host(awq.gemm(*args, N=N, bits=4, split_k=False))
    b = host(awq.gemm_splitk_noalloc(*args, N=N, bits=4))
    torch.cuda.synchronize()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
