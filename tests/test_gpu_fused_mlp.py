"""GPU parity of the folded activation scale (awq_gemv_scaled) and the fused
gate/up projection (awq_gemv_gate_up) against the oracle.

Bars.  awq_gemv_scaled: max|y - y_ref| / max|y_ref| <= 2e-3 with y_ref the
oracle's fp64 product of x' = fp16(fp32(x) * inv_s); where the scaled and the
plain launch take the same kernel, the scaled output also equals, bit for bit,
awq_gemv on the oracle's x' (the staging computes x' exactly).
awq_gemv_gate_up: the same 2e-3 bar on h = SiLU(g) * u relative to max|h_ref|
(the GPU sums g and u in fp32 and rounds h once; the oracle is fp64).
"""
import numpy as np
import pytest

import oracle as O
import weight_only_quantization_pack_amd as awq
from weight_only_quantization_pack_amd import workloads as WL

from gpu_util import TOL, announce, dev, guarded_empty, host, rel_err, sentinel_intact

pytestmark = pytest.mark.gpu


def layer(N, K, bits, seed, group_size=128, s=None):
    q, d, z = O.quantize(WL.random_weights(N, K, seed=seed), s, bits, group_size)
    return O.pack(q, bits), d, z


def on_gpu(lay):
    qw, d, z = lay
    return dev(qw.reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z))


def inv_scale(K, seed):
    rng = np.random.default_rng(seed)
    s = rng.lognormal(0, 1, K).astype(np.float32)
    return (np.float32(1) / s).astype(np.float32)


def gemv_scaled(x, inv_s, lay, N, bits, group_size):
    import torch
    y = awq.gemv(dev(x), *on_gpu(lay), N=N, bits=bits, group_size=group_size, inv_s=dev(inv_s))
    torch.cuda.synchronize()
    return host(y)


def gate_up(x, inv_s, g, u, N, bits, group_size):
    import torch
    h = awq.gemv_gate_up(dev(x), on_gpu(g), on_gpu(u), N=N, bits=bits, group_size=group_size,
                         inv_s=None if inv_s is None else dev(inv_s))
    torch.cuda.synchronize()
    return host(h)


# (M, N, K): x staged once with 1, 2, 4 and 8 loads per lane (8: M = 1 with
# K = 28672, M = 13 with K = 2048, M = 16 with K = 1408; inv_s of chunks past
# the fourth loaded behind the ring), ragged N, one group, and the sliced path
# (x too large for LDS: M = 3 with K = 11008, M = 4 with K = 8192, M = 8 with
# K = 4096; M = 16 with K = 4096 loads the next slice after the sweep)
SHAPES = [(1, 512, 512), (1, 4096, 4096), (2, 37, 384), (4, 1000, 4096), (3, 130, 11008),
          (1, 64, 128), (1, 300, 28672), (4, 200, 8192), (8, 96, 4096), (13, 50, 2048),
          (16, 600, 1408), (16, 200, 4096)]


@pytest.mark.parametrize("group_size", [128, 64])
@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemv_scaled(gpu, M, N, K, bits, group_size):
    announce("gemv_scaled", f"M={M} N={N} K={K} bits={bits} gs={group_size}")
    lay = layer(N, K, bits, seed=M + N + K, group_size=group_size)
    x = WL.random_activations(M, K, seed=M * 7 + K, sigma=1.5)
    inv_s = inv_scale(K, K + 1)
    y = gemv_scaled(x, inv_s, lay, N, bits, group_size).astype(np.float64)
    xs = O.apply_inv_scale(x, inv_s)
    err = rel_err(y, O.matmul(xs, *lay, bits, K))
    assert err <= TOL, f"rel err {err:.3e}"


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (4, 1000, 4096), (1, 64, 128), (4, 200, 8192),
                                   (3, 130, 11008), (1, 300, 28672), (16, 600, 1408), (16, 200, 4096)])
def test_gemv_scaled_stages_x_prime_exactly(gpu, M, N, K):
    """Same kernel as awq_gemv on the oracle's x' (x fits in LDS with <= 8
    loads per lane, or takes the sliced path in both): identical bits."""
    import torch
    announce("gemv_scaled exact", f"M={M} N={N} K={K}")
    lay = layer(N, K, 4, seed=5)
    x = WL.random_activations(M, K, seed=6, sigma=1.5)
    inv_s = inv_scale(K, 7)
    y = gemv_scaled(x, inv_s, lay, N, 4, 128)
    y2 = host(awq.gemv(dev(O.apply_inv_scale(x, inv_s)), *on_gpu(lay), N=N, bits=4))
    torch.cuda.synchronize()
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


@pytest.mark.parametrize("group_size", [128, 64])
@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M,N,K", [(1, 512, 512), (1, 1000, 4096), (2, 37, 384), (4, 700, 4096),
                                   (1, 64, 128), (3, 130, 11008), (1, 300, 28672), (5, 200, 8192),
                                   (8, 96, 4096), (16, 600, 1408), (16, 200, 4096)])
@pytest.mark.parametrize("scaled", [False, True])
def test_gate_up(gpu, M, N, K, bits, group_size, scaled):
    announce("gate_up", f"M={M} N={N} K={K} bits={bits} gs={group_size} scaled={scaled}")
    g = layer(N, K, bits, seed=11 + N, group_size=group_size)
    u = layer(N, K, bits, seed=12 + N, group_size=group_size)
    x = WL.random_activations(M, K, seed=13 + M, sigma=1.0)
    inv_s = inv_scale(K, 14) if scaled else None
    h = gate_up(x, inv_s, g, u, N, bits, group_size).astype(np.float64)
    h_ref = O.gate_up(x, inv_s, g, u, bits, K)
    err = rel_err(h, h_ref)
    assert err <= TOL, f"rel err {err:.3e}"


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gate_up_llama70b_full(gpu, M):
    """Config-3 gate/up shape (K = 8192, N = 28672) at full size with the folded
    scale, whole output tensor (M = 1: x staged once; 4, 16: K sliced, one row
    block of both layers per workgroup)."""
    wl = WL.workload(3)
    K, N = wl.shapes[0]
    announce("gate_up 70b", f"M={M} N={N} K={K}")
    g = layer(N, K, 4, seed=31)
    u = layer(N, K, 4, seed=32)
    x = wl.activations(M, 0)
    inv_s = inv_scale(K, 33)
    h = gate_up(x, inv_s, g, u, N, 4, 128).astype(np.float64)
    h_ref = O.gate_up(x, inv_s, g, u, 4, K)
    err = rel_err(h, h_ref)
    assert err <= TOL, f"rel err {err:.3e}"


# x staged once with 12 x loads per lane (unscaled: the scaled form takes the
# sliced kernel past 8 loads), for the fused pair
@pytest.mark.parametrize("group_size", [128, 64])
@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M,N,K", [(3, 1000, 10368), (5, 300, 6400), (7, 130, 4480), (15, 600, 2176)])
def test_gate_up_x1_twelve_loads(gpu, M, N, K, bits, group_size):
    announce("gate_up xl12", f"M={M} N={N} K={K} bits={bits} gs={group_size}")
    g = layer(N, K, bits, seed=41 + N, group_size=group_size)
    u = layer(N, K, bits, seed=42 + N, group_size=group_size)
    x = WL.random_activations(M, K, seed=43 + M, sigma=1.0)
    h = gate_up(x, None, g, u, N, bits, group_size).astype(np.float64)
    err = rel_err(h, O.gate_up(x, None, g, u, bits, K))
    assert err <= TOL, f"rel err {err:.3e}"


def test_gate_up_one_hot_is_exact(gpu):
    """x = c e_k with grid-valued weights: g and u are exact in fp32, so h is
    the fp16 rounding of SiLU(g) u evaluated in fp32 (at most one fp16 ulp of
    evaluation error from exp and the division)."""
    K, N = 256, 48
    rng = np.random.default_rng(9)
    lays = []
    for _ in range(2):
        q = rng.integers(0, 16, (N, K)).astype(np.uint8)
        d = np.full((N, K // 128), 2.0 ** -3, np.float16)
        z = rng.integers(0, 16, (N, K // 128)).astype(np.float16)
        lays.append((O.pack(q, 4), d, z))
    for k, c in [(0, 1.0), (77, -2.0), (200, 0.5)]:
        x = np.zeros((1, K), np.float16)
        x[0, k] = c
        h = gate_up(x, None, lays[0], lays[1], N, 4, 128).astype(np.float64)[0]
        want = O.gate_up(x, None, lays[0], lays[1], 4, K)[0]
        ulp = np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(h - want) <= 1.01 * ulp), k


def test_gate_up_no_write_past_output_and_repeatable(gpu):
    import torch
    M, N, K = 3, 37, 384
    g, u = layer(N, K, 4, seed=1), layer(N, K, 4, seed=2)
    x = dev(WL.random_activations(M, K, seed=3))
    out, raw, n = guarded_empty((M, N), torch.float16)
    h1 = awq.gemv_gate_up(x, on_gpu(g), on_gpu(u), N=N, out=out).clone()
    h2 = awq.gemv_gate_up(x, on_gpu(g), on_gpu(u), N=N, out=out)
    torch.cuda.synchronize()
    assert sentinel_intact(raw, n)
    assert torch.equal(h1, h2)


def test_fused_empty_calls(gpu):
    import torch
    K = 256
    g = on_gpu(layer(16, K, 4, seed=1))
    x = torch.empty((0, K), dtype=torch.float16, device="cuda:0")
    assert awq.gemv_gate_up(x, g, g, N=16).shape == (0, 16)
    assert awq.gemv(x, *g, N=16, inv_s=torch.ones(K, dtype=torch.float32, device="cuda:0")).shape == (0, 16)
