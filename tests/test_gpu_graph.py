"""HIP-graph capture of the hot-path entry points (the bench replays the
decode step from a graph).  One graph holds the x1 and sliced GEMVs (plain,
scaled, int3), the fused gate/up GEMV, a split-K GEMM (with its reduction) and
a plain pipelined GEMM.  It is replayed several times; before each replay the
inputs are rewritten eagerly, and after it the eager calls on the same inputs
must give the same bits (every kernel sums in a fixed order).  The library
records no memset, so nothing in the graph is a memset node.
"""
import numpy as np
import pytest

import oracle as O
import weight_only_quantization_pack_amd as awq
from weight_only_quantization_pack_amd import workloads as WL

from gpu_util import announce, dev

pytestmark = pytest.mark.gpu


def _layer(N, K, bits, seed, group_size=128):
    q, d, z = O.quantize(WL.random_weights(N, K, seed=seed), None, bits, group_size)
    return dev(O.pack(q, bits).reshape(-1)), dev(O.tile_params(d)), dev(O.tile_params(z))


def test_graph_replays_match_eager(gpu):
    import torch
    announce("graph replay: gemv, gemv scaled, gemv int3 M=16, gate_up, gemm split-K, gemm")
    d = torch.device("cuda:0")
    A = _layer(1000, 4096, 4, 1)                 # K = 4096
    B3 = _layer(300, 2048, 3, 2)                 # int3, K = 2048
    Gl, Ul = _layer(512, 4096, 4, 3), _layer(512, 4096, 4, 4)
    L = _layer(4096, 512, 4, 5)                  # M = 2048: 256 tiles, no split
    x1 = torch.empty((1, 4096), dtype=torch.float16, device=d)
    x16 = torch.empty((16, 2048), dtype=torch.float16, device=d)
    x64 = torch.empty((64, 4096), dtype=torch.float16, device=d)
    xb = torch.empty((2048, 512), dtype=torch.float16, device=d)
    inv_s = torch.empty(4096, dtype=torch.float32, device=d)
    ws = torch.empty(max(1, awq.gemm_splitk_workspace_bytes(64, 1000, 4096)), dtype=torch.uint8, device=d)
    assert awq.gemm_splitk_workspace_bytes(64, 1000, 4096) > 0      # the split-K path is taken
    outs = {k: torch.empty(s, dtype=torch.float16, device=d) for k, s in
            [("y1", (1, 1000)), ("ys", (1, 1000)), ("y16", (16, 300)), ("ygu", (1, 512)),
             ("y64", (64, 1000)), ("yb", (2048, 4096))]}

    def run(o):
        awq.gemv(x1, *A, N=1000, out=o["y1"])
        awq.gemv(x1, *A, N=1000, out=o["ys"], inv_s=inv_s)
        awq.gemv(x16, *B3, N=300, bits=3, out=o["y16"])
        awq.gemv_gate_up(x1, Gl, Ul, N=512, inv_s=inv_s, out=o["ygu"])
        awq.gemm(x64, *A, N=1000, out=o["y64"], workspace=ws)
        awq.gemm(xb, *L, N=4096, out=o["yb"])

    def fill(seed):
        g = torch.Generator(device=d).manual_seed(seed)
        for t in (x1, x16, x64, xb):
            t.copy_(torch.randn(t.shape, generator=g, device=d).half())
        inv_s.copy_(torch.rand(4096, generator=g, device=d) + 0.5)

    stream = torch.cuda.Stream()
    fill(0)
    with torch.cuda.stream(stream):
        run(outs)                                # warm-up (code objects, attributes)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run(outs)
    torch.cuda.synchronize()
    eager = {k: torch.empty_like(v) for k, v in outs.items()}
    for rep in range(3):
        fill(100 + rep)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in outs.items()}
        with torch.cuda.stream(stream):
            run(eager)
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(got[k], eager[k]), (rep, k)
            assert torch.isfinite(got[k].float()).all(), (rep, k)
