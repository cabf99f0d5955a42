#!/usr/bin/env python3
"""Benchmark of the AWQ W4A16 g128 hot path on one MI355X.

Headline (value): decode GEMV throughput at M = 1 on the Llama-7B layer
shapes, in algorithmic GB/s.  One step = the seven linears of one Llama-7B
decoder layer at decode (q, k, v, o: 4096x4096; gate, up: 4096->11008;
down: 11008->4096), each one awq_gemv launch on packed int4 g128 weights.
Weights rotate over enough replicas (>= 768 MB, three times the 256 MB
Infinity Cache) that every step reads them from HBM (step i reads replica
i % R).  Exactly --warmup untimed steps, then exactly --steps timed steps,
each run as one captured HIP graph of that many steps (one eager step before
the captures loads the code objects), so host launch overhead is not timed.
Timing: HIP events on the launch stream around the timed graph.  Beside it,
the achievable read rate at each launch's byte count: a plain streaming-read
kernel (libawq_probe, best of a sweep of launch shapes), timed the same way.

Second half of the metric (gemm): prefill GEMM TFLOP/s at M = 2048 on the
Mistral-7B shapes (4096x14336, 14336x4096, 4096x6144), and the same shapes
at M = 512.  Also reported: the offline path (alpha search on the 4096x4096
layer with 512 calibration tokens and 20 grid points; quantize+pack) and the
CPU oracle on the host cores: the decode step (the headline leg), the M =
2048 products, quantize+pack and the 20-alpha search.

Algorithmic bytes per GEMV launch: N*K/2 (int4 codes) + 4*N*K/128 (fp16
scale and zero per group) + 2*M*K (x) + 2*M*N (y).  Flops per GEMM launch:
2*M*N*K.  Peaks: HBM 8 TB/s; dense fp16 MFMA 2.5 PFLOP/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
COLD_BYTES = 768 * 2 ** 20
GEMM_REPS = 5                  # timed loops per prefill shape (median reported)
METRIC = "W4A16 g128 GEMV GB/s (% HBM peak) at M=1 + GEMM TFLOP/s at M=2048"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gemv_bytes(M, N, K, bits=4, group_size=128):
    return N * K * bits // 8 + 4 * N * (K // group_size) + 2 * M * K + 2 * M * N


def gemm_traffic():
    """HBM bytes of the three M = 2048 prefill launches (one per shape, summed)
    from the committed rocprofv3 PMC runs, and their algorithmic bytes.

    profiles/gemm_mistral7b_m2048_traffic.json holds FETCH_SIZE + WRITE_SIZE
    of `bench.py --pmc-gemm-probe`, scaled by a copy of known size; it is used
    only while its recorded hash matches the current GEMM source, else None.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_mistral7b_m2048_traffic.json")
    csrc = os.path.join(ROOT, "weight_only_quantization_pack_amd", "csrc")
    try:
        rec = json.load(open(path))
        src = open(os.path.join(csrc, "gemm.hip"), "rb").read() + \
            open(os.path.join(csrc, "awq_internal.h"), "rb").read()
    except (OSError, ValueError):
        return None, None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None, None
    return int(rec["traffic_bytes_three_launches"]), int(rec["algorithmic_bytes_three_launches"])


def gemv_traffic_per_launch():
    """HBM bytes per decode GEMV launch from the committed rocprofv3 PMC runs.

    profiles/gemv_llama7b_decode_traffic.json holds FETCH_SIZE + WRITE_SIZE,
    scaled by a copy of known size, per launch of the decode step.  It is used
    only while its recorded hash matches the current GEMV source; after any
    change to the kernel the counters are stale and the traffic is null.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_llama7b_decode_traffic.json")
    csrc = os.path.join(ROOT, "weight_only_quantization_pack_amd", "csrc")
    try:
        rec = json.load(open(path))
        src = open(os.path.join(csrc, "gemv.hip"), "rb").read() + \
            open(os.path.join(csrc, "awq_internal.h"), "rb").read()
    except (OSError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return int(rec["traffic_bytes_per_launch"])


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--gemm-iters", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-offline", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="short run for rocprofv3 --pmc: a 256 MiB device copy (known size, "
                         "calibrates FETCH_SIZE/WRITE_SIZE) then one cold pass of the decode step")
    ap.add_argument("--pmc-gemm-probe", action="store_true",
                    help="short run for rocprofv3 --pmc: a 256 MiB device copy (known size, "
                         "calibrates FETCH_SIZE/WRITE_SIZE), then the three M=2048 prefill GEMMs, "
                         "three launches each after one warm-up launch")
    ap.add_argument("--pmc-batched-probe", action="store_true",
                    help="short run for rocprofv3 --pmc: a 256 MiB device copy, then the Llama-70B MLP "
                         "shapes at M = 64 (awq_gemm) and M = 16 (awq_gemm, then awq_gemv), three launches each")
    ap.add_argument("--pmc-search-probe", action="store_true",
                    help="only run the 20-alpha search of the 4096x4096 layer on 512 calibration "
                         "tokens three times on each path (buffered, then fused; for rocprofv3 "
                         "--pmc counter runs)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path in this "
              "build (a layer would be split by output rows, one shard per GPU, with no "
              "exchange for the matmul itself). Use --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import weight_only_quantization_pack_amd as awq
    from weight_only_quantization_pack_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    awq.load_library()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    stream = torch.cuda.Stream()          # default priority

    if args.pmc_gemm_probe:
        # calibration copy of known size, then the three shapes
        src = torch.empty(256 * 2**20, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        wl4 = WL.workload(4)
        res = {}
        with torch.cuda.stream(stream):
            for i, (K, N) in enumerate(wl4.shapes):
                W = torch.from_numpy(wl4.weights(i)).to(dev)
                qw, sc, ze = awq.quantize_pack(W, None, bits=4)
                x = torch.from_numpy(wl4.activations(2048, i)).to(dev)
                y = torch.empty((2048, N), dtype=torch.float16, device=dev)
                for _ in range(4):
                    awq.gemm(x, qw, sc, ze, N=N, bits=4, out=y)
                res[f"{K}x{N}"] = 2.0 * 2048 * N * K
                del W, qw, sc, ze, x, y
        torch.cuda.synchronize()
        # algorithmic bytes per launch: packed weights, scales and zeros, x, y
        alg = {f"{K}x{N}": N * K // 2 + 4 * N * (K // 128) + 2 * 2048 * K + 2 * 2048 * N
               for K, N in wl4.shapes}
        print(json.dumps({"pmc_gemm_probe": True, "M": 2048, "copy_bytes": 256 * 2**20,
                          "flops_per_launch": res, "algorithmic_bytes_per_launch": alg}))
        return 0

    if args.pmc_batched_probe:
        src = torch.empty(256 * 2**20, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        wl3 = WL.workload(3)
        order = []
        with torch.cuda.stream(stream):
            for i, (K, N) in enumerate(wl3.shapes):
                W = torch.from_numpy(wl3.weights(i)).to(dev)
                qw, sc, ze = awq.quantize_pack(W, None, bits=4)
                del W
                for M, fn in ((64, awq.gemm), (16, awq.gemm), (16, awq.gemv)):
                    x = torch.from_numpy(wl3.activations(M, i)).to(dev)
                    y = torch.empty((M, N), dtype=torch.float16, device=dev)
                    for _ in range(3):
                        fn(x, qw, sc, ze, N=N, bits=4, out=y)
                        order.append(f"{K}x{N} M={M} {fn.__name__}")
                del qw, sc, ze
        torch.cuda.synchronize()
        print(json.dumps({"pmc_batched_probe": True, "copy_bytes": 256 * 2**20, "launches": order}))
        return 0

    if args.pmc_search_probe:
        # calibration copy of known size, then the search three times
        src = torch.empty(256 * 2**20, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        wl5 = WL.workload(5)
        with torch.cuda.stream(stream):
            W = torch.from_numpy(wl5.weights()).to(dev)
            X = torch.from_numpy(wl5.calibration()).to(dev)
            T, (N, K), A = X.shape[0], W.shape, len(wl5.alphas)
            for fused in (False, True):
                ws = torch.empty(awq.search_workspace_bytes(T, N, K, A, fused=fused), dtype=torch.uint8,
                                 device=dev)
                for _ in range(3):
                    awq.search_scale(W, X, wl5.alphas, bits=4, workspace=ws)
                del ws
        torch.cuda.synchronize()
        # loss GEMM: 2 T N K flops per alpha; error kernel: W read once, D written
        # once per alpha (N rounded up to 16 rows)
        print(json.dumps({"pmc_search_probe": True, "copy_bytes": 256 * 2**20, "T": T, "N": N,
                          "K": K, "n_alpha": A,
                          "loss_gemm_flops": 2.0 * T * N * K * A,
                          "quant_err_bytes": 2 * N * K + A * 2 * ((N + 15) // 16 * 16) * K,
                          "loss_gemm_d_bytes": A * 2 * ((N + 15) // 16 * 16) * K,
                          "fused_loss_bytes": A * (2 * N * K + 2 * T * K)}))
        return 0

    # ------------------------------------------------------------------ decode GEMV
    wl2 = WL.workload(2)
    shape_index = {s: i for i, s in enumerate(wl2.shapes)}
    layer = WL.LLAMA7B_LAYER
    packed = {}
    xs = {}
    with torch.cuda.stream(stream):
        for (K, N), i in shape_index.items():
            W = torch.from_numpy(wl2.weights(i)).to(dev)
            packed[(K, N)] = awq.quantize_pack(W, None, bits=4)
            xs[K] = torch.from_numpy(wl2.activations(1, i)).to(dev)
            del W
    step_bytes = sum(gemv_bytes(1, N, K) for K, N in layer)
    weight_bytes = sum(N * K // 2 + 4 * N * (K // 128) for K, N in layer)
    R = max(2, math.ceil(COLD_BYTES / weight_bytes))
    reps = [[tuple(t.clone() for t in packed[s]) for s in layer] for _ in range(R)]
    ys = [torch.empty((1, N), dtype=torch.float16, device=dev) for _, N in layer]
    torch.cuda.synchronize()
    log(f"decode step: {len(layer)} GEMVs, {step_bytes / 1e6:.2f} MB algorithmic, "
        f"{R} weight replicas ({R * weight_bytes / 2**20:.0f} MiB)")

    def step(r):
        for j, (K, N) in enumerate(layer):
            qw, sc, ze = reps[r][j]
            awq.gemv(xs[K], qw, sc, ze, N=N, bits=4, out=ys[j])

    if args.pmc_probe:
        # calibration copy of known size, then each replica's decode step once
        src = torch.empty(256 * 2**20, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for r in range(R):
                step(r)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_probe": True, "copy_bytes": src.numel(), "step_bytes": step_bytes,
                          "gemv_launch_bytes": {f"{K}x{N}": gemv_bytes(1, N, K) for K, N in layer}}))
        return 0

    # Exactly --warmup untimed and --steps timed steps: each is one graph of that
    # many consecutive steps, step i reading replica i % R.  One eager step
    # before the captures loads the code objects.
    with torch.cuda.stream(stream):
        step(0)
    torch.cuda.synchronize()

    def capture(n_steps, first):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n_steps):
                step((first + i) % R)
        return g

    warm = max(0, args.warmup)
    steps = max(1, args.steps)
    warm_graph = capture(warm, 0) if warm > 0 else None
    timed_graph = capture(steps, warm)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        if warm_graph is not None:
            warm_graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        e0.record(stream)
        timed_graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / steps
    gemv_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    avg_launch_us = ms_per_step * 1e3 / len(layer)
    log(f"decode step {ms_per_step * 1e3:.2f} us  ->  {gemv_gbs:.1f} GB/s "
        f"({100 * gemv_gbs / HBM_PEAK_GBS:.1f}% of HBM peak); avg launch {avg_launch_us:.2f} us "
        f"({steps} timed steps after {warm} warm-up steps)")
    del warm_graph, timed_graph

    # the plain-read ceiling at each launch's byte count (cold, graph replay)
    ceiling = read_ceiling(torch, dev, stream, props.multi_processor_count,
                           sorted({gemv_bytes(1, N, K) for K, N in layer}
                                  | {gemv_bytes(1, N, K) for K, N in WL.workload(3).shapes}))
    step_ceiling_us = sum(ceiling[gemv_bytes(1, N, K)]["us"] for K, N in layer)
    ceiling_gbs = step_bytes / (step_ceiling_us * 1e-6) / 1e9

    # per-shape GEMV times (same graph technique, one shape per graph, its own
    # >= 768 MB of replicas so that the shape is as cold as in the step)
    del reps
    per_shape = {}
    for (K, N) in wl2.shapes:
        j = layer.index((K, N))
        Rs = max(2, math.ceil(COLD_BYTES / (N * K // 2 + 4 * N * (K // 128))))
        sreps = [tuple(t.clone() for t in packed[(K, N)]) for _ in range(Rs)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(Rs):
                qw, sc, ze = sreps[r]
                awq.gemv(xs[K], qw, sc, ze, N=N, bits=4, out=ys[j])
        with torch.cuda.stream(stream):
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n_rep = max(2, 400 // Rs)
            a.record(stream)
            for _ in range(n_rep):
                g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (n_rep * Rs)
        gbs = gemv_bytes(1, N, K) / (us * 1e-6) / 1e9
        cl = ceiling[gemv_bytes(1, N, K)]
        per_shape[f"{K}x{N}"] = {"us": round(us, 3), "GBps": round(gbs, 1),
                                 "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "cold_replicas": Rs,
                                 "read_ceiling_us": cl["us"],
                                 "frac_of_read_ceiling": round(cl["us"] / us, 4)}
        log(f"  gemv K={K} N={N}: {us:.2f} us, {gbs:.1f} GB/s")
        del g, sreps
        torch.cuda.empty_cache()

    del packed
    torch.cuda.empty_cache()

    # --------------------------------------------- batched decode (context, not the metric)
    # Llama-70B MLP shapes at M = 1, 4, 16 (awq_gemv) and 64 (awq_gemm): the
    # bandwidth -> compute crossover, cold weights as above
    wl3 = WL.workload(3)
    batched = {}
    for i, (K, N) in enumerate(wl3.shapes):
        with torch.cuda.stream(stream):
            W = torch.from_numpy(wl3.weights(i)).to(dev)
            base = awq.quantize_pack(W, None, bits=4)
            del W
        wb = N * K // 2 + 4 * N * (K // 128)
        R3 = max(2, math.ceil(COLD_BYTES / wb))
        reps3 = [tuple(t.clone() for t in base) for _ in range(R3)]
        del base
        res = {}
        for M, fn in ((1, awq.gemv), (4, awq.gemv), (16, awq.gemv), (16, awq.gemm), (64, awq.gemm)):
            key = f"M{M}" if (M <= 16) == (fn is awq.gemv) else f"M{M}_gemm"
            x = torch.from_numpy(wl3.activations(M, i)).to(dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            with torch.cuda.stream(stream):
                for r in range(R3):
                    fn(x, *reps3[r], N=N, bits=4, out=y)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(R3):
                    fn(x, *reps3[r], N=N, bits=4, out=y)
            # warm-up as long as eight timed loops (20-50 ms: the first shape
            # read slow after a shorter one), then the median of three loops
            n_rep = max(2, 100 // R3)
            loops = []
            with torch.cuda.stream(stream):
                for _ in range(8 * n_rep):
                    g.replay()
                torch.cuda.synchronize()
                for _ in range(3):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(n_rep):
                        g.replay()
                    b.record(stream)
                    torch.cuda.synchronize()
                    loops.append(a.elapsed_time(b) * 1e3 / (n_rep * R3))
            us = sorted(loops)[1]
            gbs = gemv_bytes(M, N, K) / (us * 1e-6) / 1e9
            res[key] = {"us": round(us, 2), "GBps": round(gbs, 1),
                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            "frac_of_read_ceiling_M1": round(ceiling[gemv_bytes(1, N, K)]["us"] / us, 4),
                            "TFLOPs": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 1),
                            "entry": "awq_gemv" if fn is awq.gemv else "awq_gemm"}
            log(f"  batched decode K={K} N={N} M={M} ({res[key]['entry']}): {us:.2f} us, {gbs:.1f} GB/s")
            del g, x, y
        batched[f"{K}x{N}"] = res
        del reps3
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ prefill GEMM
    wl4 = WL.workload(4)
    M = 2048
    gemm_res, gemm_m512 = {}, {}
    tot_flops, tot_ms = 0.0, 0.0
    tot512_flops, tot512_ms = 0.0, 0.0
    for i, (K, N) in enumerate(wl4.shapes):
        with torch.cuda.stream(stream):
            W = torch.from_numpy(wl4.weights(i)).to(dev)
            qw, sc, ze = awq.quantize_pack(W, None, bits=4)
            Wt = W.t().contiguous()                    # [K][N]: dense fp16 reference operand
            del W
        for Mi in (2048, 512):
            # warm-up launches, then GEMM_REPS timed loops of --gemm-iters
            # launches each; the median loop is reported (single loops vary by
            # up to ~15 % with the clock the GPU runs at)
            with torch.cuda.stream(stream):
                x = torch.from_numpy(wl4.activations(Mi, i)).to(dev)
                y = torch.empty((Mi, N), dtype=torch.float16, device=dev)
                for _ in range(max(3, args.gemm_iters)):
                    awq.gemm(x, qw, sc, ze, N=N, bits=4, out=y)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                loops = []
                for _ in range(GEMM_REPS):
                    a.record(stream)
                    for _ in range(args.gemm_iters):
                        awq.gemm(x, qw, sc, ze, N=N, bits=4, out=y)
                    b.record(stream)
                    b.synchronize()
                    loops.append(a.elapsed_time(b) / args.gemm_iters)
            torch.cuda.synchronize()
            ms = sorted(loops)[len(loops) // 2]
            flops = 2.0 * Mi * N * K
            tf = flops / (ms * 1e-3) / 1e12
            # context, not the metric: the same product with dense fp16 weights
            # through torch.matmul (hipBLASLt), i.e. what the vendor library reaches
            # on this GPU for this shape without any dequantization
            with torch.cuda.stream(stream):
                for _ in range(3):
                    ref = torch.matmul(x, Wt)
                a.record(stream)
                for _ in range(args.gemm_iters):
                    ref = torch.matmul(x, Wt)
                b.record(stream)
            torch.cuda.synchronize()
            ref_tf = flops / (a.elapsed_time(b) / args.gemm_iters * 1e-3) / 1e12
            rec = {"us": round(ms * 1e3, 2), "TFLOPs": round(tf, 1),
                   "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                   "dense_fp16_hipblaslt_TFLOPs": round(ref_tf, 1)}
            # the activation scale folded into the product (awq_gemm_scaled),
            # and the same product as two launches (awq_scale_activations into
            # a buffer, then awq_gemm), on the same inputs
            inv = torch.from_numpy((1.0 / np.random.default_rng(K).lognormal(0, 0.5, K)).astype(np.float32)).to(dev)
            svec = (1.0 / inv).contiguous()
            xs_buf = torch.empty_like(x)
            with torch.cuda.stream(stream):
                for mode in ("folded", "two_pass"):
                    for it in range(3 + args.gemm_iters):
                        if it == 3:
                            a.record(stream)
                        if mode == "folded":
                            awq.gemm(x, qw, sc, ze, N=N, bits=4, out=y, inv_s=inv)
                        else:
                            awq.scale_activations(x, svec, out=xs_buf)
                            awq.gemm(xs_buf, qw, sc, ze, N=N, bits=4, out=y)
                    b.record(stream)
                    torch.cuda.synchronize()
                    rec[f"scaled_{mode}_us"] = round(a.elapsed_time(b) / args.gemm_iters * 1e3, 2)
            del xs_buf
            if Mi == 2048:
                gemm_res[f"{K}x{N}"] = rec
                tot_flops += flops
                tot_ms += ms
            else:
                rec["split_k_workspace_bytes"] = awq.gemm_splitk_workspace_bytes(Mi, N, K)
                gemm_m512[f"{K}x{N}"] = rec
                tot512_flops += flops
                tot512_ms += ms
            log(f"  gemm M={Mi} K={K} N={N}: {ms * 1e3:.1f} us, {tf:.1f} TFLOP/s "
                f"(dense fp16 torch.matmul {ref_tf:.1f})")
            del x, y, ref
        del qw, sc, ze, Wt
    gemm_tflops = tot_flops / (tot_ms * 1e-3) / 1e12
    gemm512_tflops = tot512_flops / (tot512_ms * 1e-3) / 1e12

    # ------------------------------------------------------------------ offline path
    # ---------------------------------------- variants of the pages (context, not the metric)
    # the Llama-7B decode step with int3 codes and with 64-wide groups (own
    # algorithmic bytes), and the int3 prefill GEMM at M = 2048
    variants = {}
    for bits, gs in ((3, 128), (4, 64)):
        vb = sum(N * K * bits // 8 + 4 * N * (K // gs) for K, N in layer)
        Rv = max(2, math.ceil(COLD_BYTES / vb))
        vpacked = {}
        with torch.cuda.stream(stream):
            for (K, N), i in shape_index.items():
                W = torch.from_numpy(wl2.weights(i)).to(dev)
                vpacked[(K, N)] = awq.quantize_pack(W, None, bits=bits, group_size=gs)
                del W
        vreps = [[tuple(t.clone() for t in vpacked[sh]) for sh in layer] for _ in range(Rv)]
        del vpacked
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for r in range(Rv):
                for j, (K, N) in enumerate(layer):
                    awq.gemv(xs[K], *vreps[r][j], N=N, bits=bits, group_size=gs, out=ys[j])
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for r in range(Rv):
                for j, (K, N) in enumerate(layer):
                    awq.gemv(xs[K], *vreps[r][j], N=N, bits=bits, group_size=gs, out=ys[j])
        with torch.cuda.stream(stream):
            for _ in range(2):
                g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n_rep = max(2, 200 // Rv)
            a.record(stream)
            for _ in range(n_rep):
                g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (n_rep * Rv)
        sb = sum(gemv_bytes(1, N, K, bits, gs) for K, N in layer)
        variants[f"decode_step_int{bits}_g{gs}"] = {
            "us": round(us, 2), "GBps": round(sb / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(sb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "step_bytes": sb}
        log(f"  variant decode step int{bits} g{gs}: {us:.2f} us, {sb / (us * 1e-6) / 1e9:.1f} GB/s")
        del vreps, g
        torch.cuda.empty_cache()
    # the same layer with the fused modules of "transformers - AWQ": q/k/v as
    # one product over their concatenated rows (N = 3 x 4096), o, the gate/up
    # pair in one launch with SiLU(g) * u (awq_gemv_gate_up), down on h --
    # 4 launches instead of 7, the same weight bytes
    with torch.cuda.stream(stream):
        base = {}
        for (K, N), i in shape_index.items():
            W = torch.from_numpy(wl2.weights(i)).to(dev)
            base[(K, N)] = awq.quantize_pack(W, None, bits=4)
            del W
        q4 = base[(4096, 4096)]
        qkv = tuple(torch.cat([t, t, t]) for t in q4)      # 16-row blocks: rows concatenate
    fused_bytes = (gemv_bytes(1, 3 * 4096, 4096) + gemv_bytes(1, 4096, 4096)
                   + 2 * (11008 * 4096 // 2 + 4 * 11008 * 32) + 2 * 4096 + 2 * 11008
                   + gemv_bytes(1, 4096, 11008))
    Rf = max(2, math.ceil(COLD_BYTES / weight_bytes))
    freps = [(tuple(t.clone() for t in qkv), tuple(t.clone() for t in q4),
              tuple(t.clone() for t in base[(4096, 11008)]), tuple(t.clone() for t in base[(4096, 11008)]),
              tuple(t.clone() for t in base[(11008, 4096)])) for _ in range(Rf)]
    del base, qkv, q4
    y_qkv = torch.empty((1, 3 * 4096), dtype=torch.float16, device=dev)
    y_o = torch.empty((1, 4096), dtype=torch.float16, device=dev)
    h = torch.empty((1, 11008), dtype=torch.float16, device=dev)
    y_d = torch.empty((1, 4096), dtype=torch.float16, device=dev)

    def fused_step(r):
        qkv_w, o_w, g_w, u_w, d_w = freps[r]
        awq.gemv(xs[4096], *qkv_w, N=3 * 4096, out=y_qkv)
        awq.gemv(xs[4096], *o_w, N=4096, out=y_o)
        awq.gemv_gate_up(xs[4096], g_w, u_w, N=11008, out=h)
        awq.gemv(xs[11008], *d_w, N=4096, out=y_d)

    with torch.cuda.stream(stream):
        for r in range(Rf):
            fused_step(r)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for r in range(Rf):
            fused_step(r)
    with torch.cuda.stream(stream):
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_rep = max(2, 200 // Rf)
        a.record(stream)
        for _ in range(n_rep):
            g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (n_rep * Rf)
    variants["decode_step_fused_modules"] = {
        "us": round(us, 2), "GBps": round(fused_bytes / (us * 1e-6) / 1e9, 1),
        "frac_hbm": round(fused_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "step_bytes": fused_bytes,
        "launches": ["gemv qkv 4096x12288", "gemv o 4096x4096", "gemv_gate_up 4096x11008",
                     "gemv down 11008x4096"]}
    log(f"  variant decode step fused modules: {us:.2f} us, {fused_bytes / (us * 1e-6) / 1e9:.1f} GB/s")
    del freps, g
    torch.cuda.empty_cache()

    tot3_flops, tot3_ms = 0.0, 0.0
    for i, (K, N) in enumerate(wl4.shapes):
        with torch.cuda.stream(stream):
            W = torch.from_numpy(wl4.weights(i)).to(dev)
            qw, sc, ze = awq.quantize_pack(W, None, bits=3)
            del W
            x = torch.from_numpy(wl4.activations(M, i)).to(dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            for _ in range(2):
                awq.gemm(x, qw, sc, ze, N=N, bits=3, out=y)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(max(2, args.gemm_iters // 2)):
                awq.gemm(x, qw, sc, ze, N=N, bits=3, out=y)
            b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / max(2, args.gemm_iters // 2)
        tot3_flops += 2.0 * M * N * K
        tot3_ms += ms
        del qw, sc, ze, x, y
    variants["gemm_int3_M2048_TFLOPs"] = round(tot3_flops / (tot3_ms * 1e-3) / 1e12, 1)
    log(f"  variant int3 GEMM M={M}: {variants['gemm_int3_M2048_TFLOPs']} TFLOP/s")

    offline = None
    if not args.no_offline:
        wl5 = WL.workload(5)
        with torch.cuda.stream(stream):
            W = torch.from_numpy(wl5.weights()).to(dev)
            X = torch.from_numpy(wl5.calibration()).to(dev)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

            def time_search(Wt, Xt, fused, reps):
                """Mean ms of awq_search_scale on the path a workspace of each size selects."""
                wst = torch.empty(awq.search_workspace_bytes(Xt.shape[0], Wt.shape[0], Wt.shape[1],
                                                             len(wl5.alphas), fused=fused),
                                  dtype=torch.uint8, device=dev)
                for _ in range(2):
                    res = awq.search_scale(Wt, Xt, wl5.alphas, bits=4, workspace=wst)
                torch.cuda.synchronize()
                a.record(stream)
                for _ in range(reps):
                    res = awq.search_scale(Wt, Xt, wl5.alphas, bits=4, workspace=wst)
                b.record(stream)
                torch.cuda.synchronize()
                return a.elapsed_time(b) / reps, wst.numel(), res

            # the default path (the fused loss kernel forms W - w_hat / s in
            # registers) and the buffered one (D written per chunk of alphas,
            # then the loss GEMM), each selected by its workspace size
            search_ms, ws_fused, (s, loss, best) = time_search(W, X, True, 5)
            search_buf_ms, ws_buf, _ = time_search(W, X, False, 5)
            search_ws = (ws_fused, ws_buf)
            # both paths on the Llama-70B MLP shapes (same tokens and grid)
            search_70b = {}
            for (N70, K70) in ((28672, 8192), (8192, 28672)):
                W70 = torch.from_numpy(WL.random_weights(N70, K70, seed=3)).to(dev)
                X70 = torch.from_numpy(WL.random_activations(X.shape[0], K70, seed=4)).to(dev)
                f_ms, f_ws, _ = time_search(W70, X70, True, 3)
                b_ms, b_ws, _ = time_search(W70, X70, False, 3)
                search_70b[f"{K70}x{N70}"] = {"fused_ms": round(f_ms, 3), "buffered_ms": round(b_ms, 3),
                                              "fused_workspace_bytes": f_ws, "buffered_workspace_bytes": b_ws}
                del W70, X70
            # the gate/up pair of the Llama-7B MLP (4096 -> 11008 -> 4096) searched
            # on the block's output (awq_search_scale_mlp), same tokens and grid
            Wg = torch.from_numpy(wl2.weights(1)).to(dev)          # 4096 x 11008 layer: [11008][4096]
            Wu = torch.from_numpy(WL.random_weights(11008, 4096, seed=7)).to(dev)
            Wd = torch.from_numpy(wl2.weights(2)).to(dev)          # 11008 x 4096 layer: [4096][11008]
            wsm = torch.empty(awq.search_mlp_workspace_bytes(X.shape[0], 4096, 11008, 4096, len(wl5.alphas)),
                              dtype=torch.uint8, device=dev)
            for _ in range(2):
                awq.search_scale_mlp(Wg, Wu, Wd, X, wl5.alphas, workspace=wsm)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(3):
                awq.search_scale_mlp(Wg, Wu, Wd, X, wl5.alphas, workspace=wsm)
            b.record(stream)
            torch.cuda.synchronize()
            search_mlp_ms = a.elapsed_time(b) / 3
            search_mlp_ws = wsm.numel()
            del Wg, Wu, Wd, wsm
            a.record(stream)
            for _ in range(20):
                qp = awq.quantize_pack(W, s, bits=4)
            b.record(stream)
            torch.cuda.synchronize()
            qp_us = a.elapsed_time(b) * 1e3 / 20
        qp_bytes = W.numel() * 2 + W.shape[1] * 4 + W.numel() // 2 + 4 * W.numel() // 128
        offline = {"search_4096x4096_T512_20alpha_ms": round(search_ms, 3),
                   "search_path": "fused loss kernel (the default: a workspace of awq_search_workspace_bytes_fused)",
                   "search_buffered_path_ms": round(search_buf_ms, 3),
                   "search_workspace_bytes": {"fused": search_ws[0], "buffered": search_ws[1]},
                   "search_llama70b_mlp_T512_20alpha": search_70b,
                   "search_mlp_block_llama7b_T512_20alpha_ms": round(search_mlp_ms, 3),
                   "search_mlp_block_workspace_bytes": search_mlp_ws,
                   "search_loss_gemm_TFLOPs_incl_quant": round(
                       20 * 2.0 * 512 * 4096 * 4096 / (search_ms * 1e-3) / 1e12, 1),
                   "quantize_pack_4096x4096_us": round(qp_us, 2),
                   "quantize_pack_GBps": round(qp_bytes / (qp_us * 1e-6) / 1e9, 1),
                   "best_alpha": float(wl5.alphas[int(best.item())])}
        log(f"offline: search {search_ms:.3f} ms, quantize_pack {qp_us:.1f} us")
        del W, X

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layer, wl2, shape_index, step_bytes, wl4, WL.workload(5))

    out = {
        "metric": METRIC,
        "value": round(gemv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x fp16 activations, fp32 accumulate",
        "data": "synthetic (seeded: W ~ N(0,0.02), x = lognormal(0,1.5) channel scale x N(0,1))",
        "config": {"workload": "Llama-7B decoder-layer decode GEMV, M=1, int4 g128 asym",
                   "shapes_KxN": [f"{K}x{N}" for K, N in layer], "M": 1, "bits": 4,
                   "group_size": 128, "step_bytes": step_bytes, "cold_weight_replicas": R,
                   "launch": "HIP graph replay"},
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": gemv_traffic_per_launch(), "traffic_unit": "HBM bytes per launch",
                     "algorithmic_bytes_per_launch": round(step_bytes / len(layer)),
                     "kernel": "k_gemv_x1<4,128,8,U,XL,false,false> (ring U=2, XL=1 for K=4096; U=4, XL=4 for K=11008)", "avg_launch_us": round(avg_launch_us, 3),
                     "read_ceiling": {"GBps": round(ceiling_gbs, 1), "step_us": round(step_ceiling_us, 3),
                                      "frac": round(gemv_gbs / ceiling_gbs, 4),
                                      "what": "a plain streaming-read kernel (libawq_probe) reading each "
                                              "launch's byte count once, cold, in graph replay; best of a "
                                              "sweep of launch shapes",
                                      "per_launch_bytes": {str(k): v for k, v in ceiling.items()}}},
        "gemv_per_shape": per_shape,
        "batched_decode_llama70b_mlp": batched,
        "variants": variants,
        "gemm": {"M": M, "TFLOPs": round(gemm_tflops, 1), "per_shape": gemm_res,
                 "M512": {"TFLOPs": round(gemm512_tflops, 1), "per_shape": gemm_m512},
                 "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1),
                              "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(gemm_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                              "traffic": gemm_traffic()[0],
                              "traffic_unit": "HBM bytes of one launch of each of the three shapes (sum)",
                              "algorithmic_bytes": gemm_traffic()[1],
                              "kernel": "k_gemm_w4p: 128 x 448 tiles (4 waves x 7 column blocks) for 4096x14336 (512 tiles), 128 x 256 (8 waves x 2) for 14336x4096 (256), 128 x 384 (8 waves x 3) for 4096x6144 (256)"}},
        "offline": offline,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
    }
    print(json.dumps(out), flush=True)
    return 0


def read_ceiling(torch, dev, stream, cus, sizes):
    """Time of a plain streaming read of each byte count: the achievable HBM
    read rate at that size, to set each GEMV launch against.

    libawq_probe's read kernel (16-byte non-temporal buffer loads, several in
    flight per lane, one XOR word per workgroup) over a sweep of launch shapes
    (lanes per workgroup, loads in flight per lane, workgroups per CU); the
    fastest is kept.  Each size reads consecutive disjoint slices of a 1 GiB
    buffer (four times the 256 MB Infinity Cache), one launch per slice,
    captured in one graph and replayed: the same cold-cache technique and
    launch path as the GEMV timings.  Returns {bytes: {"us", "GBps", "config"}}.
    """
    import ctypes
    path = os.path.join(ROOT, "weight_only_quantization_pack_amd", "lib", "libawq_probe.so")
    probe = ctypes.CDLL(path)
    probe.awq_probe_read.restype = ctypes.c_int
    probe.awq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    span = 1 << 30
    buf = torch.zeros(span, dtype=torch.uint8, device=dev)
    out = torch.zeros(8 * cus, dtype=torch.int32, device=dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    res = {}
    for B in sizes:
        stride = (B + 4095) // 4096 * 4096
        n = span // stride
        best = None
        for threads, unroll in ((256, 8), (512, 4), (512, 8), (256, 16)):
            for per_cu in (1, 2, 4):
                groups = per_cu * cus

                def sweep():
                    for r in range(n):
                        rc = probe.awq_probe_read(ctypes.c_void_p(buf.data_ptr() + r * stride), B, threads,
                                                  unroll, groups, ctypes.c_void_p(out.data_ptr()), sptr)
                        if rc != 0:
                            raise RuntimeError(f"read probe failed: hip error {rc}")
                with torch.cuda.stream(stream):
                    sweep()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    sweep()
                with torch.cuda.stream(stream):
                    g.replay()
                    torch.cuda.synchronize()
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    n_rep = max(2, 200 // n)
                    a.record(stream)
                    for _ in range(n_rep):
                        g.replay()
                    b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / (n_rep * n)
                if best is None or us < best["us"]:
                    best = {"us": round(us, 3), "GBps": round(B / (us * 1e-6) / 1e9, 1),
                            "config": f"{threads} lanes x {unroll} loads, {per_cu} workgroups per CU"}
                del g
        res[B] = best
        log(f"  read ceiling {B / 1e6:.2f} MB: {best['us']:.2f} us = {best['GBps']:.1f} GB/s ({best['config']})")
    del buf, out
    torch.cuda.empty_cache()
    return res


def cpu_baseline(layer, wl2, shape_index, step_bytes, wl4, wl5):
    """The oracle (not tuned) on the host cores: one decode step of the layer
    (the headline leg), the three M = 2048 prefill products, quantize+pack of
    the 4096 x 4096 layer and its 20-alpha search."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()
                            if d.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = 1
    log("cpu baseline: oracle packing the layer (untimed) ...")
    packs, xs = {}, {}
    for (K, N), i in shape_index.items():
        q, d, z = O.quantize(wl2.weights(i), None, 4)
        packs[(K, N)] = (O.pack(q, 4), d, z)
        xs[K] = wl2.activations(1, i)
    times = []
    t_budget = time.perf_counter()
    while len(times) < 3 and (time.perf_counter() - t_budget) < 30:
        t0 = time.perf_counter()
        for K, N in layer:
            qw, d, z = packs[(K, N)]
            O.matmul(xs[K], qw, d, z, 4, K)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    log(f"cpu baseline: {t:.3f} s per decode step ({len(times)} reps)")
    del packs

    # prefill: the three Mistral-7B products at M = 2048, once each
    flops, secs = 0.0, 0.0
    for i, (K, N) in enumerate(wl4.shapes):
        q, d, z = O.quantize(wl4.weights(i), None, 4)
        qw = O.pack(q, 4)
        x = wl4.activations(2048, i)
        t0 = time.perf_counter()
        O.matmul(x, qw, d, z, 4, K)
        secs += time.perf_counter() - t0
        flops += 2.0 * 2048 * N * K
    log(f"cpu baseline: M = 2048 prefill, three shapes in {secs:.2f} s")

    # quantize + pack of the 4096 x 4096 layer with an activation scale, and
    # the whole 20-alpha search of it on 512 calibration tokens
    W, X = wl5.weights(), wl5.calibration()
    s = O.candidate_scale(O.act_stat(X), 0.5)
    qp = []
    for _ in range(3):
        t0 = time.perf_counter()
        q, d, z = O.quantize(W, s, 4)
        O.pack(q, 4)
        qp.append(time.perf_counter() - t0)
    qp_t = float(np.median(qp))
    qp_bytes = W.size * 2 + W.shape[1] * 4 + W.size // 2 + 4 * W.size // 128
    t0 = time.perf_counter()
    O.search_scale(W, X, wl5.alphas, 4)
    search_t = time.perf_counter() - t0
    log(f"cpu baseline: quantize+pack {qp_t * 1e3:.0f} ms, 20-alpha search {search_t:.2f} s")

    return {"value": round(step_bytes / t / 1e9, 3), "unit": "GB/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": f"{len(times)} full decode steps of the Llama-7B layer (7 GEMVs, M=1) through "
                      f"oracle.matmul: numpy unpack + fp64 dequantize (single-threaded) and fp64 "
                      f"product (OpenBLAS, {blas_threads} threads); median {t:.3f} s per step; "
                      f"host has {os.cpu_count()} logical CPUs",
            "legs": {
                "gemm_m2048": {"value": round(flops / secs / 1e12, 4), "unit": "TFLOP/s",
                               "sample": "the three Mistral-7B prefill products at M = 2048 through "
                                         "oracle.matmul (fp64 BLAS product), once each, "
                                         f"{secs:.2f} s in total"},
                "quantize_pack_4096x4096": {"value": round(qp_bytes / qp_t / 1e9, 4), "unit": "GB/s",
                                            "ms": round(qp_t * 1e3, 1),
                                            "sample": "oracle.quantize (fp32 numpy) + oracle.pack "
                                                      "of the whole layer with s = s_x^0.5, median of 3"},
                "search_4096x4096_T512_20alpha": {"value": round(search_t * 1e3, 1), "unit": "ms",
                                                  "sample": "the whole 20-alpha oracle.search_scale "
                                                            "(fp64 loss per alpha), once"}}}


if __name__ == "__main__":
    sys.exit(main())
