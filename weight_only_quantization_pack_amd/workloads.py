"""Seeded synthetic inputs for the five layer workloads.

This module only draws random numbers; it holds none of the quantization
arithmetic, so both the HIP library's tests and the CPU oracle can take
their inputs from here.  There are no model weights or calibration corpora
in this project, so these distributions stand in for them:

  weights      W[n, k] ~ N(0, 0.02) (fp32 draw, rounded to fp16)
  activations  x[m, k] = c_k * N(0, 1), c_k a per-input-channel magnitude
  outliers     a chosen set of input channels multiplied by a factor

Seeds: numpy PCG64 with seed = 1000*workload + 10*shape_index + stream,
stream 0 = W, 1 = x, 2 = X_cal, 3 = outlier channel indices,
4 = channel magnitudes, 5 = the fresh evaluation x of the offline pass.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

W_STD = 0.02

S_W, S_X, S_XCAL, S_OUTLIER, S_MAG, S_XEVAL = range(6)


def _rng(workload: int, shape_index: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(1000 * workload + 10 * shape_index + stream)


def _to_f16(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float16)


@dataclass
class Workload:
    """One of the five synthetic layer workloads."""
    index: int
    name: str
    shapes: list                     # list of (K, N)
    Ms: list                         # activation row counts exercised
    w_outlier_channels: int = 0      # input channels of W scaled up
    w_outlier_factor: float = 1.0
    mag_sigma: float | None = None   # lognormal(0, sigma) channel magnitudes
    x_outlier_frac: float = 0.0      # fraction of activation channels scaled
    x_outlier_factor: float = 1.0
    calib_tokens: int = 0            # T of the calibration set (0 = none)
    alphas: list = field(default_factory=list)
    bits: tuple = (4,)

    # -- draws -------------------------------------------------------------
    def weights(self, shape_index: int = 0) -> np.ndarray:
        K, N = self.shapes[shape_index]
        rng = _rng(self.index, shape_index, S_W)
        W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(W_STD)
        if self.w_outlier_channels:
            idx = _rng(self.index, shape_index, S_OUTLIER).choice(
                K, self.w_outlier_channels, replace=False)
            W[:, idx] *= np.float32(self.w_outlier_factor)
        return _to_f16(W)

    def channel_magnitudes(self, shape_index: int = 0) -> np.ndarray:
        K = self.shapes[shape_index][0]
        c = np.ones(K, dtype=np.float32)
        if self.mag_sigma is not None:
            c = _rng(self.index, shape_index, S_MAG).lognormal(
                0.0, self.mag_sigma, K).astype(np.float32)
        if self.x_outlier_frac > 0:
            n_out = max(1, int(round(self.x_outlier_frac * K)))
            idx = _rng(self.index, shape_index, S_OUTLIER + 10).choice(K, n_out, replace=False)
            c[idx] *= np.float32(self.x_outlier_factor)
        return c

    def _acts(self, rows: int, shape_index: int, stream: int) -> np.ndarray:
        K = self.shapes[shape_index][0]
        c = self.channel_magnitudes(shape_index)
        z = _rng(self.index, shape_index, stream).standard_normal((rows, K), dtype=np.float32)
        return _to_f16(z * c[None, :])

    def activations(self, M: int, shape_index: int = 0) -> np.ndarray:
        return self._acts(M, shape_index, S_X)

    def calibration(self, shape_index: int = 0) -> np.ndarray:
        if not self.calib_tokens:
            raise ValueError(f"workload {self.index} has no calibration set")
        return self._acts(self.calib_tokens, shape_index, S_XCAL)

    def eval_activations(self, M: int, shape_index: int = 0) -> np.ndarray:
        return self._acts(M, shape_index, S_XEVAL)


WORKLOADS = {
    1: Workload(1, "single linear 512x512, int4 g128, alpha 0.5",
                shapes=[(512, 512)], Ms=[1, 16], w_outlier_channels=4,
                w_outlier_factor=20.0, mag_sigma=1.0, calib_tokens=128,
                alphas=[0.5]),
    2: Workload(2, "Llama-7B decode GEMV, M=1",
                shapes=[(4096, 4096), (4096, 11008), (11008, 4096)], Ms=[1],
                mag_sigma=1.5),
    3: Workload(3, "Llama-70B MLP batched decode",
                shapes=[(8192, 28672), (28672, 8192)], Ms=[1, 4, 16, 64],
                x_outlier_frac=0.01, x_outlier_factor=30.0),
    4: Workload(4, "Mistral-7B prefill GEMM",
                shapes=[(4096, 14336), (14336, 4096), (4096, 6144)], Ms=[512, 2048],
                mag_sigma=1.0),
    5: Workload(5, "full AWQ offline pass, 4096x4096, 20-point alpha grid",
                shapes=[(4096, 4096)], Ms=[1], mag_sigma=1.5, calib_tokens=512,
                alphas=[i / 20 for i in range(20)], bits=(4, 3)),
}

# The Llama-7B decoder layer's linears at decode: q, k, v, o (4096x4096),
# gate, up (4096 -> 11008) and down (11008 -> 4096), as (K, N).
LLAMA7B_LAYER = [(4096, 4096)] * 4 + [(4096, 11008)] * 2 + [(11008, 4096)]


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def random_weights(N: int, K: int, seed: int, std: float = W_STD) -> np.ndarray:
    """Plain N(0, std) fp16 weights for ad-hoc shapes (ragged and edge cases)."""
    rng = np.random.default_rng(seed)
    return _to_f16(rng.standard_normal((N, K), dtype=np.float32) * np.float32(std))


def random_activations(M: int, K: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    """c_k * N(0,1) fp16 activations with lognormal(0, sigma) channel scales."""
    rng = np.random.default_rng(seed)
    c = rng.lognormal(0.0, sigma, K).astype(np.float32)
    return _to_f16(rng.standard_normal((M, K), dtype=np.float32) * c[None, :])
