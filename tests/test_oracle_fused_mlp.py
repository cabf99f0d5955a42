"""Pins for the oracle's folded activation scale and the gate/up half of the
fused MLP ("transformers - AWQ", "Fused modules"; the activation side of the
equivalent transform, section 02.02 "AWQ" of the VPTQ blog).

Each check comes from outside the oracle's formulas: SiLU against the
hyperbolic-tangent form of the logistic function, its odd-part identity and
closed values; the folded scale against exact power-of-two products and
against ``scale_activations`` (one fp16 ulp apart at most); gate_up against
a hand-derived closed form on one-hot activations over exactly representable
weights, which also tells gate from up.
"""
import numpy as np
import pytest

import oracle as O


def test_silu_tanh_form_and_identities():
    t = np.linspace(-30, 30, 20001)
    # sigmoid(t) = (1 + tanh(t / 2)) / 2 (cancels below -2, where
    # sigmoid(t) = e^t / (1 + e^t) is used instead)
    want = np.where(t >= -2, t * 0.5 * (1.0 + np.tanh(t / 2.0)), t * np.exp(t) / (1.0 + np.exp(t)))
    assert np.allclose(O.silu(t), want, rtol=1e-13, atol=1e-300)
    # SiLU(t) - SiLU(-t) = t (t sigmoid(t) + t sigmoid(-t) = t)
    assert np.allclose(O.silu(t) - O.silu(-t), t, rtol=0, atol=8e-15)
    assert O.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3 / 4
    assert abs(O.silu(np.log(3.0)) - 0.75 * np.log(3.0)) <= 2.3e-16
    # tails: SiLU(t) -> t above, -> t e^t below
    assert O.silu(50.0) == 50.0
    assert abs(O.silu(-50.0) / (-50.0 * np.exp(-50.0)) - 1.0) < 1e-15
    assert O.silu(-1000.0) == 0.0
    # slope 1/2 at 0
    h = 1e-6
    assert abs((O.silu(h) - O.silu(-h)) / (2 * h) - 0.5) < 1e-9


def test_apply_inv_scale_power_of_two_is_exact():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((3, 256)) * 4).astype(np.float16)
    e = rng.integers(-3, 4, 256)
    inv_s = np.ldexp(1.0, e).astype(np.float32)
    got = O.apply_inv_scale(x, inv_s)
    assert np.array_equal(got.astype(np.float64), x.astype(np.float64) * inv_s.astype(np.float64)[None, :])


def test_apply_inv_scale_within_one_ulp_of_division():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 512)) * rng.lognormal(0, 1.5, 512)).astype(np.float16)
    s = rng.lognormal(0, 1, 512).astype(np.float32)
    inv_s = (np.float32(1) / s).astype(np.float32)
    a = O.apply_inv_scale(x, inv_s)
    b = O.scale_activations(x, s)
    ia = a.view(np.int16).astype(np.int32)
    ib = b.view(np.int16).astype(np.int32)
    assert np.all(np.abs(ia - ib) <= 1)                 # same sign; at most one fp16 step
    assert np.mean(ia == ib) > 0.99


def _exact_layer(N, K, seed, bits=4):
    """Weights on a quantization grid: (i - 7) 2^-e per row, so w_hat == W."""
    rng = np.random.default_rng(seed)
    i = rng.integers(0, 16, (N, K))
    i[:, ::128] = 0
    i[:, 1::128] = 15                                  # every group spans 0..15
    e = rng.integers(5, 8, (N, 1))
    W = ((i - 7) * np.ldexp(1.0, -e)).astype(np.float16)
    q, d, z = O.quantize(W, None, bits)
    assert np.array_equal(O.dequantize(q, d, z), W.astype(np.float64))
    return W, (O.pack(q, bits), d, z)


def test_gate_up_closed_form_one_hot():
    N, K = 40, 256
    Wg, gate = _exact_layer(N, K, 1)
    Wu, up = _exact_layer(N, K, 2)
    inv_s = np.ones(K, np.float32)
    inv_s[::3] = 2.0
    for k0, c in [(0, 1.5), (5, -2.0), (129, 0.75), (255, 3.0)]:
        x = np.zeros((1, K), np.float16)
        x[0, k0] = c
        xs = c * float(inv_s[k0])
        g = xs * Wg[:, k0].astype(np.float64)
        u = xs * Wu[:, k0].astype(np.float64)
        want = g * 0.5 * (1.0 + np.tanh(g / 2.0)) * u
        got = O.gate_up(x, inv_s, gate, up, 4, K)[0]
        assert np.allclose(got, want, rtol=1e-14, atol=0)
        swapped = O.gate_up(x, inv_s, up, gate, 4, K)[0]
        assert not np.allclose(swapped, want, rtol=1e-6, atol=0)
    # no scale: x used as is
    x = np.zeros((1, K), np.float16)
    x[0, 3] = 2.0
    g = 2.0 * Wg[:, 3].astype(np.float64)
    u = 2.0 * Wu[:, 3].astype(np.float64)
    assert np.allclose(O.gate_up(x, None, gate, up, 4, K)[0], g * 0.5 * (1 + np.tanh(g / 2)) * u,
                       rtol=1e-14, atol=0)


def test_gate_up_rows_matches_full():
    rng = np.random.default_rng(4)
    K, N = 256, 48
    gate = O.quantize((rng.standard_normal((N, K)) * 0.02).astype(np.float16), None, 4)
    up = O.quantize((rng.standard_normal((N, K)) * 0.02).astype(np.float16), None, 4)
    gate = (O.pack(gate[0], 4), gate[1], gate[2])
    up = (O.pack(up[0], 4), up[1], up[2])
    x = rng.standard_normal((3, K)).astype(np.float16)
    inv_s = rng.lognormal(0, 0.5, K).astype(np.float32)
    full = O.gate_up(x, inv_s, gate, up, 4, K)
    rows = np.array([0, 17, 47])
    assert np.array_equal(O.gate_up_rows(x, inv_s, gate, up, 4, K, rows), full[:, rows])


@pytest.mark.parametrize("bits", [4, 3])
def test_gate_up_equivalent_transform_keeps_the_product(bits):
    """With s folded into the weights and 1/s into x, the fused output stays
    close to the unquantized silu(x Wg^T) (x Wu^T): the transform is exact in
    real arithmetic, so the gap is the quantization error alone."""
    rng = np.random.default_rng(21)
    K, N = 512, 64
    Wg = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    Wu = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = (rng.standard_normal((4, K)) * rng.lognormal(0, 1, K)).astype(np.float16)
    s = O.candidate_scale(O.act_stat(x), 0.5)
    gq = O.quantize(Wg, s, bits)
    uq = O.quantize(Wu, s, bits)
    gate = (O.pack(gq[0], bits), gq[1], gq[2])
    up = (O.pack(uq[0], bits), uq[1], uq[2])
    got = O.gate_up(x, (np.float32(1) / s).astype(np.float32), gate, up, bits, K)
    x64 = x.astype(np.float64)
    g = x64 @ Wg.astype(np.float64).T
    u = x64 @ Wu.astype(np.float64).T
    want = O.silu(g) * u
    rel = np.max(np.abs(got - want)) / np.max(np.abs(want))
    assert rel < (0.15 if bits == 4 else 0.35)
