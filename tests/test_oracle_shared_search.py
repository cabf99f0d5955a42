"""Pins for the oracle's shared-input scale search (one s for the layers
that read one input; section 02.02 "AWQ" of the VPTQ blog, "Usage" step 1 of
the llm-awq README).

Checked from outside the concatenation that defines it: each grid point's
shared loss is the row-weighted mean of the layers' own output MSEs computed
one layer at a time; the pick is the brute-force first minimum of that mean;
one layer reduces to the single-layer search; the order of the layers does
not matter; and a layer pair whose own optima differ gets the alpha of the
weighted sum, not either layer's.
"""
import numpy as np
import pytest

import oracle as O


def _layers(seed, Ns=(96, 32, 32), K=256):
    rng = np.random.default_rng(seed)
    Ws = []
    for i, n in enumerate(Ns):
        W = (rng.standard_normal((n, K)) * 0.02).astype(np.float32)
        W[:, rng.choice(K, 3, replace=False)] *= 10 + 10 * i
        Ws.append(W.astype(np.float16))
    X = (rng.standard_normal((48, K)) * rng.lognormal(0, 1.5, K)).astype(np.float16)
    return Ws, X


ALPHAS = [0.0, 0.2, 0.4, 0.6, 0.8]


@pytest.mark.parametrize("bits", [4, 3])
def test_shared_loss_is_the_row_weighted_mean_of_layer_losses(bits):
    Ws, X = _layers(1)
    s, losses, best = O.search_scale_shared(Ws, X, ALPHAS, bits)
    s_x = O.act_stat(X)
    Ns = np.array([w.shape[0] for w in Ws], np.float64)
    want = []
    for a in ALPHAS:
        sa = O.candidate_scale(s_x, a)
        per = []
        for W in Ws:
            q, d, z = O.quantize(W, sa, bits)
            per.append(O.output_mse(X, W, O.dequantize(q, d, z), sa))
        want.append(float(np.dot(Ns, per) / Ns.sum()))
    assert np.allclose(losses, want, rtol=1e-12, atol=0)
    first_min = min(range(len(want)), key=lambda i: (want[i], i))
    assert best == first_min
    assert np.array_equal(s, O.candidate_scale(s_x, ALPHAS[best]))


def test_one_layer_is_the_single_layer_search():
    Ws, X = _layers(2, Ns=(64,))
    a = O.search_scale_shared(Ws, X, ALPHAS, 4)
    b = O.search_scale(Ws[0], X, ALPHAS, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_layer_order_does_not_matter():
    Ws, X = _layers(3)
    a = O.search_scale_shared(Ws, X, ALPHAS, 4)
    b = O.search_scale_shared(Ws[::-1], X, ALPHAS, 4)
    assert np.allclose(a[1], b[1], rtol=1e-12, atol=0) and a[2] == b[2]


def test_layers_with_different_optima_get_the_weighted_choice():
    """Layer A (weights independent of the channel) alone prefers a middle
    alpha; layer B, whose weights shrink as its input channel grows (so x w
    is flat across channels), prefers the largest one.  The shared search
    lands on the minimum of their mean loss, which is not B's own choice."""
    rng = np.random.default_rng(9)
    K = 256
    X = (rng.standard_normal((64, K)) * rng.lognormal(0, 2.0, K)).astype(np.float16)
    sx = O.act_stat(X).astype(np.float64)
    A = (rng.standard_normal((64, K)) * 0.02).astype(np.float16)
    B = (rng.standard_normal((64, K)) * 0.02 / (sx / sx.mean())[None, :]).astype(np.float32)
    B = (B / np.abs(B).max() * 0.5).astype(np.float16)
    grid = [i / 10 for i in range(10)]
    _, la, ba = O.search_scale(A, X, grid, 4)
    _, lb, bb = O.search_scale(B, X, grid, 4)
    _, ls, bs = O.search_scale_shared([A, B], X, grid, 4)
    assert ba != bb
    assert np.allclose(ls, (la + lb) / 2, rtol=1e-12, atol=0)
    assert bs == int(np.argmin((la + lb) / 2))
    assert bs != bb and ls[bs] <= ls[0]
