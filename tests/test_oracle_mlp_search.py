"""Pins for the oracle's block-output search of the gate/up scale
(``mlp_block_loss`` / ``search_scale_mlp``; "Usage" step 1 of the llm-awq
README, section 02.02 "AWQ" of the VPTQ blog, the MLP of "transformers - AWQ"
"Fused modules").

Checked from outside its numpy form: pure-Python loops on a tiny block, an
exact zero for weights already on the quantization grid, exact power-of-two
scaling in the down projection, invariance under a joint permutation of the
intermediate channels, gate and up not interchangeable, the identity down
projection, and the search's first minimum.
"""
import math

import numpy as np
import pytest

import oracle as O


def _block(seed, K=256, I=48, K_out=40, T=24):
    rng = np.random.default_rng(seed)
    Wg = (rng.standard_normal((I, K)) * 0.05).astype(np.float16)
    Wu = (rng.standard_normal((I, K)) * 0.05).astype(np.float16)
    Wg[:, rng.choice(K, 3, replace=False)] *= 8
    Wd = (rng.standard_normal((K_out, I)) * 0.05).astype(np.float16)
    X = (rng.standard_normal((T, K)) * rng.lognormal(0, 1.0, K)).astype(np.float16)
    return X, Wg, Wu, Wd


@pytest.mark.parametrize("bits,zero_point", [(4, True), (3, True), (4, False)])
def test_loops_on_a_tiny_block(bits, zero_point):
    X, Wg, Wu, Wd = _block(1, K=128, I=6, K_out=5, T=3)
    s = O.candidate_scale(O.act_stat(X), 0.5)
    got = O.mlp_block_loss(X, Wg, Wu, Wd, s, bits, 128, zero_point)

    def w_hat(W):
        q, d, z = O.quantize(W, s, bits, 128, zero_point)
        return [[(int(q[n, k]) - float(z[n, k // 128])) * float(d[n, k // 128]) / float(s[k])
                 for k in range(W.shape[1])] for n in range(W.shape[0])]

    def silu(t):
        return t / (1.0 + math.exp(-t))

    hg, hu = w_hat(Wg), w_hat(Wu)
    T, K = X.shape
    I, K_out = Wg.shape[0], Wd.shape[0]
    x = [[float(X[t, k]) for k in range(K)] for t in range(T)]
    tot = 0.0
    for t in range(T):
        dh = []
        for i in range(I):
            gq = sum(x[t][k] * hg[i][k] for k in range(K))
            uq = sum(x[t][k] * hu[i][k] for k in range(K))
            g = sum(x[t][k] * float(Wg[i, k]) for k in range(K))
            u = sum(x[t][k] * float(Wu[i, k]) for k in range(K))
            dh.append(silu(gq) * uq - silu(g) * u)
        for o in range(K_out):
            e = sum(dh[i] * float(Wd[o, i]) for i in range(I))
            tot += e * e
    want = tot / (T * K_out)
    assert abs(got - want) <= 1e-10 * want


def test_weights_on_the_grid_give_zero_at_alpha_zero():
    """Gate and up rows whose groups hold (q - 7) * 2^-6 with codes 0 and 15
    present: with s = 1 (alpha = 0) they quantize to themselves, so the block
    output is unchanged and the loss is exactly 0."""
    rng = np.random.default_rng(2)
    I, K = 16, 256
    mats = []
    for _ in range(2):
        q = rng.integers(0, 16, (I, K))
        q[:, ::128], q[:, 1::128] = 0, 15
        mats.append(((q - 7) * 2.0 ** -6).astype(np.float16))
    X, _, _, Wd = _block(3, K=K, I=I)
    s, losses, best = O.search_scale_mlp(X, mats[0], mats[1], Wd, [0.0, 0.5])
    assert losses[0] == 0.0 and best == 0


def test_down_projection_scaling_is_exact():
    X, Wg, Wu, Wd = _block(4)
    s = O.candidate_scale(O.act_stat(X), 0.35)
    base = O.mlp_block_loss(X, Wg, Wu, Wd, s)
    for p in (1, 3):
        Wd2 = (Wd.astype(np.float32) * 2.0 ** p).astype(np.float16)
        assert np.array_equal(Wd2.astype(np.float64), Wd.astype(np.float64) * 2.0 ** p)   # exact in fp16
        assert O.mlp_block_loss(X, Wg, Wu, Wd2, s) == base * 4.0 ** p


def test_joint_permutation_of_intermediate_channels():
    X, Wg, Wu, Wd = _block(5)
    s = O.candidate_scale(O.act_stat(X), 0.6)
    perm = np.random.default_rng(6).permutation(Wg.shape[0])
    a = O.mlp_block_loss(X, Wg, Wu, Wd, s, 3)
    b = O.mlp_block_loss(X, Wg[perm], Wu[perm], Wd[:, perm], s, 3)
    assert abs(a - b) <= 1e-12 * a
    # permuting only the down projection's columns is a different block
    c = O.mlp_block_loss(X, Wg, Wu, Wd[:, perm], s, 3)
    assert abs(a - c) > 1e-3 * a


def test_gate_and_up_are_not_interchangeable():
    X, Wg, Wu, Wd = _block(7)
    s = O.candidate_scale(O.act_stat(X), 0.5)
    a = O.mlp_block_loss(X, Wg, Wu, Wd, s)
    b = O.mlp_block_loss(X, Wu, Wg, Wd, s)
    assert abs(a - b) > 1e-2 * a


def test_identity_down_projection_is_the_gate_up_error():
    """Wd = identity: the loss is the mean squared error of SiLU(g) * u itself,
    with g, u from the fake-quantized pair (the same weights the oracle's
    fused gate/up evaluates)."""
    X, Wg, Wu, _ = _block(8, I=32)
    s = O.candidate_scale(O.act_stat(X), 0.4)
    eye = np.eye(32, dtype=np.float16)
    got = O.mlp_block_loss(X, Wg, Wu, eye, s)
    Xd = X.astype(np.float64)
    hat = []
    for W in (Wg, Wu):
        q, d, z = O.quantize(W, s)
        hat.append(O.dequantize(q, d, z) / s.astype(np.float64))
    hq = O.silu(Xd @ hat[0].T) * (Xd @ hat[1].T)
    h = O.silu(Xd @ Wg.astype(np.float64).T) * (Xd @ Wu.astype(np.float64).T)
    assert abs(got - float(np.mean((hq - h) ** 2))) <= 1e-12 * got


def test_search_takes_the_first_minimum_and_beats_rtn():
    X, Wg, Wu, Wd = _block(9)
    alphas = [0.0, 0.25, 0.5, 0.5, 0.75]
    s, losses, best = O.search_scale_mlp(X, Wg, Wu, Wd, alphas)
    for a, l in zip(alphas, losses):
        assert l == O.mlp_block_loss(X, Wg, Wu, Wd, O.candidate_scale(O.act_stat(X), a))
    assert best == int(np.flatnonzero(losses == losses.min())[0])
    assert losses[best] <= losses[0]
    assert np.array_equal(s, O.candidate_scale(O.act_stat(X), alphas[best]))
    if losses[2] == losses.min():
        assert best == 2                       # duplicate grid point: the first one
