"""Pins for the oracle's 64-wide groups ("Quantizing a model with AutoAWQ"
([P4]): q_group_size, typical values 64 and 128).

A packed tile still spans 128 codes, so with 64-wide groups a tile carries
two groups.  Checks from outside the oracle's formula: brute force per
64-code group over the fp16 table and the integer codes, a closed form with
two different scales in one tile, idempotence, the half-step bound, and
that a 64-group never quantizes worse than the 128-group holding it.
"""
import numpy as np
import pytest

import oracle as O

_ALL_F16 = np.arange(0x0001, 0x7C00, dtype=np.uint16).view(np.float16)
_ALL_F16_AS32 = _ALL_F16.astype(np.float32)


def _round_down_f16(x32):
    return _ALL_F16[np.searchsorted(_ALL_F16_AS32, np.float32(x32), side="right") - 1]


def _nearest(a, lo, hi):
    """Integer in [lo, hi] nearest to a, exact halves to the even one."""
    return min(range(lo, hi + 1), key=lambda j: (abs(a - j), j % 2))


def _brute_group(v, bits, zero_point):
    Q = (1 << bits) - 1
    if zero_point:
        lo = min(0.0, float(v.min()))
        hi = max(0.0, float(v.max()))
        d32 = np.float32(np.float32(max(np.float32(hi - lo), np.float32(1e-5))) / np.float32(Q))
        dh = _round_down_f16(d32)
        z = min(max(_nearest(float(np.float32(np.float32(-lo) / np.float32(dh))), -64, 64), 0), Q)
    else:
        qs = (1 << (bits - 1)) - 1
        amax = max(float(np.abs(v).max()), 1e-5)
        dh = _round_down_f16(np.float32(np.float32(amax) / np.float32(qs)))
        z = 1 << (bits - 1)
    d = np.float32(dh)
    codes = [min(max(_nearest(float(np.float32(np.float32(t) / d)), -64, 64) + z, 0), Q) for t in v]
    return dh, z, np.array(codes)


def _tiles(seed):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    b = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    b[:, 64:] *= 8                                   # the two halves on very different scales
    c = np.abs(rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    c[:, 64:] = -c[:, 64:]                           # one-sided halves of opposite sign
    d = np.zeros((4, 128), np.float32)
    d[:, 64:] = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)   # an all-zero half
    t = ((rng.integers(-3, 3, (4, 128)) + 0.5) * 2.0 ** -6).astype(np.float32)   # .5 ties
    return [a, b, c, d, t]


@pytest.mark.parametrize("zero_point", [True, False])
@pytest.mark.parametrize("bits", [4, 3])
def test_group64_brute_force(bits, zero_point):
    for tile in _tiles(60 + bits):
        q, d, z = O.quantize_values(tile, bits, 64, zero_point)
        assert d.shape == (4, 2)
        for n in range(4):
            for g in range(2):
                dh, zz, codes = _brute_group(tile[n, 64 * g:64 * g + 64], bits, zero_point)
                assert d[n, g].view(np.uint16) == dh.view(np.uint16)
                assert float(z[n, g]) == zz
                assert np.array_equal(q[n, 64 * g:64 * g + 64].astype(np.int64), codes)


def test_group64_closed_form_two_scales_in_one_tile():
    # half 0: (i - 7) 2^-6, half 1: (i - 7) 2^-5, i = 0..15 repeating:
    # span 15 * 2^-6 (2^-5) / 15 -> D = 2^-6 and 2^-5 exactly, z = 7, q = i
    i = np.arange(64) % 16
    v = np.concatenate([(i - 7) * 2.0 ** -6, (i - 7) * 2.0 ** -5]).astype(np.float32)[None, :]
    q, d, z = O.quantize_values(v, 4, 64)
    assert np.array_equal(q[0], np.concatenate([i, i]).astype(np.uint8))
    assert [int(t) for t in d[0].view(np.uint16)] == [0x2400, 0x2800]      # fp16 2^-6, 2^-5
    assert [float(t) for t in z[0]] == [7.0, 7.0]
    w_hat = O.dequantize(q, d, z, 64)
    assert np.array_equal(w_hat, v.astype(np.float64))                      # exact grid values


def _layer(seed=3, n=256):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n, 256)) * 0.02).astype(np.float32)
    W[:, rng.choice(256, 4, replace=False)] *= 20
    s = rng.lognormal(0, 1, 256).astype(np.float32)
    return W.astype(np.float16), s


@pytest.mark.parametrize("zero_point", [True, False])
@pytest.mark.parametrize("bits", [4, 3])
def test_group64_idempotent_and_bounded(bits, zero_point):
    W, s = _layer()
    q, d, z = O.quantize(W, s, bits, 64, zero_point)
    w_hat = O.dequantize(q, d, z, 64)
    q2, d2, z2 = O.quantize_values(w_hat.astype(np.float32), bits, 64, zero_point)
    assert np.array_equal(q, q2) and np.array_equal(d.view(np.uint16), d2.view(np.uint16))
    assert np.array_equal(z, z2)
    v = (W.astype(np.float32) * s[None, :]).astype(np.float64)
    dd = np.repeat(d.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(v - w_hat) <= 0.52 * dd)


def test_group64_refines_group128():
    """Per element the 64-group scale is at most the 128-group scale holding it,
    so the total squared error is no larger (checked on a whole layer)."""
    W, s = _layer(7, 512)
    q6, d6, z6 = O.quantize(W, s, 4, 64)
    q1, d1, z1 = O.quantize(W, s, 4, 128)
    assert np.all(d6.astype(np.float64) <= np.repeat(d1.astype(np.float64), 2, axis=1))
    v = (W.astype(np.float32) * s[None, :]).astype(np.float64)
    e6 = np.sum((v - O.dequantize(q6, d6, z6, 64)) ** 2)
    e1 = np.sum((v - O.dequantize(q1, d1, z1, 128)) ** 2)
    assert e6 < e1


def test_group64_matmul_reads_the_group_size_from_the_parameters():
    W, _ = _layer(9, 48)
    q, d, z = O.quantize(W, None, 4, 64)
    x = np.random.default_rng(1).standard_normal((3, 256)).astype(np.float16)
    want = x.astype(np.float64) @ O.dequantize(q, d, z, 64).T
    assert np.array_equal(O.matmul(x, O.pack(q, 4), d, z, 4, 256), want)
    rows = np.array([0, 5, 47])
    assert np.array_equal(O.matmul_rows(x, O.pack(q, 4), d, z, 4, 256, rows), want[:, rows])
