"""Pins for the oracle's symmetric quantizer (zero_point=False).

"Quantizing a model with AutoAWQ" ([P4]): zero_point chooses asymmetric
quantization with a zero point (True) or symmetric quantization (False).
The reading: the textbook zero-centred grid, D = largest fp16 <= max|v| /
(2^(b-1) - 1), codes rint(v/D) in -Qs..Qs stored with the fixed offset
z = 2^(b-1).  Each check comes from outside the oracle's formula: brute force
over the fp16 table and over integer codes, a hand-derived closed form with
literal packed words, and invariants of a zero-centred round-to-nearest grid
(negation symmetry, idempotence, the half-step error bound with no clamping).
"""
import numpy as np
import pytest

import oracle as O

_ALL_F16 = np.arange(0x0001, 0x7C00, dtype=np.uint16).view(np.float16)
_ALL_F16_AS32 = _ALL_F16.astype(np.float32)


def _round_down_f16(x32):
    return _ALL_F16[np.searchsorted(_ALL_F16_AS32, np.float32(x32), side="right") - 1]


def _nearest_even(val):
    lo = int(np.floor(val))
    d_lo, d_hi = val - lo, (lo + 1) - val
    if d_lo != d_hi:
        return lo if d_lo < d_hi else lo + 1
    return lo if lo % 2 == 0 else lo + 1


def _brute_symmetric_group(v, bits):
    """(fp16 scale, zero, codes) of one group by enumeration."""
    Q, qs, z = (1 << bits) - 1, (1 << (bits - 1)) - 1, 1 << (bits - 1)
    amax = max(max(abs(float(t)) for t in v), 1e-5)
    dh = _round_down_f16(np.float32(np.float32(amax) / np.float32(qs)))
    d = np.float32(dh)
    codes = []
    for t in v:
        a = float(np.float32(np.float32(t) / d))          # the fp32 quotient
        # nearest integer by enumeration over the whole code range
        best = min(range(-z, Q - z + 1), key=lambda j: (abs(a - j), j % 2))
        assert best == _nearest_even(a) or abs(a) > qs + 0.5
        codes.append(min(max(best + z, 0), Q))
    return dh, z, np.array(codes)


def _tiles(bits):
    rng = np.random.default_rng(40 + bits)
    out = [(rng.standard_normal((4, 128)) * 0.02).astype(np.float32)]
    t = ((rng.integers(-3, 3, (4, 128)) + 0.5) * 2.0 ** -6).astype(np.float32)   # exact .5 ties
    t[:, 0] = 3.5 * 2.0 ** -6
    out.append(t)
    out.append(np.abs(rng.standard_normal((4, 128)) * 0.02).astype(np.float32) + np.float32(0.01))
    out.append(-np.abs(rng.standard_normal((4, 128)) * 0.02).astype(np.float32) - np.float32(0.01))
    out.append(np.zeros((4, 128), np.float32))
    o = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    o[:, 17] *= 20
    out.append(o)
    return out


@pytest.mark.parametrize("bits", [4, 3])
def test_symmetric_brute_force_on_4x128_tiles(bits):
    for tile in _tiles(bits):
        q, d, z = O.quantize_values(tile, bits, zero_point=False)
        for n in range(4):
            dh, zz, codes = _brute_symmetric_group(tile[n], bits)
            assert d[n, 0].view(np.uint16) == dh.view(np.uint16)
            assert float(z[n, 0]) == zz
            assert np.array_equal(q[n].astype(np.int64), codes)


def test_symmetric_closed_form_int4():
    # values (i - 7) * 2^-6, i = 0..14 repeating: max|v| = 7 * 2^-6, so
    # D = 7 * 2^-6 / 7 = 2^-6 exactly, z = 8 and q = (i - 7) + 8 = i + 1.
    i = np.arange(128) % 15
    v = ((i - 7) * 2.0 ** -6).astype(np.float32)[None, :]
    q, d, z = O.quantize_values(v, 4, zero_point=False)
    assert np.array_equal(q[0], (i + 1).astype(np.uint8))
    assert int(d[0, 0].view(np.uint16)) == 0x2400            # fp16 2^-6
    assert float(z[0, 0]) == 8.0
    # packed words: code 8j+2t at bits 4t, code 8j+2t+1 at bits 16+4t.
    # codes 1..8 -> low nibbles 1,3,5,7 and high nibbles 2,4,6,8;
    # codes 9..15,1 -> low 9,11,13,15 and high 10,12,14,1.
    words = O.pack_rows(q, 4)[0]
    assert int(words[0]) == 0x86427531
    assert int(words[1]) == 0x1ECAFDB9


def test_symmetric_closed_form_int3():
    # values (i - 3) * 2^-6, i = 0..6 repeating: D = 3 * 2^-6 / 3 = 2^-6, z = 4, q = i + 1
    i = np.arange(128) % 7
    v = ((i - 3) * 2.0 ** -6).astype(np.float32)[None, :]
    q, d, z = O.quantize_values(v, 3, zero_point=False)
    assert np.array_equal(q[0], (i + 1).astype(np.uint8))
    assert int(d[0, 0].view(np.uint16)) == 0x2400
    assert float(z[0, 0]) == 4.0


def _layer(n_rows=512, seed=5):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n_rows, 256)) * 0.02).astype(np.float32)
    W[:, rng.choice(256, 4, replace=False)] *= 20
    s = rng.lognormal(0, 1, 256).astype(np.float32)
    return W.astype(np.float16), s


@pytest.mark.parametrize("bits", [4, 3])
def test_symmetric_negation(bits):
    """A zero-centred grid with half-to-even rounding commutes with negation."""
    W, s = _layer()
    v = W.astype(np.float32) * s[None, :]
    q1, d1, z1 = O.quantize_values(v, bits, zero_point=False)
    q2, d2, z2 = O.quantize_values(-v, bits, zero_point=False)
    assert np.array_equal(d1.view(np.uint16), d2.view(np.uint16)) and np.array_equal(z1, z2)
    zz = np.repeat(z1.astype(np.int64), 128, axis=1)
    assert np.array_equal(q2.astype(np.int64), 2 * zz - q1.astype(np.int64))


@pytest.mark.parametrize("bits", [4, 3])
def test_symmetric_idempotent_and_half_step_bound(bits):
    W, s = _layer()
    q, d, z = O.quantize(W, s, bits, zero_point=False)
    qs = (1 << (bits - 1)) - 1
    zz = np.repeat(z.astype(np.int64), 128, axis=1)
    # |v| / D <= qs (1 + 2^-10) < qs + 1/2: no code is clamped
    assert np.all(np.abs(q.astype(np.int64) - zz) <= qs)
    w_hat = O.dequantize(q, d, z)
    v = W.astype(np.float32).astype(np.float64) * s.astype(np.float64)[None, :]
    v32 = (W.astype(np.float32) * s[None, :]).astype(np.float64)
    dd = np.repeat(d.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(v32 - w_hat) <= 0.5 * dd * (1 + 2.0 ** -20))
    assert np.max(np.abs(v - w_hat) / dd) < 0.51
    q2, d2, z2 = O.quantize_values(w_hat.astype(np.float32), bits, zero_point=False)
    assert np.array_equal(q, q2) and np.array_equal(d.view(np.uint16), d2.view(np.uint16))
    assert np.array_equal(z, z2)


def test_symmetric_zero_group():
    q, d, z = O.quantize_values(np.zeros((1, 128), np.float32), 4, zero_point=False)
    assert np.all(q == 8) and float(z[0, 0]) == 8.0
    assert d[0, 0].view(np.uint16) == _round_down_f16(np.float32(1e-5) / np.float32(7)).view(np.uint16)
    assert np.all(O.dequantize(q, d, z) == 0.0)


def test_symmetric_search_is_a_grid_search():
    """L(alpha*) <= L(0) and the first minimum wins on a duplicated grid."""
    rng = np.random.default_rng(8)
    W, _ = _layer(64, seed=9)
    X = (rng.standard_normal((32, 256)) * rng.lognormal(0, 1.5, 256)).astype(np.float16)
    alphas = [0.0, 0.25, 0.5, 0.5, 0.75]
    s, losses, best = O.search_scale(W, X, alphas, 4, zero_point=False)
    assert losses[best] <= losses[0]
    assert best == int(np.argmin(losses)) and best != 3
    q, d, z = O.quantize(W, O.candidate_scale(O.act_stat(X), alphas[best]), 4, zero_point=False)
    assert np.isclose(O.output_mse(X, W, O.dequantize(q, d, z), s), losses[best], rtol=0, atol=0)
