"""Pins for the oracle's rotary embedding.

Invariants (identity at p=0, per-pair norm, composition, relative position)
catch a wrong rotation structure; the 50-digit complex twin and the hand
values catch a wrong sign, a wrong pairing or a wrong frequency exponent.
"""

import mpmath
import numpy as np
import pytest

import oracle

THETA = 1.0e6


def test_hand_values(golden):
    for name, idx, pos, exp in golden("rope_hand.txt"):
        x = np.zeros(128)
        x[int(idx)] = 1.0
        y = oracle.rope(x, int(pos), THETA)
        e = np.zeros(128)
        for item in exp.split():
            i, v = item.split(":")
            e[int(i)] = float(v)
        assert np.allclose(y, e, rtol=0, atol=1e-12), name


def test_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((5, 128))
    assert np.array_equal(oracle.rope(x, 0, THETA), x)


def test_pair_norms_preserved():
    g = np.random.default_rng(1)
    x = g.standard_normal((16, 128))
    p = g.integers(0, 4096, 16)
    y = oracle.rope(x, p, THETA)
    n0 = x[:, :64] ** 2 + x[:, 64:] ** 2
    n1 = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-13, atol=1e-13)


def test_composition():
    g = np.random.default_rng(2)
    x = g.standard_normal(128)
    for a, b in [(3, 5), (100, 2047), (1, 0), (1000, 1176)]:
        assert np.allclose(oracle.rope(oracle.rope(x, a, THETA), b, THETA),
                           oracle.rope(x, a + b, THETA), rtol=0, atol=1e-11)


def test_relative_position():
    g = np.random.default_rng(3)
    q, k = g.standard_normal(128), g.standard_normal(128)
    for m, n in [(0, 7), (5, 5), (2047, 2049), (100, 2175)]:
        lhs = oracle.rope(q, m, THETA) @ oracle.rope(k, n, THETA)
        rhs = q @ oracle.rope(k, n - m, THETA)
        assert abs(lhs - rhs) < 1e-10


def _rope_mp(x, p, theta, d):
    """(x_i + i x_{i+d/2}) * exp(i p theta^(-2i/d)) at 50 digits."""
    mpmath.mp.dps = 50
    half = d // 2
    out = [None] * d
    for i in range(half):
        a = mpmath.mpf(p) * mpmath.power(mpmath.mpf(theta),
                                         -mpmath.mpf(2 * i) / d)
        z = mpmath.mpc(mpmath.mpf(float(x[i])), mpmath.mpf(float(x[i + half])))
        z = z * mpmath.expj(a)
        out[i], out[i + half] = z.real, z.imag
    return np.array([float(v) for v in out])


@pytest.mark.parametrize("d,p", [(8, 3), (128, 0), (128, 7), (128, 2047),
                                 (128, 2175)])
def test_complex_twin(d, p):
    x = np.random.default_rng(d + p).standard_normal(d)
    assert np.allclose(oracle.rope(x, p, THETA), _rope_mp(x, p, THETA, d),
                       rtol=0, atol=1e-12)


def test_frequencies_closed_form():
    f = oracle.rope_inv_freq(128, THETA)
    assert f[0] == 1.0
    assert abs(f[32] - 1e-3) < 1e-18
    assert abs(f[16] - 10 ** -1.5) < 1e-17
    assert np.all(np.diff(f) < 0)
