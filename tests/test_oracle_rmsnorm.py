"""Pins for the oracle's per-head RMSNorm (closed forms and hand values)."""

import numpy as np
import pytest

import oracle


def test_hand_values(golden):
    for name, xs, eps, w, exp in golden("rmsnorm_hand.txt"):
        x = np.array([float(t) for t in xs.split()])
        wv = None if w == "-" else np.array([float(t) for t in w.split()])
        y = oracle.rmsnorm(x, wv, float(eps))
        e = np.array([float(t) for t in exp.split()])
        assert np.allclose(y, e, rtol=0, atol=1e-15), name


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_output_rms_closed_form(eps):
    # With w = 1: RMS(y) = sqrt(ms / (ms + eps)) exactly in real arithmetic.
    g = np.random.default_rng(3)
    x = g.standard_normal((64, 128)) * g.uniform(0.01, 10, (64, 1))
    y = oracle.rmsnorm(x, None, eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)),
                       np.sqrt(ms / (ms + eps)), rtol=1e-14, atol=0)


def test_constant_vector():
    for c in [1e-4, 0.3, -2.0, 17.0]:
        x = np.full(128, c)
        y = oracle.rmsnorm(x, None, 1e-6)
        assert np.allclose(y, c / np.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)


def test_scale_invariance_without_eps():
    g = np.random.default_rng(4)
    x = g.standard_normal((8, 128))
    for a in [1e-3, 2.0, 1e3]:
        assert np.allclose(oracle.rmsnorm(a * x, None, 0.0),
                           oracle.rmsnorm(x, None, 0.0), rtol=1e-14, atol=0)


def test_weight_is_elementwise_after_norm():
    g = np.random.default_rng(5)
    x = g.standard_normal(128)
    w = g.standard_normal(128)
    assert np.allclose(oracle.rmsnorm(x, w, 1e-6),
                       oracle.rmsnorm(x, None, 1e-6) * w, rtol=1e-15, atol=0)
    # and not "normalise w*x"
    assert not np.allclose(oracle.rmsnorm(x, w, 1e-6),
                           oracle.rmsnorm(w * x, None, 1e-6))
