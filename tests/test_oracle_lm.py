"""Pins for the oracle's greedy check (LM head and the 2.0-logit rule)."""

import mpmath
import numpy as np

import oracle


def test_lm_logits_brute_force():
    g = np.random.default_rng(0)
    n, D, H, V = 2, 6, 4, 7
    o = g.standard_normal((n, D))
    Wo = g.standard_normal((D, H)) * 0.5
    Wl = g.standard_normal((H, V))
    got = oracle.lm_logits(o, Wo, Wl, 1e-6, chunk=3)
    mpmath.mp.dps = 40
    for r in range(n):
        h = [sum(mpmath.mpf(float(o[r, i])) * mpmath.mpf(float(Wo[i, j]))
                 for i in range(D)) for j in range(H)]
        rms = mpmath.sqrt(sum(x * x for x in h) / H + mpmath.mpf(1e-6))
        h = [x / rms for x in h]
        for c in range(V):
            ref = sum(h[j] * mpmath.mpf(float(Wl[j, c])) for j in range(H))
            assert abs(got[r, c] - float(ref)) < 1e-13


def test_margin_rule():
    logits = np.array([0.0, 5.0, 3.0, 3.0000001, 5.0])
    assert oracle.margin_ok(logits, 1) and oracle.margin_ok(logits, 4)
    assert oracle.margin_ok(logits, 2)        # exactly 2.0 below: passes
    assert oracle.margin_ok(logits, 3)
    assert not oracle.margin_ok(logits, 0)
    assert not oracle.margin_ok(np.array([0.0, 2.0000001]), 0)
    assert oracle.argmax_lowest(logits) == 1  # tie -> lowest id
