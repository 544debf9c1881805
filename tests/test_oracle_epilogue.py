"""Pins for the oracle's attention epilogue (output projection, residual add,
post-attention RMSNorm in the reference's cast placement)."""

from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle.epilogue import attn_epilogue, o_proj


def _vec(s):
    return None if s == "-" else np.array([float(t) for t in s.split()])


def _mat(s):
    return np.array([[float(t) for t in row.split()] for row in s.split(";")])


def test_hand_values(golden):
    for name, o, w, res, eps, wt, h, r, out in golden("epilogue_hand.txt"):
        got_out, got_r, got_h = attn_epilogue(_vec(o)[None], _mat(w), _vec(res)[None],
                                              _vec(wt), float(eps))
        assert np.array_equal(got_h[0], _vec(h)), name
        assert np.array_equal(got_r[0], _vec(r)), name
        assert np.array_equal(got_out[0], _vec(out)), name


def _bf16_draws(g, shape, scale=1.0):
    x = torch.from_numpy((g.standard_normal(shape) * scale).astype(np.float32))
    return x.to(torch.bfloat16).double().numpy()


def test_projection_equals_exact_rational_sum():
    # every output: the exact rational sum of the products, rounded once
    g = np.random.default_rng(21)
    o = _bf16_draws(g, (3, 24))
    w = _bf16_draws(g, (5, 24), 0.05)
    h = o_proj(o, w)
    for t in range(3):
        for n in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(o[t], w[n]))
            assert h[t, n] == oracle.bf16_round(float(exact)), (t, n)


def test_identity_and_zero_weights():
    g = np.random.default_rng(22)
    o = _bf16_draws(g, (4, 16))
    res = _bf16_draws(g, (4, 16))
    _, _, h = attn_epilogue(o, np.eye(16), res)
    assert np.array_equal(h, o)  # bf16 inputs pass through the projection unchanged
    out, r, h = attn_epilogue(o, np.zeros((16, 16)), res)
    assert np.array_equal(h, np.zeros((4, 16)))
    assert np.array_equal(r, res)
    ref, _ = oracle.rmsnorm_hidden(res, None, 1e-6)
    assert np.array_equal(out, ref)


def test_matches_torch_bf16_linear_layer():
    # the reference's linear layer in bf16 (fp32 sums, one rounding): equal
    # except where the fp32 sum falls on the other side of a bf16 rounding
    # boundary, then by one unit
    g = np.random.default_rng(23)
    o = torch.from_numpy(g.standard_normal((64, 512)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((g.standard_normal((256, 512)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    ref = torch.nn.functional.linear(o, w).double().numpy()
    h = o_proj(o.double().numpy(), w.double().numpy())
    diff = h != ref
    assert diff.mean() < 0.005, diff.mean()
    ulp = np.exp2(np.floor(np.log2(np.abs(h[diff]))) - 7)
    assert np.all(np.abs(h[diff] - ref[diff]) <= ulp * 1.0001)


def test_residual_stream_is_the_bf16_sum():
    g = np.random.default_rng(24)
    o = _bf16_draws(g, (8, 32))
    w = _bf16_draws(g, (48, 32), 0.1)
    res = _bf16_draws(g, (8, 48), 3.0)
    _, r, h = attn_epilogue(o, w, res)
    assert np.array_equal(r, (torch.from_numpy(res).to(torch.bfloat16) +
                              torch.from_numpy(h).to(torch.bfloat16)).double().numpy())
