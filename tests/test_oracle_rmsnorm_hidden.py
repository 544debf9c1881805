"""Pins for the oracle's hidden-state RMSNorm (reference cast placement)."""

import numpy as np
import pytest
import torch

import oracle
from oracle.rmsnorm_hidden import rmsnorm_hidden


def _vec(s):
    return None if s == "-" else np.array([float(t) for t in s.split()])


def test_hand_values(golden):
    for name, xs, rs, eps, ws, exp, rexp in golden("rmsnorm_hidden_hand.txt"):
        out, r = rmsnorm_hidden(_vec(xs), _vec(ws), float(eps), _vec(rs))
        assert np.array_equal(out, _vec(exp)), name
        if rexp != "-":
            assert np.array_equal(r, _vec(rexp)), name


def test_constant_vector_closed_form():
    # r = c (a bf16 value): y = sign(c) / sqrt(1 + eps / c^2)
    for c in [2.0 ** -10, 0.375, -3.0, 96.0]:
        for eps in [0.0, 1e-6]:
            out, _ = rmsnorm_hidden(np.full(64, c), None, eps)
            y = np.sign(c) / np.sqrt(1.0 + eps / (c * c))
            assert np.all(out == torch.tensor(y, dtype=torch.float64)
                          .to(torch.bfloat16).double().item())


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_residual_sum_matches_torch_bf16_add():
    # the residual stream is a bf16 tensor: torch's own bf16 addition
    g = np.random.default_rng(11)
    x = _bf16(g.standard_normal((16, 256)) * 3)
    res = _bf16(g.standard_normal((16, 256)) * g.uniform(1e-4, 30, (16, 1)))
    _, r = rmsnorm_hidden(x.double().numpy(), None, 1e-6, res.double().numpy())
    assert np.array_equal(r, (x + res).double().numpy())


def test_matches_float32_reference_arithmetic():
    # The reference computes in float32 (mean of squares, rsqrt), casts to
    # bf16 and multiplies by the bf16 weight.  fp32 rounding moves a value
    # across a bf16 rounding boundary only rarely, and then by one unit.
    g = np.random.default_rng(12)
    H = 2560
    x = _bf16(g.standard_normal((64, H)) * g.uniform(0.05, 20, (64, 1)))
    res = _bf16(g.standard_normal((64, H)))
    w = _bf16(1.0 + 0.3 * g.standard_normal(H))
    h = (x + res).float()
    var = h.pow(2).mean(-1, keepdim=True)
    ref = (w * (h * torch.rsqrt(var + 1e-6)).to(torch.bfloat16)).double().numpy()
    out, _ = rmsnorm_hidden(x.double().numpy(), w.double().numpy(), 1e-6,
                            res.double().numpy())
    diff = out != ref
    assert diff.mean() < 2e-3
    # where they differ, by at most two bf16 units of the value
    ulp = np.exp2(np.floor(np.log2(np.abs(ref[diff]))) - 7)
    assert np.all(np.abs(out[diff] - ref[diff]) <= 2 * ulp)


def test_agrees_with_per_head_norm_before_the_casts():
    g = np.random.default_rng(13)
    x = g.standard_normal((8, 128))
    out, _ = rmsnorm_hidden(x, None, 1e-6)
    assert np.array_equal(out, oracle.bf16_round(oracle.rmsnorm(x, None, 1e-6)))


@pytest.mark.parametrize("mutant", ["weight_before_cast", "eps_outside", "residual_unrounded"])
def test_mutations_are_caught(golden, mutant):
    def wrong(x, weight=None, eps=1e-6, residual=None):
        x = np.asarray(x, dtype=np.float64)
        r = x if residual is None else x + np.asarray(residual)
        if mutant != "residual_unrounded" and residual is not None:
            r = oracle.bf16_round(r)
        ms = np.mean(r * r, axis=-1, keepdims=True)
        y = r / (np.sqrt(ms) + eps) if mutant == "eps_outside" else r / np.sqrt(ms + eps)
        w = 1.0 if weight is None else np.asarray(weight)
        if mutant == "weight_before_cast":
            return oracle.bf16_round(w * y), r
        return oracle.bf16_round(w * oracle.bf16_round(y)), r

    caught = False
    for name, xs, rs, eps, ws, exp, rexp in golden("rmsnorm_hidden_hand.txt"):
        out, r = wrong(_vec(xs), _vec(ws), float(eps), _vec(rs))
        if not np.array_equal(out, _vec(exp)) or (rexp != "-" and not np.array_equal(r, _vec(rexp))):
            caught = True
    assert caught, mutant
