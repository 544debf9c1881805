"""Pins for the oracle's bf16 rounding (round to nearest, ties to even)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _torch_bits_f32(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_matches_torch_on_fp32_inputs():
    # fp32 -> bf16 in torch is a single RNE, so on fp32-representable inputs the
    # two must agree bit for bit, including ties, subnormals, overflow, inf.
    g = np.random.default_rng(0)
    x = g.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    ties = (np.arange(-4096, 4096, dtype=np.int32) << 16 | 0x8000)
    ties = ties.astype(np.uint32).view(np.float32)
    sub = np.array([1e-40, -3e-41, 2**-133, 2**-134, 3 * 2**-135, 1e-45],
                   dtype=np.float32)
    big = np.array([3.389e38, 3.3895e38, 3.4e38, -3.4e38, np.inf, -np.inf,
                    0.0, -0.0], dtype=np.float32)
    allx = np.concatenate([x, ties[np.isfinite(ties)], sub, big])
    ours = oracle.bf16_bits(allx.astype(np.float64))
    ref = _torch_bits_f32(allx)
    assert np.array_equal(ours, ref)


def test_nan_is_quiet_nan():
    b = oracle.bf16_bits(np.array([np.nan]))
    assert (int(b[0]) & 0x7FFF) == 0x7FC0


def _bf16_value(bits):
    return Fraction(float(oracle.bits_to_f64(np.array([bits], np.uint16))[0]))


@pytest.mark.parametrize("seed", [1, 2])
def test_nearest_even_on_fp64_inputs(seed):
    # Direct fp64 -> bf16: compare with both neighbours in exact arithmetic.
    g = np.random.default_rng(seed)
    xs = g.standard_normal(3000) * np.exp2(g.integers(-20, 20, 3000))
    # exact midpoints between adjacent bf16 values (ties) and near-ties
    base = oracle.bits_to_f64(np.arange(0x3F00, 0x3F40, dtype=np.uint16))
    mids = (base[:-1] + base[1:]) / 2
    xs = np.concatenate([xs, mids, np.nextafter(mids, np.inf),
                         np.nextafter(mids, -np.inf)])
    bits = oracle.bf16_bits(xs)
    for x, b in zip(xs, bits):
        b = int(b)
        fx = Fraction(float(x))
        r = _bf16_value(b)
        mag = b & 0x7FFF
        sign = b & 0x8000
        up = _bf16_value(sign | (mag + 1))
        dn = _bf16_value(sign | (mag - 1)) if mag else -up
        dr, du, dd = abs(fx - r), abs(fx - up), abs(fx - dn)
        assert dr <= du and dr <= dd
        if dr == du or dr == dd:  # a tie: the chosen one has an even mantissa
            assert (b & 1) == 0


def test_widening_is_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    vals = oracle.bits_to_f64(bits)
    assert np.array_equal(oracle.bf16_bits(vals), bits)
