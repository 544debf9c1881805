"""The rounding argument behind the hidden-state RMSNorm's fp32 path, checked
on the CPU with IEEE fp32 arithmetic (numpy).  The kernel forms
bf16(x + residual) from the fp32 sum, bf16(r / s) from r * fp32(1/s) unless
that quotient lies within 8 fp32 ulps of a bf16 rounding midpoint (then the
fp64 division decides), and bf16(w * y) from the fp32 product.  Each must
equal one round-to-nearest-even of the exact value, which is what the fp64
oracle computes.  The GPU kernel itself is checked bit for bit against the
oracle in tests/test_gpu_rmsnorm_hidden.py."""

import numpy as np


def rne_bf16_of_f64(x):
    """One round to nearest even of fp64 values to bf16 bits (normal range)."""
    u = x.view(np.uint64)
    r = (u + np.uint64(0x00000FFFFFFFFFFF) + ((u >> np.uint64(45)) & np.uint64(1))) & \
        ~np.uint64(0x00001FFFFFFFFFFF)
    return (r.view(np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(
        np.uint16)


def rne16(f):
    u = f.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >>
            np.uint32(16)).astype(np.uint16)


def bf(b):
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def off_range(f):
    e = (f.view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF)
    return (e < 9) | (e == 0xFF)


def fast_quotient(rv, s):
    """bf16(r / s) the way the kernel forms it; also whether it took fp64."""
    q = (rv * (1.0 / s).astype(np.float32)).astype(np.float32)
    lo = q.view(np.uint32) & np.uint32(0xFFFF)
    exact = (off_range(q) & (q != 0)) | ((lo > 0x8000 - 8) & (lo < 0x8000 + 8))
    want = rne_bf16_of_f64(rv.astype(np.float64) / s)
    return np.where(exact, want, rne16(q)), exact, want


def test_residual_sum_weight_product_and_quotient():
    rng = np.random.default_rng(7)
    for scale in (1e-30, 1e-3, 1.0, 7.5, 1e4, 1e30):
        n = 200_000
        x = rne16((rng.standard_normal(n) * scale).astype(np.float32))
        res = rne16((rng.standard_normal(n) * scale *
                     rng.choice([1e-6, 1.0, 1e6], n)).astype(np.float32))
        xf, rf = bf(x), bf(res)
        # the residual add: the fp32 sum rounded once equals the exact sum's rounding
        want_r = rne_bf16_of_f64(xf.astype(np.float64) + rf.astype(np.float64))
        sf = (xf + rf).astype(np.float32)
        fin = np.isfinite(sf)
        assert np.array_equal(rne16(sf)[fin], want_r[fin])
        # r / s through the fp32 path with the midpoint fallback
        rv = bf(want_r)
        s = (np.abs(rng.standard_normal()) * scale + 1e-3) * rng.uniform(0.5, 2.0, n)
        got, _, want = fast_quotient(rv, s)
        ok = np.isfinite(rv.astype(np.float64) / s) & \
            (np.abs(rv.astype(np.float64) / s) > 1e-37)
        assert np.array_equal(got[ok], want[ok])
        # the weight product: exact in fp32 in range
        w = rne16((rng.standard_normal(n) * 0.3 + 1.0).astype(np.float32))
        wf, yf = bf(w), bf(want)
        p = (wf * yf).astype(np.float32)
        want_o = rne_bf16_of_f64(wf.astype(np.float64) * yf.astype(np.float64))
        sel = np.isfinite(p) & ~(off_range(p) & (p != 0))
        assert np.array_equal(rne16(p)[sel], want_o[sel])


def test_quotients_near_midpoints_take_the_fp64_division():
    # exact quotients placed within 3e-7 of bf16 rounding midpoints: the fp32
    # quotient is then within 8 ulps of the midpoint, so every one of them
    # must go to the fp64 division, and the result is the exact rounding
    rng = np.random.default_rng(8)
    n = 200_000
    m = rng.integers(0x3F80, 0x4000, n).astype(np.uint32)
    mid = ((m << np.uint32(16)) | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    rv = np.abs(bf(rne16(rng.standard_normal(n).astype(np.float32))))
    rv = np.where(rv == 0, np.float32(1.0), rv)
    s = rv.astype(np.float64) / (mid * (1 + rng.uniform(-3e-7, 3e-7, n)))
    got, exact, want = fast_quotient(rv, s)
    assert exact.all()
    assert np.array_equal(got, want)


def test_planted_wrong_margin_is_caught():
    # with no fallback at all (margin 0), some near-midpoint quotients round
    # the wrong way: the margin is what makes the fp32 path exact
    rng = np.random.default_rng(9)
    n = 200_000
    m = rng.integers(0x3F80, 0x4000, n).astype(np.uint32)
    mid = ((m << np.uint32(16)) | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    rv = np.abs(bf(rne16(rng.standard_normal(n).astype(np.float32))))
    rv = np.where(rv == 0, np.float32(1.0), rv)
    s = rv.astype(np.float64) / (mid * (1 + rng.uniform(-3e-7, 3e-7, n)))
    q = (rv * (1.0 / s).astype(np.float32)).astype(np.float32)
    want = rne_bf16_of_f64(rv.astype(np.float64) / s)
    assert (rne16(q) != want).any()
