"""GPU parity when later keys score far above the first tile.

The attention kernels fix each workgroup's reference max from the first key
tile and redo the block with the exact row max when a later score overflows
that reference.  These cases force that path: with a huge rotary base the
rotation is negligible except on pairs 0 and 1, so keys can be aimed exactly.
Keys at positions below 64 point opposite the queries (score about -261 in
log2 units with norm weights of 4), later keys along them (+261).  The exact
softmax then averages V over the visible aligned keys with equal weights,
which both sides compute exactly up to rounding.

The oracle keeps q' unrounded while the kernels round q' * scale * log2(e)
to bf16 for the MFMA (the reading of the q-side rounding), a relative error
of at most 2^-8 per element.  Every score then moves by at most
2^-8 * scale * sum_i |q'_i| |k_i|, and the log-sum-exp, being 1-Lipschitz in
the largest score change, by at most the largest such bound over the visible
keys; the kernels' row sums of bf16-rounded probabilities add at most 2^-8
more in ln l.  At |score| ~ 261 (log2) the first term is ~0.7, so the LSE is
compared per row against that bound (lse_bound) rather than at 1e-2.  The
outputs do not depend on it: every visible aligned key has the same score.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import EPS, check_cache, compare, f64, new_cache, say

pytestmark = pytest.mark.gpu
SCALE = 1.0 / np.sqrt(128)
THETA_HUGE = 1e300
FLIP = 64  # keys at positions >= FLIP point along the queries


def _direction():
    x = np.ones(128)
    x[[0, 1, 64, 65]] = 0.0  # pairs 0 and 1 still turn under a huge base
    return x


def _keys(positions, Hkv):
    x = _direction()
    sign = np.where(np.asarray(positions) >= FLIP, 1.0, -1.0)
    return np.broadcast_to(sign[:, None, None] * x, (len(sign), Hkv, 128)).copy()


def _weights():
    return torch.full((128,), 4.0, dtype=torch.bfloat16)


def lse_bound(qp, Kc, pos, G):
    """Per (token, head) row: the largest change of the natural-log LSE that
    the bf16 rounding of the scaled q' can cause (see the module docstring),
    plus 2^-7 for the rounded row sum and fp32 noise.  qp [T, Hq, d] oracle
    q', Kc [Hkv, cap, d] the cache row, pos [T] positions."""
    T, Hq, _ = qp.shape
    out = np.empty((T, Hq))
    for t in range(T):
        for h in range(Hq):
            kk = np.abs(Kc[h // G, :pos[t] + 1])
            out[t, h] = 2.0 ** -8 * SCALE * (kk @ np.abs(qp[t, h])).max()
    return out + 2.0 ** -7


def _params(Hq, w):
    return qa.Params(Hq, SCALE, THETA_HUGE, EPS, w.cuda(), w.cuda())


def test_prefill_later_keys_far_above_first_tile():
    S, Hq, Hkv, cap = 320, 8, 2, 384
    say(f"score-range prefill: S={S} Hq={Hq} Hkv={Hkv}")
    pos = np.arange(S, dtype=np.int32)
    q = torch.from_numpy(np.broadcast_to(_direction(), (S, Hq, 128)).copy()).to(torch.bfloat16)
    k = torch.from_numpy(_keys(pos, Hkv)).to(torch.bfloat16)
    v = W.normal_bf16((S, Hkv, 128), 70, 0, 0, "v")
    w = _weights()
    cache = new_cache(1, Hkv, cap)
    lse = torch.full((S, Hq), float("nan"), device="cuda")
    cu = torch.tensor([0, S], dtype=torch.int32, device="cuda")
    out, lse, ws = qa.prefill(cache, _params(Hq, w), q.cuda(), k.cuda(), v.cuda(),
                              cu, torch.from_numpy(pos).cuda(), S, lse=lse)
    assert qa.device_error(ws) == 0
    oc = oracle.Cache.empty(1, Hkv, cap, 128)
    wd = w.double().numpy()
    ref, ref_lse, oc = oracle.prefill(oc, q.double().numpy(), k.double().numpy(),
                                      v.double().numpy(), [0, S], pos, scale=SCALE,
                                      theta=THETA_HUGE, eps=EPS, q_w=wd, k_w=wd)
    check_cache(cache, oc)
    got = f64(out)
    compare(got, ref, "prefill out, large score range")
    qp = oracle.rope(oracle.rmsnorm(q.double().numpy(), wd, EPS), pos[:, None],
                     THETA_HUGE)
    bound = lse_bound(qp, oc.k[0], pos, Hq // Hkv)
    d = np.abs(f64(lse) - ref_lse)
    say(f"  prefill lse: max |d| {d.max():.4f}, smallest bound {bound.min():.4f}, "
        f"largest d / bound {(d / bound).max():.3f}")
    assert (d <= bound).all()
    # closed form: token t >= FLIP averages V over slots FLIP .. t
    vv = v.double().numpy()
    for t in (FLIP, 100, S - 1):
        mean = vv[FLIP:t + 1].mean(axis=0)  # [Hkv, d]
        exp = np.repeat(mean, Hq // Hkv, axis=0)
        assert np.abs(got[t] - exp).max() < 2e-2, t


def test_verify_later_keys_far_above_first_tile():
    B, Hq, Hkv, cap, start, n = 2, 8, 2, 400, 300, 8
    say(f"score-range verify: B={B} start={start} n={n}")
    w = _weights()
    p = _params(Hq, w)
    wd = w.double().numpy()
    cache = new_cache(B, Hkv, cap)
    oc = oracle.Cache.empty(B, Hkv, cap, 128)
    # prefix 0 .. start-1 written by a prefill of the aimed keys
    pos = np.tile(np.arange(start, dtype=np.int32), B)
    T = B * start
    qp = torch.from_numpy(np.broadcast_to(_direction(), (T, Hq, 128)).copy()).to(torch.bfloat16)
    kp = torch.from_numpy(_keys(pos, Hkv)).to(torch.bfloat16)
    vp = W.normal_bf16((T, Hkv, 128), 71, 0, 0, "v")
    cu = np.arange(0, T + 1, start, dtype=np.int32)
    qa.prefill(cache, p, qp.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(cu).cuda(),
               torch.from_numpy(pos).cuda(), start)
    _, _, oc = oracle.prefill(oc, qp.double().numpy(), kp.double().numpy(),
                              vp.double().numpy(), cu, pos, scale=SCALE,
                              theta=THETA_HUGE, eps=EPS, q_w=wd, k_w=wd)
    qv = torch.from_numpy(np.broadcast_to(_direction(), (B, n, Hq, 128)).copy()).to(torch.bfloat16)
    kv = torch.from_numpy(_keys(np.full(B * n, start), Hkv).reshape(B, n, Hkv, 128)).to(torch.bfloat16)
    vv = W.normal_bf16((B, n, Hkv, 128), 72, 0, 0, "v")
    lse = torch.full((B, n, Hq), float("nan"), device="cuda")
    starts = [start] * B
    out, _, ws = qa.verify(cache, p, qv.cuda(), kv.cuda(), vv.cuda(),
                           torch.tensor(starts, dtype=torch.int32, device="cuda"),
                           cap, lse=lse)
    assert qa.device_error(ws) == 0
    ref, ref_lse, oc2 = oracle.verify(oc, qv.double().numpy(), kv.double().numpy(),
                                      vv.double().numpy(), starts, scale=SCALE,
                                      theta=THETA_HUGE, eps=EPS, q_w=wd, k_w=wd)
    compare(f64(out), ref, "verify out, large score range")
    vpos = start + np.arange(n)
    for b in range(B):
        qp = oracle.rope(oracle.rmsnorm(qv[b].double().numpy(), wd, EPS),
                         vpos[:, None], THETA_HUGE)
        bound = lse_bound(qp, oc2.k[b], vpos, Hq // Hkv)
        d = np.abs(f64(lse[b]) - ref_lse[b])
        say(f"  verify lse seq {b}: max |d| {d.max():.4f}, largest d / bound "
            f"{(d / bound).max():.3f}")
        assert (d <= bound).all()
    check_cache(cache, oc2)
