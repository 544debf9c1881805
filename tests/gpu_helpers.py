"""Shared pieces of the GPU parity tests (HIP path through the C ABI vs the
fp64 oracle on the same seeded inputs)."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import workloads as W
from prefill_attention_rmsnorm_amd import qa

THETA = 1.0e6
EPS = 1.0e-6
NAN_BITS = 0x7FC1

# Tolerance of the attention output ("max-abs 1e-2, max-rel 2e-2"; the
# relative error is taken per (token, head) row against that row's largest
# reference magnitude, since element-wise relative error is unbounded near 0).
ATOL = 1e-2
RREL = 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(
        np.uint16)


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (the largest error of rounding x to bf16)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.exp2(e - 8)


def compare(gpu, ref, what, atol=ATOL, rrel=RREL, mask=None, out_bf16=True):
    """Check the tolerance and report error statistics.

    max-abs: the largest |gpu - ref| beyond the rounding of the exact value to
    the bf16 output format (half an ulp of ref), which alone exceeds 1e-2 for
    |ref| >= 4.  max-rel: per (token, head) row, max|gpu - ref| over
    max|ref|.  Both must hold.  Pass rrel=inf for quantities compared on an
    absolute scale only (the log-sum-exp, which can sit near zero).
    """
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        gpu, ref = gpu[mask], ref[mask]
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    d = np.abs(gpu - ref)
    excess = np.maximum(d - bf16_half_ulp(ref), 0.0) if out_bf16 else d
    rows_ref = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    rows_d = d.reshape(-1, ref.shape[-1]).max(axis=1)
    row_rel = float((rows_d / np.maximum(rows_ref, 1e-30)).max()) \
        if rows_d.size else 0.0
    st = dict(max_abs=float(d.max()) if d.size else 0.0,
              max_abs_beyond_rounding=float(excess.max()) if d.size else 0.0,
              mean_abs=float(d.mean()) if d.size else 0.0,
              p99_abs=float(np.percentile(d, 99)) if d.size else 0.0,
              max_row_rel=row_rel, n_over_atol=int((excess > atol).sum()),
              n=int(d.size))
    say(f"  {what}: {st}")
    assert st["max_abs_beyond_rounding"] <= atol and row_rel <= rrel, \
        f"{what}: {st}"
    return st


def params(Hq, head_dim=128, q_w=None, k_w=None):
    return qa.Params(Hq, 1.0 / math.sqrt(head_dim), THETA, EPS, q_w, k_w)


def new_cache(B, Hkv, cap):
    return qa.Cache.empty(B, Hkv, cap, fill_bits=NAN_BITS)


def prefix_fill(cache: qa.Cache, ocache: oracle.Cache, starts, seed):
    """Slots [0, start_b) of row b hold seeded bf16 ~N(0,1) K and V, in both
    caches (as if written by earlier calls)."""
    B, Hkv, cap, d = cache.k.shape
    for b, s in enumerate(starts):
        if s <= 0:
            continue
        kk = W.normal_bf16((Hkv, s, d), seed, b, 0, "cache_k")
        vv = W.normal_bf16((Hkv, s, d), seed, b, 0, "cache_v")
        cache.k[b, :, :s] = kk.cuda()
        cache.v[b, :, :s] = vv.cuda()
        ocache.k[b, :, :s] = kk.double().numpy()
        ocache.v[b, :, :s] = vv.double().numpy()


def check_cache(cache: qa.Cache, ocache: oracle.Cache, what="cache"):
    """K and V bytes equal the oracle's (RNE of k', raw v); unwritten slots
    keep the NaN sentinel."""
    kb, vb = bits(cache.k), bits(cache.v)
    written = ~np.isnan(ocache.k[..., 0])
    ok_k = oracle.bf16_bits(ocache.k[written])
    ok_v = oracle.bf16_bits(ocache.v[written])
    mism_k = np.argwhere(kb[written] != ok_k)
    mism_v = np.argwhere(vb[written] != ok_v)
    say(f"  {what}: {int(written.sum())} written slots, "
        f"K mismatches {len(mism_k)}, V mismatches {len(mism_v)}")
    assert len(mism_k) == 0, f"K bytes differ at {mism_k[:5].tolist()}"
    assert len(mism_v) == 0, f"V bytes differ at {mism_v[:5].tolist()}"
    assert (kb[~written] == NAN_BITS).all() and (vb[~written] == NAN_BITS).all(), \
        "an unwritten slot was modified"


def seq_index(lens):
    return np.repeat(np.arange(len(lens)), lens)


class LMHead:
    """Test-side LM head over the attention output (W_o [Hq*128, hidden], a
    final RMSNorm, W_lm [hidden, vocab], all random-init ~N(0, 0.02)): an fp32
    torch version on the GPU for the engine and the fp64 oracle version for
    the replay."""

    def __init__(self, widx, n_q_heads, hidden, vocab):
        say(f"LM head: W_o [{n_q_heads * 128}, {hidden}], W_lm [{hidden}, {vocab}]")
        self.w_o = W.normal_bf16((n_q_heads * 128, hidden), widx, 0, 0, "w_o",
                                 std=0.02)
        self.w_lm = W.normal_bf16((hidden, vocab), widx, 0, 0, "w_lm",
                                  std=0.02)
        self.w_o_np = self.w_o.double().numpy()
        self.w_lm_np = self.w_lm.float().numpy()
        self.w_o_gpu = self.w_o.float().cuda()
        self.w_lm_gpu = self.w_lm.float().cuda()

    def gpu_logits(self, o_gpu):
        """Engine side: the fp32 LM head on the GPU attention output."""
        h = o_gpu.reshape(o_gpu.shape[0], -1).float() @ self.w_o_gpu
        h = h * torch.rsqrt(h.pow(2).mean(-1, keepdim=True) + EPS)
        return h @ self.w_lm_gpu

    def gpu_tokens(self, o_gpu):
        """Engine side: argmax of the fp32 LM head on the GPU output."""
        return self.gpu_logits(o_gpu).argmax(-1).cpu().numpy()

    def ref_logits(self, o_ref):
        return oracle.lm_logits(o_ref.reshape(o_ref.shape[0], -1), self.w_o_np,
                                self.w_lm_np, EPS)
