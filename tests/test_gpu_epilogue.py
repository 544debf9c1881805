"""GPU parity of qa_attn_epilogue (output projection GEMM with the residual
add, then the post-attention RMSNorm) against the oracle's attn_epilogue.

Tolerance (derived from the arithmetic, the pages fix none for this step):
the GPU sums the projection h in fp32 and the oracle in fp64; both round the
sum once to bf16, so their h differ only where the fp32 sum lands on the
other side of a bf16 rounding boundary, by one unit of h.  The residual add
then differs by at most that unit plus one unit of the new residual's own
rounding (where the projection cancels the residual, a unit of h can be far
larger than a unit of the result).  The norm divides by the row's RMS and
multiplies by the weight, so the output may differ by that unit of h carried
through (|w| ulp(h) / rms) plus three of its own units (the roundings the
shift can move).  The share of elements that differ at all is small and is
reported and bounded.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import EPS, bits, f64, say

pytestmark = pytest.mark.gpu


def _ulp(x):
    ax = np.abs(np.asarray(x, dtype=np.float64))
    return np.exp2(np.floor(np.log2(np.maximum(ax, 2.0 ** -126))) - 7)


def _check(got, ref, allowed, what, max_frac):
    d = np.abs(got - ref)
    frac = float((d > 0).mean())
    ratio = d / allowed
    say(f"  {what}: max |d| {d.max():.3e}, max |d| / allowed {ratio.max():.3f}, "
        f"max {float((d / _ulp(ref)).max()):.1f} units of the result, "
        f"differing {frac:.2e} of {d.size}")
    assert np.isfinite(got).all()
    assert ratio.max() <= 1.0 + 1e-9, (what, ratio.max())
    assert frac <= max_frac, (what, frac)


def run_epilogue(T, in_dim, hidden, seed, weight=True, o_pad=0, o=None):
    say(f"epilogue case: T={T} in_dim={in_dim} hidden={hidden} seed={seed} "
        f"weight={weight} o_pad={o_pad}")
    if o is None:
        o = W.normal_bf16((T, in_dim + o_pad), seed, 0, 0, "q")
    w_o = W.normal_bf16((hidden, in_dim), seed, 0, 0, "w_o", std=0.02)
    res = W.normal_bf16((T, hidden), seed, 0, 0, "hidden_res")
    nw = (W.normal_bf16((hidden,), seed, 0, 0, "norm_w", std=0.1) + 1.0).to(
        torch.bfloat16) if weight else None
    og = o.cuda()[:, :in_dim]
    rg = res.cuda()
    out = qa.attn_epilogue(og, w_o.cuda(), rg, None if nw is None else nw.cuda(), EPS)
    torch.cuda.synchronize()
    wd = None if nw is None else nw.double().numpy()
    ref_out, ref_r, ref_h = oracle.attn_epilogue(
        o[:, :in_dim].double().numpy(), w_o.double().numpy(), res.double().numpy(),
        wd, EPS)
    _check(f64(rg), ref_r, _ulp(ref_r) + _ulp(ref_h), "residual", 1e-3)
    rms = np.sqrt(np.mean(ref_r * ref_r, axis=1, keepdims=True) + EPS)
    wabs = 1.0 if wd is None else np.abs(wd)[None, :]
    _check(f64(out), ref_out, 3 * _ulp(ref_out) + wabs * _ulp(ref_h) / rms, "out", 1e-2)
    return out, rg


def test_qwen3_b4_s2048_layer():
    # the B=4 x 2048 prefill layer's epilogue: 8192 tokens, 32 x 128 -> 2560
    run_epilogue(8192, 4096, 2560, seed=50)


def test_decode_rows_and_ragged_tail():
    run_epilogue(4, 4096, 2560, seed=51)
    run_epilogue(300, 512, 2560, seed=52, weight=False, o_pad=64)


def test_streaming_path_token_tiles():
    """Up to 32 tokens run the streaming kernel: one and two token tiles of 16,
    a ragged second tile, the largest batch it takes, and every width of K it
    has a variant for; 33 tokens go back to the GEMM."""
    run_epilogue(17, 4096, 2560, seed=56)
    run_epilogue(32, 4096, 2560, seed=57, o_pad=128)
    run_epilogue(16, 2048, 1024, seed=58, weight=False)
    run_epilogue(3, 8192, 512, seed=59)
    run_epilogue(5, 512, 256, seed=60)
    run_epilogue(33, 4096, 2560, seed=61)


def test_streaming_path_feature_split():
    """The streaming kernel's output features per workgroup follow the width:
    11 for 2688 (245 workgroups, the last holding 4 features) and the cap of
    16 for 4096."""
    run_epilogue(4, 1024, 2688, seed=62)
    run_epilogue(2, 512, 4096, seed=63, weight=False)


def test_other_widths():
    run_epilogue(130, 1024, 4096, seed=53)
    run_epilogue(1, 64, 128, seed=54)


def test_after_prefill_attention_output():
    # end to end: the tiny workload's prefill output feeds the epilogue
    w = W.get("tiny")
    S, Hq, Hkv = w.prompt_lens[0], w.n_q_heads, w.n_kv_heads
    q = W.normal_bf16((S, Hq, 128), 55, 0, 0, "q").cuda()
    k = W.normal_bf16((S, Hkv, 128), 55, 0, 0, "k").cuda()
    v = W.normal_bf16((S, Hkv, 128), 55, 0, 0, "v").cuda()
    cache = qa.Cache.empty(1, Hkv, S)
    cu, pos = W.packed_layout([S])
    p = qa.Params(Hq, w.scale, w.theta, w.eps)
    att, _, _ = qa.prefill(cache, p, q, k, v, torch.from_numpy(cu).cuda(),
                           torch.from_numpy(pos).cuda(), S)
    run_epilogue(S, Hq * 128, w.hidden, seed=55, o=att.reshape(S, -1).cpu())


def test_empty_call_is_noop():
    o = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    w_o = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    res = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    out = qa.attn_epilogue(o, w_o, res)
    assert out.shape == (0, 128)
