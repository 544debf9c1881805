"""GPU parity of qa_rmsnorm_hidden (residual add + RMSNorm in the reference's
cast placement) vs the fp64 oracle: bit-exact output and residual bytes."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import bits, say

pytestmark = pytest.mark.gpu
EPS = 1e-6


def run(T, H, residual, weight, seed, scale=1.0):
    say(f"rmsnorm case: T={T} H={H} residual={residual} weight={weight} "
        f"seed={seed} scale={scale}")
    x = W.normal_bf16((T, H), seed, 0, 0, "hidden_x", std=scale)
    r = W.normal_bf16((T, H), seed, 0, 1, "hidden_res", std=scale) \
        if residual else None
    w = (W.normal_bf16((H,), seed, 0, 2, "norm_w", std=0.3) + 1.0).to(
        torch.bfloat16) if weight else None
    xg = x.cuda()
    rg = None if r is None else r.cuda()
    wg = None if w is None else w.cuda()
    out = qa.rmsnorm_hidden(xg, residual=rg, weight=wg, eps=EPS)
    torch.cuda.synchronize()
    ref, ref_r = oracle.rmsnorm_hidden(
        x.double().numpy(), None if w is None else w.double().numpy(), EPS,
        None if r is None else r.double().numpy())
    got = bits(out)
    want = oracle.bf16_bits(ref)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} output mismatches, first at {bad[:5]}"
    if r is not None:
        assert np.array_equal(bits(rg), oracle.bf16_bits(ref_r))
    else:
        assert np.array_equal(bits(xg), bits(x))  # x untouched


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("weight", [False, True])
def test_qwen3_4b_rows(residual, weight):
    # hidden 2560, the four prompts of the B=4 x 2048 workload's first 512
    # tokens each
    run(2048, 2560, residual, weight, seed=60)


# up to 512 rows run one workgroup per row, more run one wave per row
@pytest.mark.parametrize("T,H", [(1, 8), (3, 128), (7, 520), (65, 4096),
                                 (5, 8192), (512, 2560), (513, 2560), (600, 8192)])
def test_shapes(T, H):
    run(T, H, True, True, seed=61)


def test_wide_dynamic_range():
    # tiny and huge rows: the sum of squares and the roundings away from 1
    run(64, 2560, True, True, seed=62, scale=1e-18)
    run(64, 2560, True, True, seed=63, scale=1e17)


def test_zero_row_and_cancelling_residual():
    x = torch.zeros((2, 256), dtype=torch.bfloat16)
    x[1] = W.normal_bf16((256,), 64, 0, 0, "hidden_x")
    r = (-x).clone()
    r[0] = 0
    xg, rg = x.cuda(), r.cuda()
    out = qa.rmsnorm_hidden(xg, residual=rg, eps=EPS)
    torch.cuda.synchronize()
    # x + residual is exactly zero in both rows: the norm of a zero row is 0
    assert not bits(out).any() and not (bits(rg) & 0x7FFF).any()


def test_empty_call_and_fused_counter():
    x = torch.zeros((0, 2560), dtype=torch.bfloat16, device="cuda")
    before = qa.counters()
    qa.rmsnorm_hidden(x)
    assert qa.counters()[3] == before[3]
    y = torch.ones((4, 2560), dtype=torch.bfloat16, device="cuda")
    qa.rmsnorm_hidden(y)
    torch.cuda.synchronize()
    assert qa.counters()[3] == before[3] + 1
