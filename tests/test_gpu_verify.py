"""GPU parity of qa_verify (draft block vs cache + block) vs the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import (EPS, THETA, check_cache, compare, f64, new_cache,
                          params, prefix_fill, say)

pytestmark = pytest.mark.gpu
SCALE = 1.0 / np.sqrt(128)


def run_verify(B, Hq, Hkv, cap, starts, n, seed, max_ctx=None):
    say(f"verify case: B={B} Hq={Hq} Hkv={Hkv} cap={cap} starts={starts} "
        f"n={n} seed={seed}")
    cache = new_cache(B, Hkv, cap)
    oc = oracle.Cache.empty(B, Hkv, cap, 128)
    prefix_fill(cache, oc, starts, seed)
    q = W.normal_bf16((B, n, Hq, 128), seed, 2, 0, "q")
    k = W.normal_bf16((B, n, Hkv, 128), seed, 2, 0, "k")
    v = W.normal_bf16((B, n, Hkv, 128), seed, 2, 0, "v")
    max_ctx = max_ctx or cap
    lse = torch.empty((B, n, Hq), device="cuda")
    start_t = torch.tensor(starts, dtype=torch.int32, device="cuda")
    out, _, ws = qa.verify(cache, params(Hq), q.cuda(), k.cuda(), v.cuda(),
                           start_t, max_ctx, lse=lse)
    assert qa.device_error(ws) == 0
    ref, ref_lse, oc2 = oracle.verify(oc, q.double().numpy(),
                                      k.double().numpy(), v.double().numpy(),
                                      starts, scale=SCALE, theta=THETA,
                                      eps=EPS)
    st = compare(f64(out), ref, "verify out")
    compare(f64(lse)[..., None], ref_lse[..., None], "verify lse", atol=1e-2,
            rrel=float("inf"), out_bf16=False)
    check_cache(cache, oc2)
    return out, cache, st


def test_config4_shape():
    w = W.get(4)
    run_verify(w.batch, w.n_q_heads, w.n_kv_heads, w.capacity,
               [w.verify_start] * w.batch, w.verify_block, seed=40)


def test_ragged_starts_and_split_boundaries():
    # starts chosen so the block straddles 64-key tiles and split edges
    run_verify(4, 32, 8, 1200, [0, 63, 500, 1180], 16, seed=41)


# (8, 8, 48) and (16, 8, 40): blocks past 32 tokens take the double-buffered
# pass without the ring, on 2 waves (48 rows) and on 4 waves (80 rows)
@pytest.mark.parametrize("Hq,Hkv,n", [(8, 8, 1), (8, 4, 3), (16, 2, 16),
                                      (4, 1, 32), (8, 8, 48), (16, 8, 40)])
def test_shapes(Hq, Hkv, n):
    run_verify(2, Hq, Hkv, 300, [100, 7], n, seed=42)


def test_one_sequence_many_splits():
    # 8 (sequence, kv head) pairs: 31 old-slot splits plus the block's own,
    # merged by the merge kernel in two batches of 16 splits
    run_verify(1, 32, 8, 2064, [2048], 16, seed=44)


def test_large_batch_one_old_split():
    # 32 sequences x 8 kv heads: 256 pairs, one old-slot split per pair (plus
    # the block's own workgroup); starts from 0 (no old slots) upward
    g = np.random.default_rng(43)
    starts = [0, 1, 63, 64] + [int(x) for x in g.integers(0, 300, 28)]
    run_verify(32, 32, 8, 320, starts, 8, seed=43)


def test_verify_equals_sequential_decodes():
    B, Hq, Hkv, cap, n, L = 2, 32, 8, 600, 16, 500
    cache_v = new_cache(B, Hkv, cap)
    cache_d = new_cache(B, Hkv, cap)
    oc = oracle.Cache.empty(B, Hkv, cap, 128)
    prefix_fill(cache_v, oc, [L, L], 43)
    prefix_fill(cache_d, oracle.Cache.empty(B, Hkv, cap, 128), [L, L], 43)
    q = W.normal_bf16((B, n, Hq, 128), 43, 2, 0, "q").cuda()
    k = W.normal_bf16((B, n, Hkv, 128), 43, 2, 0, "k").cuda()
    v = W.normal_bf16((B, n, Hkv, 128), 43, 2, 0, "v").cuda()
    p = params(Hq)
    outv, _, _ = qa.verify(cache_v, p, q, k, v,
                           torch.full((B,), L, dtype=torch.int32,
                                      device="cuda"), cap)
    ws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)
    for i in range(n):
        od, _, _ = qa.decode(cache_d, p, q[:, i].contiguous(),
                             k[:, i].contiguous(), v[:, i].contiguous(),
                             torch.full((B,), L + i, dtype=torch.int32,
                                        device="cuda"), cap, ws=ws)
        d = np.abs(f64(od) - f64(outv[:, i])).max()
        assert d < 1e-2, (i, d)
    assert torch.equal(cache_v.k.view(torch.int16), cache_d.k.view(torch.int16))
    assert torch.equal(cache_v.v.view(torch.int16), cache_d.v.view(torch.int16))


def test_invalid_start_flags_and_zeroes():
    B, Hq, Hkv, cap, n = 2, 8, 2, 64, 4
    cache = new_cache(B, Hkv, cap)
    oc = oracle.Cache.empty(B, Hkv, cap, 128)
    prefix_fill(cache, oc, [10, 10], 44)
    q = W.normal_bf16((B, n, Hq, 128), 44, 2, 0, "q").cuda()
    k = W.normal_bf16((B, n, Hkv, 128), 44, 2, 0, "k").cuda()
    v = W.normal_bf16((B, n, Hkv, 128), 44, 2, 0, "v").cuda()
    start = torch.tensor([10, 62], dtype=torch.int32, device="cuda")
    out, _, ws = qa.verify(cache, params(Hq), q, k, v, start, cap)
    assert qa.device_error(ws) & qa.QA_DEVERR_POSITION
    assert torch.count_nonzero(out[1].float()) == 0
    assert torch.isfinite(out[0].float()).all()
