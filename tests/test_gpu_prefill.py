"""GPU parity of qa_prefill (prologue + MFMA flash attention) vs the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import (EPS, THETA, check_cache, compare, f64, new_cache,
                          params, prefix_fill, say, seq_index)

pytestmark = pytest.mark.gpu


def run_prefill(lens, Hq, Hkv, cap, *, seed, starts=None, batch=None,
                weights=False, fused_qkv=False, rows=None, with_lse=True):
    B = batch or len(lens)
    T = int(sum(lens))
    starts = starts or [0] * len(lens)
    say(f"prefill case: lens={list(lens)} starts={starts} Hq={Hq} Hkv={Hkv} "
        f"cap={cap} seed={seed} weights={weights} fused={fused_qkv}")
    q = W.normal_bf16((T, Hq, 128), seed, 0, 0, "q")
    k = W.normal_bf16((T, Hkv, 128), seed, 0, 0, "k")
    v = W.normal_bf16((T, Hkv, 128), seed, 0, 0, "v")
    q_w = k_w = None
    if weights:
        q_w = W.normal_bf16((128,), seed, 0, 0, "norm_w", std=0.3) + 1.0
        k_w = W.normal_bf16((128,), seed, 0, 1, "norm_w", std=0.3) + 1.0
        q_w, k_w = q_w.to(torch.bfloat16), k_w.to(torch.bfloat16)
    cu, pos = W.packed_layout(lens, starts)

    cache = new_cache(B, Hkv, cap)
    ocache = oracle.Cache.empty(B, Hkv, cap, 128)
    prefix_fill(cache, ocache, starts, seed)

    if fused_qkv:
        qkv = torch.cat([q, k, v], dim=1).cuda()  # [T, Hq+2Hkv, 128]
        qg, kg, vg = qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]
    else:
        qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    p = params(Hq, q_w=None if q_w is None else q_w.cuda(),
               k_w=None if k_w is None else k_w.cuda())
    lse = torch.full((T, Hq), float("nan"), device="cuda") if with_lse else None
    cu_t = torch.from_numpy(cu).cuda()
    pos_t = torch.from_numpy(pos).cuda()
    out, lse, ws = qa.prefill(cache, p, qg, kg, vg, cu_t, pos_t, max(lens),
                              lse=lse)
    assert qa.device_error(ws) == 0
    torch.cuda.synchronize()

    qw = None if q_w is None else q_w.double().numpy()
    kw = None if k_w is None else k_w.double().numpy()
    seq = seq_index(lens)
    oc = oracle.write_kv(ocache, k.double().numpy(), v.double().numpy(), seq,
                         pos, theta=THETA, eps=EPS, k_w=kw)
    ref, ref_lse = oracle.attend_tokens(oc, q.double().numpy(), seq, pos,
                                        scale=1 / np.sqrt(128), theta=THETA,
                                        eps=EPS, q_w=qw, rows=rows)
    check_cache(cache, oc)
    got = f64(out)
    if rows is None:
        st = compare(got, ref, "prefill out")
        if with_lse:
            compare(f64(lse)[..., None], ref_lse[..., None], "prefill lse",
                    atol=1e-2, rrel=float("inf"), out_bf16=False)
    else:
        tt = np.array([r[0] for r in rows])
        hh = np.array([r[1] for r in rows])
        st = compare(got[tt, hh], ref[tt, hh], "prefill out (sampled rows)")
        if with_lse:
            compare(f64(lse)[tt, hh][:, None], ref_lse[tt, hh][:, None],
                    "prefill lse (sampled)", atol=1e-2, rrel=float("inf"), out_bf16=False)
    return out, cache, st


def test_tiny_config():
    w = W.get("tiny")
    run_prefill(list(w.prompt_lens), w.n_q_heads, w.n_kv_heads, w.capacity,
                seed=0)


def test_qwen3_b1_s512():
    w = W.get(1)
    run_prefill(list(w.prompt_lens), w.n_q_heads, w.n_kv_heads, w.capacity,
                seed=1)


def test_ragged_tails_small():
    # single-token sequence, partial tiles, a sequence shorter than a tile
    run_prefill([1, 37, 130, 64], 8, 2, 160, seed=2)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (8, 1), (16, 2)])
def test_gqa_groups(Hq, Hkv):
    run_prefill([50, 100, 3], Hq, Hkv, 128, seed=3)


def test_chunked_prefill_after_prefix():
    run_prefill([40, 70], 8, 2, 192, seed=4, starts=[64, 10])


def test_norm_weights_and_fused_qkv_strides():
    run_prefill([33, 65], 8, 2, 96, seed=5, weights=True, fused_qkv=True)


def test_fewer_sequences_than_cache_rows():
    run_prefill([20, 9], 4, 1, 32, seed=6, batch=4)


def test_deterministic_rerun():
    lens, Hq, Hkv, cap = [300, 129], 8, 2, 320
    T = sum(lens)
    q = W.normal_bf16((T, Hq, 128), 7, 0, 0, "q").cuda()
    k = W.normal_bf16((T, Hkv, 128), 7, 0, 0, "k").cuda()
    v = W.normal_bf16((T, Hkv, 128), 7, 0, 0, "v").cuda()
    cu, pos = W.packed_layout(lens)
    cu, pos = torch.from_numpy(cu).cuda(), torch.from_numpy(pos).cuda()
    outs = []
    for _ in range(2):
        cache = new_cache(2, Hkv, cap)
        out, _, _ = qa.prefill(cache, params(Hq), q, k, v, cu, pos, max(lens))
        outs.append((out.clone(), cache.k.clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


def test_single_key_row_equals_v():
    # The first token of a fresh prompt sees one key: its output is V[0] to
    # within the final bf16 rounding of fp32 arithmetic (p = 1, 1/l = 1).
    lens, Hq, Hkv = [5], 4, 1
    q = W.normal_bf16((5, Hq, 128), 8, 0, 0, "q").cuda()
    k = W.normal_bf16((5, Hkv, 128), 8, 0, 0, "k").cuda()
    v = W.normal_bf16((5, Hkv, 128), 8, 0, 0, "v").cuda()
    cu, pos = W.packed_layout(lens)
    cache = new_cache(1, Hkv, 8)
    out, _, _ = qa.prefill(cache, params(Hq), q, k, v,
                           torch.from_numpy(cu).cuda(),
                           torch.from_numpy(pos).cuda(), 5)
    for h in range(Hq):
        assert torch.equal(out[0, h].view(torch.int16), v[0, 0].view(torch.int16))


def test_empty_call_is_noop():
    cache = new_cache(1, 1, 8)
    z = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((0, 1, 128), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    pos = torch.zeros(0, dtype=torch.int32, device="cuda")
    out, _, _ = qa.prefill(cache, params(4), z, zk, zk, cu, pos, 1)
    assert out.shape[0] == 0


def test_invalid_position_flags_and_zeroes():
    lens, Hq, Hkv, cap = [6], 4, 1, 8
    q = W.normal_bf16((6, Hq, 128), 9, 0, 0, "q").cuda()
    k = W.normal_bf16((6, Hkv, 128), 9, 0, 0, "k").cuda()
    v = W.normal_bf16((6, Hkv, 128), 9, 0, 0, "v").cuda()
    cu = torch.tensor([0, 6], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0, 1, 2, 3, 4, 99], dtype=torch.int32, device="cuda")
    cache = new_cache(1, Hkv, cap)
    out, _, ws = qa.prefill(cache, params(Hq), q, k, v, cu, pos, 6)
    code = qa.device_error(ws)
    assert code & qa.QA_DEVERR_POSITION
    assert torch.count_nonzero(out[5].float()) == 0
    assert torch.isfinite(out[:5].float()).all()
    assert qa.device_error(ws) == 0  # cleared by the read


def test_launch_counters_prove_hip_path():
    before = qa.counters()
    run_prefill([16], 4, 1, 16, seed=10)
    after = qa.counters()
    assert after[0] == before[0] + 1       # one prefill call
    assert after[3] >= before[3] + 2       # prologue + attention kernels


def test_full_size_b4_s2048():
    # one Qwen3-4B layer at B=4 x 2048: every (token, head) row and its LSE
    # against the oracle; 1024 q-tiles over the persistent grid, so every CU
    # takes several tiles from the counter
    w = W.get(2)
    _, _, st = run_prefill(list(w.prompt_lens), w.n_q_heads, w.n_kv_heads,
                           w.capacity, seed=12)
    say(f"FULLSIZE_STATS prefill_b4_s2048 {st}")


def test_full_size_ragged():
    w = W.get(3)
    lens = W.ragged_lengths(3, w.batch, w.ragged_choices)
    _, _, st = run_prefill(lens, w.n_q_heads, w.n_kv_heads, w.capacity,
                           seed=14)
    say(f"FULLSIZE_STATS prefill_ragged {lens} {st}")


@pytest.mark.parametrize("lens,Hq,Hkv,cap", [
    ([2048, 512, 512, 512], 32, 8, 2176),  # one heavy sequence: most late q-tiles empty
    ([2900, 700, 1900], 8, 2, 3008),       # 6 pairs (not a multiple of 8), 276 q-tiles
])
def test_skewed_batches_over_the_persistent_grid(lens, Hq, Hkv, cap):
    # every row against the oracle where the workgroups take their further
    # q-tiles from the per-XCD counters with a skewed mix of tile weights
    _, _, st = run_prefill(lens, Hq, Hkv, cap, seed=16)
    say(f"FULLSIZE_STATS prefill_skewed {lens} {st}")


def test_chunked_prefill_full_size():
    # B=4 prompts of 2048 fed as four 512-token chunks per sequence, each
    # chunk attending to the slots the earlier chunks wrote; every row of
    # every chunk and the final cache against the oracle
    w = W.get(2)
    B, Hq, Hkv, cap, S, C = (w.batch, w.n_q_heads, w.n_kv_heads, w.capacity,
                             w.prompt_lens[0], 512)
    seed = 15
    say(f"chunked prefill: B={B} S={S} chunk={C}")
    q = W.normal_bf16((B, S, Hq, 128), seed, 0, 0, "q")
    k = W.normal_bf16((B, S, Hkv, 128), seed, 0, 0, "k")
    v = W.normal_bf16((B, S, Hkv, 128), seed, 0, 0, "v")
    cache = new_cache(B, Hkv, cap)
    oc = oracle.Cache.empty(B, Hkv, cap, 128)
    p = params(Hq)
    ws = qa.workspace(qa.QA_OP_PREFILL, B, Hq, Hkv, B * C)
    lse = torch.empty((B * C, Hq), device="cuda")
    seq = seq_index([C] * B)
    stats = []
    for c0 in range(0, S, C):
        qc = q[:, c0:c0 + C].reshape(B * C, Hq, 128)
        kc = k[:, c0:c0 + C].reshape(B * C, Hkv, 128)
        vc = v[:, c0:c0 + C].reshape(B * C, Hkv, 128)
        cu, pos = W.packed_layout([C] * B, [c0] * B)
        out, _, _ = qa.prefill(cache, p, qc.cuda(), kc.cuda(), vc.cuda(),
                               torch.from_numpy(cu).cuda(),
                               torch.from_numpy(pos).cuda(), C, lse=lse, ws=ws)
        oc = oracle.write_kv(oc, kc.double().numpy(), vc.double().numpy(), seq,
                             pos, theta=THETA, eps=EPS)
        ref, ref_lse = oracle.attend_tokens(oc, qc.double().numpy(), seq, pos,
                                            scale=1 / np.sqrt(128), theta=THETA,
                                            eps=EPS)
        stats.append(compare(f64(out), ref, f"chunk at {c0}"))
        compare(f64(lse)[..., None], ref_lse[..., None], f"chunk lse at {c0}",
                atol=1e-2, rrel=float("inf"), out_bf16=False)
    assert qa.device_error(ws) == 0
    check_cache(cache, oc)
    say(f"FULLSIZE_STATS prefill_chunked_4x512 {stats[-1]}")
