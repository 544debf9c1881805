"""GPU parity of qa_decode (split-K, fused prologue and merge) vs the oracle."""

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


def _seeded_prefix(B, Hkv, cap, lens, seed):
    """GPU + oracle caches whose rows b hold lens[b] seeded slots."""
    cache = new_cache(B, Hkv, cap)
    oc = oracle.Cache.empty(B, Hkv, cap, 128)
    prefix_fill(cache, oc, lens, seed)
    return cache, oc


def run_steps(B, Hq, Hkv, cap, lens, steps, seed, max_ctx=None, weights=False,
              check_every=1):
    say(f"decode case: B={B} Hq={Hq} Hkv={Hkv} cap={cap} lens={lens} "
        f"steps={steps} seed={seed} max_ctx={max_ctx}")
    cache, oc = _seeded_prefix(B, Hkv, cap, lens, seed)
    max_ctx = max_ctx or cap
    q_w = k_w = None
    if weights:
        q_w = (W.normal_bf16((128,), seed, 0, 0, "norm_w", std=0.3) + 1.0).to(
            torch.bfloat16)
        k_w = (W.normal_bf16((128,), seed, 0, 1, "norm_w", std=0.3) + 1.0).to(
            torch.bfloat16)
    p = params(Hq, q_w=None if q_w is None else q_w.cuda(),
               k_w=None if k_w is None else k_w.cuda())
    ws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, max_ctx)
    lse = torch.empty((B, Hq), device="cuda")
    pos = np.array(lens, dtype=np.int32)
    stats = []
    for s in range(steps):
        q = W.normal_bf16((B, Hq, 128), seed, 1, s, "q")
        k = W.normal_bf16((B, Hkv, 128), seed, 1, s, "k")
        v = W.normal_bf16((B, Hkv, 128), seed, 1, s, "v")
        out, _, _ = qa.decode(cache, p, q.cuda(), k.cuda(), v.cuda(),
                              torch.from_numpy(pos).cuda(), max_ctx, lse=lse,
                              ws=ws)
        ref, ref_lse, oc = oracle.decode(
            oc, q.double().numpy(), k.double().numpy(), v.double().numpy(),
            pos, scale=SCALE, theta=THETA, eps=EPS,
            q_w=None if q_w is None else q_w.double().numpy(),
            k_w=None if k_w is None else k_w.double().numpy())
        if s % check_every == 0 or s == steps - 1:
            stats.append(compare(f64(out), ref, f"decode step {s}"))
            compare(f64(lse)[..., None], ref_lse[..., None], f"lse step {s}",
                    atol=1e-2, rrel=float("inf"), out_bf16=False)
        pos = pos + 1
    assert qa.device_error(ws) == 0
    check_cache(cache, oc)
    return stats


def test_tiny_config_steps():
    w = W.get("tiny")
    run_steps(1, w.n_q_heads, w.n_kv_heads, w.capacity, [64], 8, seed=20)


def test_qwen3_b1_512_32_steps():
    w = W.get(1)
    run_steps(1, w.n_q_heads, w.n_kv_heads, w.capacity, [512], 32, seed=21,
              check_every=4)


def test_b4_full_context_2048():
    w = W.get(2)
    run_steps(4, w.n_q_heads, w.n_kv_heads, w.capacity, [2048] * 4, 3,
              seed=22)


def test_ragged_contexts():
    w = W.get(3)
    lens = W.ragged_lengths(3, w.batch, w.ragged_choices)
    run_steps(4, w.n_q_heads, w.n_kv_heads, w.capacity, lens, 3, seed=23)


@pytest.mark.parametrize("lens", [[2175, 1, 2, 1000], [0, 2175, 0, 0],
                                  [5, 2175, 2175, 3]])
def test_extreme_length_mix(lens):
    # Cache workgroups are shared out by context length: a near-full context
    # beside near-empty ones gets most of them (runs still within the split
    # capacity), and an empty context none.
    w = W.get(2)
    run_steps(4, w.n_q_heads, w.n_kv_heads, w.capacity, lens, 1, seed=26)


def test_large_batch_one_split_per_pair():
    # 64 sequences x 8 kv heads: 512 (sequence, kv head) pairs, so the split
    # layout falls to its floor (one cache split of up to 16 tiles per pair)
    g = np.random.default_rng(27)
    lens = [int(x) for x in g.integers(0, 250, 64)]
    run_steps(64, 32, 8, 260, lens, 2, seed=27)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (16, 2)])
def test_groups_and_short_contexts(Hq, Hkv):
    run_steps(3, Hq, Hkv, 200, [0, 1, 130], 3, seed=24)


def test_merge_kernel_many_splits():
    # 2 (sequence, kv head) pairs do not fill a round of the 8-XCD deal, so the
    # partials go through the merge kernel: ~63 splits, several batches of 16
    run_steps(1, 16, 2, 1100, [1000], 2, seed=28)


def test_norm_weights():
    run_steps(2, 8, 2, 300, [100, 257], 2, seed=25, weights=True)


@pytest.mark.parametrize("tiles", range(1, 17))
def test_every_split_length(tiles):
    # 2 sequences x 8 kv heads: 32 cache splits per pair, so max_ctx = 512 t
    # gives runs of up to 16 t rows -- each split length the kernel is built
    # for.  One sequence fills the context, the other a third of it.
    B, Hq, Hkv, cap = 2, 32, 8, 512 * tiles
    run_steps(B, Hq, Hkv, cap, [cap - 1, cap // 3], 1, 40 + tiles)


def test_split_count_invariance():
    # The same step with max_ctx = context (few splits) and max_ctx = capacity
    # (more, partly empty splits) agrees to fp32 reordering noise.
    B, Hq, Hkv, cap, L = 2, 32, 8, 2176, 700
    outs = []
    for max_ctx in (L + 1, cap):
        cache, _ = _seeded_prefix(B, Hkv, cap, [L, L], 26)
        q = W.normal_bf16((B, Hq, 128), 26, 1, 0, "q").cuda()
        k = W.normal_bf16((B, Hkv, 128), 26, 1, 0, "k").cuda()
        v = W.normal_bf16((B, Hkv, 128), 26, 1, 0, "v").cuda()
        pos = torch.full((B,), L, dtype=torch.int32, device="cuda")
        out, _, _ = qa.decode(cache, params(Hq), q, k, v, pos, max_ctx)
        outs.append(f64(out))
    assert np.abs(outs[0] - outs[1]).max() < 2e-3


def test_decode_matches_prefill_row():
    # decode of token t after a prefill of t tokens == row t of a prefill of
    # t+1 tokens (both on the GPU).
    Hq, Hkv, S = 32, 8, 300
    q = W.normal_bf16((S, Hq, 128), 27, 0, 0, "q").cuda()
    k = W.normal_bf16((S, Hkv, 128), 27, 0, 0, "k").cuda()
    v = W.normal_bf16((S, Hkv, 128), 27, 0, 0, "v").cuda()
    p = params(Hq)
    c1 = new_cache(1, Hkv, S)
    cu, pos = W.packed_layout([S])
    full, _, _ = qa.prefill(c1, p, q, k, v, torch.from_numpy(cu).cuda(),
                            torch.from_numpy(pos).cuda(), S)
    c2 = new_cache(1, Hkv, S)
    cu, pos = W.packed_layout([S - 1])
    qa.prefill(c2, p, q[:-1], k[:-1], v[:-1], torch.from_numpy(cu).cuda(),
               torch.from_numpy(pos).cuda(), S - 1)
    out, _, _ = qa.decode(c2, p, q[-1:].contiguous(), k[-1:].contiguous(),
                          v[-1:].contiguous(),
                          torch.tensor([S - 1], dtype=torch.int32,
                                       device="cuda"), S)
    d = np.abs(f64(out[0]) - f64(full[-1])).max()
    say(f"  decode vs prefill row: max diff {d}")
    assert d < 1e-2
    assert torch.equal(c1.k.view(torch.int16), c2.k.view(torch.int16))


def test_invalid_position_flags_and_zeroes():
    B, Hq, Hkv, cap = 2, 4, 1, 16
    cache, _ = _seeded_prefix(B, Hkv, cap, [5, 5], 28)
    q = W.normal_bf16((B, Hq, 128), 28, 1, 0, "q").cuda()
    k = W.normal_bf16((B, Hkv, 128), 28, 1, 0, "k").cuda()
    v = W.normal_bf16((B, Hkv, 128), 28, 1, 0, "v").cuda()
    pos = torch.tensor([5, 16], dtype=torch.int32, device="cuda")
    out, _, ws = qa.decode(cache, params(Hq), q, k, v, pos, cap)
    assert qa.device_error(ws) & qa.QA_DEVERR_POSITION
    assert torch.count_nonzero(out[1].float()) == 0
    assert torch.isfinite(out[0].float()).all()


@pytest.mark.parametrize("B,lens", [(4, [250, 120, 7, 299]), (3, [250, 120, 7])])
def test_merge_counters_left_at_zero(B, lens):
    # With B x Hkv a multiple of 8 (here 8 pairs) the split-K partials are
    # merged inside the decode launch, by the last workgroup of each (sequence,
    # kv head) to count in on a counter in the workspace; otherwise (6 pairs)
    # a second kernel merges them.  Either way every call must leave the
    # counters at zero (as a fresh workspace has them), flag nothing, and give
    # the same bytes call after call and as a fresh workspace does.
    Hq, Hkv, cap = 8, 2, 300
    cache, _ = _seeded_prefix(B, Hkv, cap, lens, 31)
    q = W.normal_bf16((B, Hq, 128), 31, 1, 0, "q").cuda()
    k = W.normal_bf16((B, Hkv, 128), 31, 1, 0, "k").cuda()
    v = W.normal_bf16((B, Hkv, 128), 31, 1, 0, "v").cuda()
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    p = params(Hq)
    ws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)
    fresh = ws.clone()
    outs = []
    for _ in range(5):
        out, _, _ = qa.decode(cache, p, q, k, v, pos, cap, ws=ws)
        outs.append(out.clone())
    torch.cuda.synchronize()
    assert qa.device_error(ws) == 0
    n, tail = ws.numel(), 256 * ((B * Hkv * 128 + 255) // 256)  # counters close the layout
    assert torch.equal(ws[n - tail:], fresh[n - tail:])
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    ref, _, ws2 = qa.decode(cache, p, q, k, v, pos, cap)
    assert qa.device_error(ws2) == 0
    assert torch.equal(ref.view(torch.int16), outs[0].view(torch.int16))
    say(f"  B={B}: {B * Hkv} pairs, 5 calls on one workspace, counters back at zero")


def test_deterministic_rerun():
    B, Hq, Hkv, cap = 4, 32, 8, 1100
    cache, _ = _seeded_prefix(B, Hkv, cap, [1000, 900, 1099, 3], 29)
    q = W.normal_bf16((B, Hq, 128), 29, 1, 0, "q").cuda()
    k = W.normal_bf16((B, Hkv, 128), 29, 1, 0, "k").cuda()
    v = W.normal_bf16((B, Hkv, 128), 29, 1, 0, "v").cuda()
    pos = torch.tensor([1000, 900, 1099, 3], dtype=torch.int32, device="cuda")
    ws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)
    a, _, _ = qa.decode(cache, params(Hq), q, k, v, pos, cap, ws=ws)
    a = a.clone()
    b, _, _ = qa.decode(cache, params(Hq), q, k, v, pos, cap, ws=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_stale_merge_counters_are_flagged():
    # A decode workspace that served a prefill (its cos/sin table written over
    # the merge counters) and was not cleared again: the in-launch merge must
    # not run silently on those counters -- the call sets QA_DEVERR_MERGE.
    # After qa_workspace_init the same buffer gives the fresh-workspace result.
    B, Hq, Hkv, cap = 4, 8, 2, 300
    lens = [250, 120, 7, 299]
    cache, _ = _seeded_prefix(B, Hkv, cap, lens, 32)
    q = W.normal_bf16((B, Hq, 128), 32, 1, 0, "q").cuda()
    k = W.normal_bf16((B, Hkv, 128), 32, 1, 0, "k").cuda()
    v = W.normal_bf16((B, Hkv, 128), 32, 1, 0, "v").cuda()
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    p = params(Hq)
    ws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)
    n = ws.numel()
    # the largest prefill whose table fits: it covers all but the last
    # 256 bytes of the buffer, i.e. the counters of pairs 2 .. 7
    T = (n - 256) // 512
    assert 256 + T * 512 >= n - 256 and qa.workspace_bytes(
        qa.QA_OP_PREFILL, 1, Hq, Hkv, T) <= n
    pc = new_cache(1, Hkv, T)
    pq = W.normal_bf16((T, Hq, 128), 32, 2, 0, "q").cuda()
    pk = W.normal_bf16((T, Hkv, 128), 32, 2, 0, "k").cuda()
    pv = W.normal_bf16((T, Hkv, 128), 32, 2, 0, "v").cuda()
    cu, ppos = W.packed_layout([T])
    qa.prefill(pc, p, pq, pk, pv, torch.from_numpy(cu).cuda(),
               torch.from_numpy(ppos).cuda(), T, ws=ws)
    assert qa.device_error(ws) == 0
    qa.decode(cache, p, q, k, v, pos, cap, ws=ws)
    code = qa.device_error(ws)
    say(f"  decode on a stale workspace: error word {code}")
    assert code & qa.QA_DEVERR_MERGE
    # cleared again, the buffer behaves as a fresh workspace
    qa.lib().qa_workspace_init(qa._ptr(ws), n, qa._stream(None))
    c2, _ = _seeded_prefix(B, Hkv, cap, lens, 32)
    out, _, _ = qa.decode(c2, p, q, k, v, pos, cap, ws=ws)
    out = out.clone()
    assert qa.device_error(ws) == 0
    c3, _ = _seeded_prefix(B, Hkv, cap, lens, 32)
    ref, _, _ = qa.decode(c3, p, q, k, v, pos, cap)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
