"""Every entry point can be captured in a HIP graph and replayed (qa.h: the
calls allocate nothing and synchronise nothing).  Each graph is replayed
several times with eager work of the same kind between replays, and every
replay must reproduce the eager result bit for bit (the kernels are
deterministic: no result depends on scheduling).  For prefill this also
checks that the attention grid's q-tile counters are re-zeroed by every
call (they are cleared by the K/V prologue kernel, not by a memset)."""

import numpy as np
import pytest
import torch

import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import NAN_BITS, bits, new_cache, params, say

pytestmark = pytest.mark.gpu
REPLAYS = 3


def _replay_check(name, run, outs, disturb):
    """Eager reference, then capture run() and replay it REPLAYS times with
    disturb() (eager work that overwrites the outputs) before each replay."""
    run()
    torch.cuda.synchronize()
    ref = [bits(o).copy() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for r in range(REPLAYS):
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(bits(o), ref[i]), f"{name}: replay {r} output {i}"
    say(f"  {name}: {REPLAYS} replays bit-identical to the eager call")


def test_prefill_graph():
    B, Hq, Hkv, cap = 3, 32, 8, 640
    lens = [600, 257, 64]
    T = sum(lens)
    q = W.normal_bf16((T, Hq, 128), 80, 0, 0, "q").cuda()
    k = W.normal_bf16((T, Hkv, 128), 80, 0, 0, "k").cuda()
    v = W.normal_bf16((T, Hkv, 128), 80, 0, 0, "v").cuda()
    cu, pos = W.packed_layout(lens)
    cu, pos = torch.from_numpy(cu).cuda(), torch.from_numpy(pos).cuda()
    cache = new_cache(B, Hkv, cap)
    p = params(Hq)
    out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    ws = qa.workspace(qa.QA_OP_PREFILL, B, Hq, Hkv, T)

    def run():
        qa.prefill(cache, p, q, k, v, cu, pos, max(lens), out=out, lse=lse, ws=ws)

    def disturb():  # outputs cleared, the cache back to its NaN sentinel
        out.zero_()
        lse.zero_()
        cache.k.view(torch.int16).fill_(NAN_BITS)
        cache.v.view(torch.int16).fill_(NAN_BITS)
    _replay_check("prefill", run, [out, lse, cache.k, cache.v], disturb)
    assert qa.device_error(ws) == 0


def test_decode_and_verify_graphs():
    B, Hq, Hkv, cap = 4, 32, 8, 1100
    lens = [1024, 700, 3, 1000]
    cache = new_cache(B, Hkv, cap)
    # a written prefix for every row (values as if from earlier calls)
    for b, L in enumerate(lens):
        cache.k[b, :, :L] = W.normal_bf16((Hkv, L, 128), 81, b, 0, "cache_k").cuda()
        cache.v[b, :, :L] = W.normal_bf16((Hkv, L, 128), 81, b, 0, "cache_v").cuda()
    p = params(Hq)
    q = W.normal_bf16((B, Hq, 128), 81, 9, 0, "q").cuda()
    k = W.normal_bf16((B, Hkv, 128), 81, 9, 0, "k").cuda()
    v = W.normal_bf16((B, Hkv, 128), 81, 9, 0, "v").cuda()
    dpos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)

    def run_d():
        qa.decode(cache, p, q, k, v, dpos, cap, out=out, lse=lse, ws=ws)

    def disturb_d():
        out.zero_()
        lse.zero_()
    _replay_check("decode", run_d, [out, lse], disturb_d)

    n = 16
    vq = W.normal_bf16((B, n, Hq, 128), 81, 10, 0, "q").cuda()
    vk = W.normal_bf16((B, n, Hkv, 128), 81, 10, 0, "k").cuda()
    vv = W.normal_bf16((B, n, Hkv, 128), 81, 10, 0, "v").cuda()
    start = torch.tensor([L + 1 for L in lens], dtype=torch.int32, device="cuda")
    vout = torch.empty((B, n, Hq, 128), dtype=torch.bfloat16, device="cuda")
    vlse = torch.empty((B, n, Hq), dtype=torch.float32, device="cuda")
    vws = qa.workspace(qa.QA_OP_VERIFY, B, Hq, Hkv, cap, n)

    def run_v():
        qa.verify(cache, p, vq, vk, vv, start, cap, out=vout, lse=vlse, ws=vws)

    def disturb_v():
        vout.zero_()
        vlse.zero_()
    _replay_check("verify", run_v, [vout, vlse], disturb_v)
    assert qa.device_error(ws) == 0 and qa.device_error(vws) == 0


def test_rmsnorm_graph():
    T, H = 300, 2560
    x = W.normal_bf16((T, H), 82, 0, 0, "hidden_x").cuda()
    res0 = W.normal_bf16((T, H), 82, 0, 1, "hidden_res").cuda()
    res = res0.clone()
    w = (W.normal_bf16((H,), 82, 0, 2, "norm_w", std=0.3) + 1.0).to(
        torch.bfloat16).cuda()
    out = torch.empty_like(x)

    def run():
        res.copy_(res0)
        qa.rmsnorm_hidden(x, residual=res, weight=w, out=out)

    def disturb():
        out.zero_()
        res.zero_()
    _replay_check("rmsnorm_hidden", run, [out, res], disturb)


def test_captured_multilayer_decode_step_vs_oracle():
    """The benchmark's decode step, checked against the oracle: the qa_decode
    calls of several layers and the on-device position increment captured in
    one graph (one workspace shared by the layers, as in bench.py), replayed
    step after step from position 2048 at the B=4 Qwen3-4B shape.  Fresh
    inputs are copied into the graph's static buffers between replays; every
    layer's output and LSE at every step is compared with oracle.decode and
    the caches byte for byte at the end."""
    import oracle

    from .gpu_helpers import EPS, THETA, check_cache, compare, f64, prefix_fill

    w = W.get(2)
    B, Hq, Hkv, cap, S = w.batch, w.n_q_heads, w.n_kv_heads, w.capacity, 2048
    L, NSTEP, seed = 3, 8, 90
    say(f"captured decode step: {L} layers, {NSTEP} steps from {S}, B={B}")
    caches, ocs = [], []
    for l in range(L):
        c = new_cache(B, Hkv, cap)
        oc = oracle.Cache.empty(B, Hkv, cap, 128)
        prefix_fill(c, oc, [S] * B, seed + l)
        caches.append(c)
        ocs.append(oc)
    p = params(Hq)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    qs = [torch.zeros((B, Hq, 128), **bf) for _ in range(L)]
    ks = [torch.zeros((B, Hkv, 128), **bf) for _ in range(L)]
    vs = [torch.zeros((B, Hkv, 128), **bf) for _ in range(L)]
    outs = [torch.empty((B, Hq, 128), **bf) for _ in range(L)]
    lses = [torch.empty((B, Hq), dtype=torch.float32, device="cuda")
            for _ in range(L)]
    dpos = torch.full((B,), S, dtype=torch.int32, device="cuda")
    ws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)

    def step():
        for l in range(L):
            qa.decode(caches[l], p, qs[l], ks[l], vs[l], dpos, cap, out=outs[l],
                      lse=lses[l], ws=ws)
        dpos.add_(1)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the path outside the capture
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    dpos.fill_(S)  # the warm-up's slot S is rewritten by the first replay
    torch.cuda.synchronize()
    pos = np.full(B, S, dtype=np.int64)
    for st in range(NSTEP):
        inp = []
        for l in range(L):
            q = W.normal_bf16((B, Hq, 128), seed, l, st, "q")
            k = W.normal_bf16((B, Hkv, 128), seed, l, st, "k")
            v = W.normal_bf16((B, Hkv, 128), seed, l, st, "v")
            qs[l].copy_(q)
            ks[l].copy_(k)
            vs[l].copy_(v)
            inp.append((q, k, v))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, (q, k, v) in enumerate(inp):
            ref, ref_lse, ocs[l] = oracle.decode(
                ocs[l], q.double().numpy(), k.double().numpy(),
                v.double().numpy(), pos, scale=w.scale, theta=THETA, eps=EPS)
            compare(f64(outs[l]), ref, f"step {st} layer {l}")
            compare(f64(lses[l])[..., None], ref_lse[..., None],
                    f"step {st} layer {l} lse", atol=1e-2, rrel=float("inf"),
                    out_bf16=False)
        pos = pos + 1
    assert dpos.cpu().tolist() == [S + NSTEP] * B
    assert qa.device_error(ws) == 0
    for l in range(L):
        check_cache(caches[l], ocs[l], f"layer {l} cache")
