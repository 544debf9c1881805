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
