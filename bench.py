"""Benchmark of the GQA attention path on one MI355X.

Workload: Qwen3-4B attention shapes, batch 4, 36 layers, 2048-token prompts,
then 128 decode steps that each read all 36 layers' caches
(4 x 8 x 2176 x 128 bf16 for K and for V per layer), plus one verification
call of a 16-token draft block per sequence after a 2048-slot cache.

One bench step = the whole path once:
  prefill of all 36 layers (K/V prologue + flash attention per layer),
  128 decode steps x 36 layers (each decode step is one captured HIP graph of
  36 qa_decode launches plus the on-device position increment),
  one qa_verify call (16-token block, batch 4, 2048 + 16 keys).
Inputs are synthetic (seeded device draws, bf16 ~N(0,1)) and resident in HBM
before timing starts.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-ragged] [--profile-kernels]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA attn: decode µs/step + HBM GB/s; prefill TFLOP/s (B=4, ctx 2048)"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 (256 CU x 2.4 GHz x 4096)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_info():
    p = os.path.join(ROOT, "prefill_attention_rmsnorm_amd", "_build",
                     "BUILD_INFO.json")
    try:
        with open(p) as f:
            return json.load(f)
    except OSError:
        return {}


class Workload:
    """Device buffers of the benchmark workload."""

    def __init__(self, torch, qa, W):
        self.torch, self.qa = torch, qa
        w = W.get(2)
        self.w = w
        self.B, self.L = w.batch, w.n_layers
        self.Hq, self.Hkv, self.S = w.n_q_heads, w.n_kv_heads, w.prompt_lens[0]
        self.cap, self.steps = w.capacity, w.decode_steps
        dev = "cuda"
        g = torch.Generator(device=dev)
        g.manual_seed(2)
        T = self.B * self.S

        def rnd(*shape):
            return torch.randn(*shape, generator=g, device=dev,
                               dtype=torch.float32).to(torch.bfloat16)

        log(f"bench: allocating {self.L} layers (caches + prefill inputs)")
        self.caches = [qa.Cache.empty(self.B, self.Hkv, self.cap)
                       for _ in range(self.L)]
        self.pq = [rnd(T, self.Hq, 128) for _ in range(self.L)]
        self.pk = [rnd(T, self.Hkv, 128) for _ in range(self.L)]
        self.pv = [rnd(T, self.Hkv, 128) for _ in range(self.L)]
        self.dq = [rnd(self.B, self.Hq, 128) for _ in range(self.L)]
        self.dk = [rnd(self.B, self.Hkv, 128) for _ in range(self.L)]
        self.dv = [rnd(self.B, self.Hkv, 128) for _ in range(self.L)]
        self.params = qa.Params(self.Hq, w.scale, w.theta, w.eps)
        cu = torch.arange(0, T + 1, self.S, dtype=torch.int32, device=dev)
        self.cu = cu
        self.ppos = torch.arange(self.S, dtype=torch.int32,
                                 device=dev).repeat(self.B)
        self.pout = torch.empty((T, self.Hq, 128), dtype=torch.bfloat16,
                                device=dev)
        self.pws = qa.workspace(qa.QA_OP_PREFILL, self.B, self.Hq, self.Hkv, T)
        self.dpos = torch.full((self.B,), self.S, dtype=torch.int32,
                               device=dev)
        self.dpos0 = self.dpos.clone()
        self.dout = torch.empty((self.B, self.Hq, 128), dtype=torch.bfloat16,
                                device=dev)
        self.dws = qa.workspace(qa.QA_OP_DECODE, self.B, self.Hq, self.Hkv,
                                self.cap)
        # verification workload: 2048 seeded slots + a 16-token block
        w4 = W.get(4)
        self.vB, self.vn, self.vL0, self.vcap = (w4.batch, w4.verify_block,
                                                 w4.verify_start, w4.capacity)
        self.vcache = qa.Cache.empty(self.vB, self.Hkv, self.vcap)
        self.vcache.k[:, :, :self.vL0] = rnd(self.vB, self.Hkv, self.vL0, 128)
        self.vcache.v[:, :, :self.vL0] = rnd(self.vB, self.Hkv, self.vL0, 128)
        self.vq = rnd(self.vB, self.vn, self.Hq, 128)
        self.vk = rnd(self.vB, self.vn, self.Hkv, 128)
        self.vv = rnd(self.vB, self.vn, self.Hkv, 128)
        self.vstart = torch.full((self.vB,), self.vL0, dtype=torch.int32,
                                 device=dev)
        self.vout = torch.empty((self.vB, self.vn, self.Hq, 128),
                                dtype=torch.bfloat16, device=dev)
        self.vws = qa.workspace(qa.QA_OP_VERIFY, self.vB, self.Hq, self.Hkv,
                                self.vcap, self.vn)
        torch.cuda.synchronize()
        self.graph = None

    # -- phases ---------------------------------------------------------------
    def prefill_layer(self, l):
        self.qa.prefill(self.caches[l], self.params, self.pq[l], self.pk[l],
                        self.pv[l], self.cu, self.ppos, self.S, out=self.pout,
                        ws=self.pws)

    def prefill_all(self):
        for l in range(self.L):
            self.prefill_layer(l)

    def decode_layer(self, l):
        self.qa.decode(self.caches[l], self.params, self.dq[l], self.dk[l],
                       self.dv[l], self.dpos, self.cap, out=self.dout,
                       ws=self.dws)

    def capture_decode_step(self):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):  # warm the path outside the capture
            for l in range(self.L):
                self.decode_layer(l)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in range(self.L):
                self.decode_layer(l)
            self.dpos.add_(1)
        torch.cuda.synchronize()
        self.graph = g

    def decode_all(self):
        self.dpos.copy_(self.dpos0)
        for _ in range(self.steps):
            self.graph.replay()

    def verify(self):
        self.qa.verify(self.vcache, self.params, self.vq, self.vk, self.vv,
                       self.vstart, self.vcap, out=self.vout, ws=self.vws)


def decode_bytes(B, Hq, Hkv, ctx):
    """Algorithmic HBM bytes of one decode launch at context ctx: K and V
    reads of ctx slots, the new K/V slot writes, q reads and output writes."""
    kv_read = 2 * B * Hkv * ctx * 128 * 2
    kv_write = 2 * B * Hkv * 128 * 2
    q_out = 2 * B * Hq * 128 * 2
    return kv_read + kv_write + q_out


def prefill_flops(B, Hq, S):
    """Causal attention flops, lower triangle with the diagonal."""
    return 2.0 * B * Hq * 128 * S * (S + 1)


def cpu_baseline(budget_s=10.0):
    """The fp64 oracle (as is, never tuned) on bounded samples of the
    workloads, on the host cores available to this process
    (len(os.sched_getaffinity(0)) threads for the BLAS pool).

    Headline leg: decode calls of the B=4, 2048-context layer shape, about
    `budget_s` of work, scaled to a 36-layer step.  Further legs: one B=4 x
    2048 prefill layer (the x36 figure is an extrapolation), one verify call
    (B=4, 16-token block after 2048 slots), the tiny workload end to end
    (64-token prefill + 8 decode steps), and one decode call on 1 thread."""
    import numpy as np

    import oracle
    import workloads as W

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None

    def limit(n):
        if threadpool_limits is None:
            import contextlib
            return contextlib.nullcontext()
        return threadpool_limits(limits=n)

    w = W.get(2)
    B, Hq, Hkv, S, cap = w.batch, w.n_q_heads, w.n_kv_heads, 2048, w.capacity
    kw = dict(scale=w.scale, theta=w.theta, eps=w.eps)

    def seeded_cache(B_, Hkv_, L, cap_, seed):
        c = oracle.Cache.empty(B_, Hkv_, cap_, 128)
        c.k[:, :, :L] = W.normal_bf16((B_, Hkv_, L, 128), seed, 0, 0,
                                      "cache_k").double().numpy()
        c.v[:, :, :L] = W.normal_bf16((B_, Hkv_, L, 128), seed, 0, 0,
                                      "cache_v").double().numpy()
        return c

    def decode_call(c, n, pos):
        q = W.normal_bf16((B, Hq, 128), 2, 1, n, "q").double().numpy()
        k = W.normal_bf16((B, Hkv, 128), 2, 1, n, "k").double().numpy()
        v = W.normal_bf16((B, Hkv, 128), 2, 1, n, "v").double().numpy()
        t0 = time.perf_counter()
        _, _, c = oracle.decode(c, q, k, v, pos, **kw)
        return c, time.perf_counter() - t0

    legs = {}
    with limit(cores):
        c = seeded_cache(B, Hkv, S, cap, 2)
        n, spent, pos = 0, 0.0, np.full(B, S, dtype=np.int64)
        while spent < budget_s and n < 64:
            c, dt = decode_call(c, n, pos)
            spent += dt
            pos = pos + 1
            n += 1
        per_layer_us = spent / n * 1e6
        # one prefill layer, B=4 x 2048
        T = B * S
        q = W.normal_bf16((T, Hq, 128), 2, 0, 0, "q").double().numpy()
        k = W.normal_bf16((T, Hkv, 128), 2, 0, 0, "k").double().numpy()
        v = W.normal_bf16((T, Hkv, 128), 2, 0, 0, "v").double().numpy()
        cu, ppos = W.packed_layout([S] * B)
        t0 = time.perf_counter()
        oracle.prefill(oracle.Cache.empty(B, Hkv, cap, 128), q, k, v, cu, ppos, **kw)
        legs["prefill_layer_us"] = round((time.perf_counter() - t0) * 1e6, 1)
        legs["prefill_36_layers_us_extrapolated"] = round(legs["prefill_layer_us"] * 36, 1)
        del q, k, v
        # one verify call
        w4 = W.get(4)
        vc = seeded_cache(w4.batch, Hkv, w4.verify_start, w4.capacity, 4)
        n_ = w4.verify_block
        vq = W.normal_bf16((B, n_, Hq, 128), 4, 0, 0, "q").double().numpy()
        vk = W.normal_bf16((B, n_, Hkv, 128), 4, 0, 0, "k").double().numpy()
        vv = W.normal_bf16((B, n_, Hkv, 128), 4, 0, 0, "v").double().numpy()
        t0 = time.perf_counter()
        oracle.verify(vc, vq, vk, vv, [w4.verify_start] * B, **kw)
        legs["verify_call_us"] = round((time.perf_counter() - t0) * 1e6, 1)
        # the tiny workload: 64-token prefill, then 8 decode steps
        w0 = W.get(0)
        S0 = w0.prompt_lens[0]
        tq = W.normal_bf16((S0, w0.n_q_heads, 128), 0, 0, 0, "q").double().numpy()
        tk = W.normal_bf16((S0, w0.n_kv_heads, 128), 0, 0, 0, "k").double().numpy()
        tv = W.normal_bf16((S0, w0.n_kv_heads, 128), 0, 0, 0, "v").double().numpy()
        cu0, pos0 = W.packed_layout([S0])
        t0 = time.perf_counter()
        _, _, tc = oracle.prefill(oracle.Cache.empty(1, w0.n_kv_heads, w0.capacity, 128),
                                  tq, tk, tv, cu0, pos0, **kw)
        for st in range(w0.decode_steps):
            dq = W.normal_bf16((1, w0.n_q_heads, 128), 0, 1, st, "q").double().numpy()
            dk = W.normal_bf16((1, w0.n_kv_heads, 128), 0, 1, st, "k").double().numpy()
            dv = W.normal_bf16((1, w0.n_kv_heads, 128), 0, 1, st, "v").double().numpy()
            _, _, tc = oracle.decode(tc, dq, dk, dv, [S0 + st], **kw)
        legs["tiny_run_us"] = round((time.perf_counter() - t0) * 1e6, 1)
    with limit(1):
        _, dt = decode_call(seeded_cache(B, Hkv, S, cap, 2), 0, np.full(B, S))
        legs["decode_step_us_1_thread"] = round(dt * 1e6 * w.n_layers, 1)
    return {"value": round(per_layer_us * w.n_layers, 1), "unit": "us/decode_step",
            "cores": cores, "kind": "oracle",
            "sample": f"{n} single-layer decode calls at B=4, context "
                      f"{S + 1}..{S + n} (fp64 numpy oracle), scaled x{w.n_layers} "
                      f"layers; legs: one prefill layer, one verify call, the "
                      f"tiny run, one decode call on 1 thread (x{w.n_layers})",
            "legs": legs}


def ragged_spread(torch, qa, W, reps=15, n_layers=8):
    """Latency of the ragged batch against the length-proportional cost.

    Batch 4 with prompt lengths drawn from {512, 1024, 1536, 2048} (packed
    prefill, then 64 decode steps at per-sequence contexts) and the same shapes
    at 2048 tokens each, one layer.  The cost of a prefill is sum S(S+1)
    (causal pairs), of a decode step the context slots read, sum L.  For each
    phase ratio = t_ragged / (t_uniform * C_ragged / C_uniform); the check
    passes when |ratio - 1| <= 0.25.  Prefill times are medians of `reps`
    calls.  A decode step is one layer's qa_decode call, the mean over 64
    graph-replayed steps that each go through `n_layers` layer caches in turn
    (median of `reps` replays): 8 caches of ~36 MB exceed the 256 MB MALL, so
    the caches stream from HBM as in the headline step."""
    import numpy as np

    w = W.get(3)
    B, Hq, Hkv, cap, nsteps = (w.batch, w.n_q_heads, w.n_kv_heads, w.capacity,
                               w.decode_steps)
    lens_r = W.ragged_lengths(3, B, w.ragged_choices)
    lens_u = [max(w.ragged_choices)] * B
    p = qa.Params(Hq, w.scale, w.theta, w.eps)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device="cuda",
                           dtype=torch.float32).to(torch.bfloat16)

    def measure(lens):
        T = sum(lens)
        cu, pos = W.packed_layout(lens)
        cu, pos = torch.from_numpy(cu).cuda(), torch.from_numpy(pos).cuda()
        q, k, v = rnd(T, Hq, 128), rnd(T, Hkv, 128), rnd(T, Hkv, 128)
        caches = [qa.Cache.empty(B, Hkv, cap) for _ in range(n_layers)]
        cache = caches[0]
        out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
        ws = qa.workspace(qa.QA_OP_PREFILL, B, Hq, Hkv, T)
        S = max(lens)
        for c in caches[1:]:
            qa.prefill(c, p, q, k, v, cu, pos, S, out=out, ws=ws)
        for _ in range(3):
            qa.prefill(cache, p, q, k, v, cu, pos, S, out=out, ws=ws)
        ts = []
        for _ in range(reps):
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            qa.prefill(cache, p, q, k, v, cu, pos, S, out=out, ws=ws)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        t_pre = float(np.median(ts))
        dq, dk, dv = rnd(B, Hq, 128), rnd(B, Hkv, 128), rnd(B, Hkv, 128)
        dpos0 = torch.tensor(lens, dtype=torch.int32, device="cuda")
        dpos = dpos0.clone()
        dout = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
        dws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            qa.decode(cache, p, dq, dk, dv, dpos, cap, out=dout, ws=dws)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(nsteps):
                for c in caches:
                    qa.decode(c, p, dq, dk, dv, dpos, cap, out=dout, ws=dws)
                dpos.add_(1)
        ts = []
        for _ in range(reps):
            dpos.copy_(dpos0)
            torch.cuda.synchronize()
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / (nsteps * n_layers))
        del caches, cache
        return t_pre, float(np.median(ts))

    pr, dr = measure(lens_r)
    pu, du = measure(lens_u)
    c_pre = sum(x * (x + 1) for x in lens_r) / sum(x * (x + 1) for x in lens_u)
    c_dec = (sum(lens_r) + B * (nsteps + 1) / 2.0) / \
        (sum(lens_u) + B * (nsteps + 1) / 2.0)

    def entry(tr, tu, c):
        ratio = tr / (tu * c)
        return {"t_ragged_us": round(tr, 2), "t_uniform_us": round(tu, 2),
                "cost_ratio": round(c, 4), "ratio": round(ratio, 4),
                "within_25pct": bool(abs(ratio - 1.0) <= 0.25)}

    return {"lengths": lens_r, "uniform_length": lens_u[0], "decode_layers": n_layers,
            "prefill": entry(pr, pu, c_pre),
            "decode_step": entry(dr, du, c_dec)}


def rmsnorm_rate(torch, qa, reps=20):
    """qa_rmsnorm_hidden at the prefill shape of the workload: 4 x 2048
    tokens of hidden 2560, with the residual add and a weight.  Algorithmic
    bytes per call: x and residual read, out and residual written (the 5 KB
    weight aside), 4 * T * H * 2.  Median of `reps` event-timed calls."""
    import numpy as np

    T, H = 4 * 2048, 2560
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    x = torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16)
    res = torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn(H, generator=g, device="cuda")).to(
        torch.bfloat16)
    out = torch.empty_like(x)
    for _ in range(3):
        qa.rmsnorm_hidden(x, residual=res, weight=w, out=out)
    ts = []
    for _ in range(reps):
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        e0.record()
        qa.rmsnorm_hidden(x, residual=res, weight=w, out=out)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    us = float(np.median(ts))
    nbytes = 4 * T * H * 2
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"tokens": T, "hidden": H, "us": round(us, 2),
            "algorithmic_bytes": nbytes, "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def epilogue_rate(torch, qa):
    """qa_attn_epilogue (output projection 4096 -> 2560 with the residual add,
    then the post-attention RMSNorm) at the workload's two shapes: the
    prefill layer's 4 x 2048 tokens, and one decode step's 4 tokens with w_o
    rotated over 16 copies (336 MB, past the 256 MB MALL) as a model's layers
    would be.  Graph-timed replays; flops 2 T 4096 2560, and for the decode
    shape the bytes of w_o per call."""
    H, D = 2560, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    res = {}
    for name, T, ncopy in (("prefill_tokens_8192", 8192, 1), ("decode_tokens_4", 4, 16)):
        o = torch.randn(T, D, generator=g, device="cuda").to(torch.bfloat16)
        ws = [(0.02 * torch.randn(H, D, generator=g, device="cuda")).to(torch.bfloat16)
              for _ in range(ncopy)]
        resid = torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16)
        nw = torch.ones(H, device="cuda", dtype=torch.bfloat16)
        out = torch.empty_like(resid)
        n = max(4, ncopy)

        def fn():
            for i in range(n):
                qa.attn_epilogue(o, ws[i % ncopy], resid, nw, 1e-6, out=out)
        us, _ = _graph_time_us(torch, fn)
        us /= n
        fl = 2.0 * T * D * H
        res[name] = {"us": round(us, 2), "TFLOPs": round(fl / (us * 1e-6) / 1e12, 1),
                     "w_o_GBps": round(H * D * 2 / (us * 1e-6) / 1e9, 1)}
        del ws
    return res


def _graph_time_us(torch, fn, reps=10, warm=2):
    """Median time of one replay of a graph that captures fn(), with events
    on the replaying stream (replays back to back, so no host enqueue gap
    enters a sample)."""
    import numpy as np

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(ts)), g


def membw_probe(torch, qa, nbytes=1 << 30, reps=10):
    """Plain device copy (qa_copy) of 1 GiB: read + write bytes over the
    median time of 4 back-to-back copies in a graph."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def fn():
        for _ in range(4):
            qa.copy(src, dst)
    us, _ = _graph_time_us(torch, fn, reps=reps)
    gbps = 4 * 2 * nbytes / (us * 1e-6) / 1e9
    del src, dst
    return {"bytes_moved_per_copy": 2 * nbytes, "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def verify_rotated(torch, qa, W, copies=8):
    """The verify call on `copies` distinct caches (8 x 34 MB > the 256 MB
    MALL), one graph of `copies` calls: per-call time with the cache bytes
    coming from HBM."""
    w4 = W.get(4)
    B, Hq, Hkv, n, L0, cap = (w4.batch, w4.n_q_heads, w4.n_kv_heads,
                              w4.verify_block, w4.verify_start, w4.capacity)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)
    caches = []
    for _ in range(copies):
        c = qa.Cache.empty(B, Hkv, cap)
        c.k[:, :, :L0] = rnd(B, Hkv, L0, 128)
        c.v[:, :, :L0] = rnd(B, Hkv, L0, 128)
        caches.append(c)
    p = qa.Params(Hq, w4.scale, w4.theta, w4.eps)
    q, k, v = rnd(B, n, Hq, 128), rnd(B, n, Hkv, 128), rnd(B, n, Hkv, 128)
    start = torch.full((B,), L0, dtype=torch.int32, device="cuda")
    out = torch.empty((B, n, Hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = qa.workspace(qa.QA_OP_VERIFY, B, Hq, Hkv, cap, n)

    def fn():
        for c in caches:
            qa.verify(c, p, q, k, v, start, cap, out=out, ws=ws)
    us, _ = _graph_time_us(torch, fn)
    per = us / copies
    nbytes = verify_bytes(B, Hq, Hkv, L0, n)
    err = qa.device_error(ws)
    return {"copies": copies, "us_per_call": round(per, 2),
            "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (per * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (per * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "device_error": err}


def verify_bytes(B, Hq, Hkv, L0, n):
    """Algorithmic HBM bytes of one verify call: K/V of the L0 cached slots
    read, the block's K/V written, q read and outputs written."""
    return 2 * B * Hkv * L0 * 256 + 2 * B * n * Hkv * 256 + 2 * B * n * Hq * 256


def small_latency(torch, qa, W):
    """Latency of the two small workloads, each step replayed from a graph.

    tiny: one 64-token prefill (4 query heads, 1 KV head) and 8 decode steps
    whose positions advance on the device, as one graph (the whole run).
    b1_s512: the B=1, 512-token prefill of one Qwen3-4B layer, and its 32
    decode steps (positions advanced on the device) as one graph; its 2.2 MB
    of cache stay in the caches, so only the time is reported."""
    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(6)

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)
    for key, idx in (("tiny", 0), ("b1_s512", 1)):
        w = W.get(idx)
        S, Hq, Hkv, cap, steps = (w.prompt_lens[0], w.n_q_heads, w.n_kv_heads,
                                  w.capacity, w.decode_steps)
        p = qa.Params(Hq, w.scale, w.theta, w.eps)
        cache = qa.Cache.empty(1, Hkv, cap)
        q, k, v = rnd(S, Hq, 128), rnd(S, Hkv, 128), rnd(S, Hkv, 128)
        cu = torch.tensor([0, S], dtype=torch.int32, device="cuda")
        pos = torch.arange(S, dtype=torch.int32, device="cuda")
        pout = torch.empty((S, Hq, 128), dtype=torch.bfloat16, device="cuda")
        pws = qa.workspace(qa.QA_OP_PREFILL, 1, Hq, Hkv, S)
        dq, dk, dv = rnd(1, Hq, 128), rnd(1, Hkv, 128), rnd(1, Hkv, 128)
        dpos = torch.full((1,), S, dtype=torch.int32, device="cuda")
        dout = torch.empty((1, Hq, 128), dtype=torch.bfloat16, device="cuda")
        dws = qa.workspace(qa.QA_OP_DECODE, 1, Hq, Hkv, cap)

        def prefill():
            qa.prefill(cache, p, q, k, v, cu, pos, S, out=pout, ws=pws)

        def decode_steps():
            dpos.fill_(S)
            for _ in range(steps):
                qa.decode(cache, p, dq, dk, dv, dpos, cap, out=dout, ws=dws)
                dpos.add_(1)

        t_pre, _ = _graph_time_us(torch, prefill)
        t_dec, _ = _graph_time_us(torch, decode_steps)

        def whole():
            prefill()
            decode_steps()
        t_all, _ = _graph_time_us(torch, whole)
        errs = qa.device_error(pws) | qa.device_error(dws)
        out[key] = {"prompt": S, "decode_steps": steps,
                    "prefill_us": round(t_pre, 2),
                    "decode_us_per_step": round(t_dec / steps, 2),
                    "run_us": round(t_all, 2), "device_error": errs}
    return out


def chunked_prefill(torch, qa, W):
    """One B=4 x 2048 prefill layer in one call, and the same prompts in four
    512-token chunks (each attending to the slots the earlier ones wrote):
    the time to the last prompt token's output either way."""
    w = W.get(2)
    B, Hq, Hkv, S, cap, C = (w.batch, w.n_q_heads, w.n_kv_heads,
                             w.prompt_lens[0], w.capacity, 512)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)
    p = qa.Params(Hq, w.scale, w.theta, w.eps)
    cache = qa.Cache.empty(B, Hkv, cap)
    q, k, v = rnd(B * S, Hq, 128), rnd(B * S, Hkv, 128), rnd(B * S, Hkv, 128)
    cu = torch.arange(0, B * S + 1, S, dtype=torch.int32, device="cuda")
    pos = torch.arange(S, dtype=torch.int32, device="cuda").repeat(B)
    out = torch.empty((B * S, Hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = qa.workspace(qa.QA_OP_PREFILL, B, Hq, Hkv, B * S)
    chunks = []
    for c0 in range(0, S, C):
        idx = torch.cat([torch.arange(b * S + c0, b * S + c0 + C, device="cuda")
                         for b in range(B)])
        chunks.append((q[idx].contiguous(), k[idx].contiguous(),
                       v[idx].contiguous(), pos[idx].contiguous(),
                       torch.arange(0, B * C + 1, C, dtype=torch.int32,
                                    device="cuda")))
    cws = qa.workspace(qa.QA_OP_PREFILL, B, Hq, Hkv, B * C)
    cout = torch.empty((B * C, Hq, 128), dtype=torch.bfloat16, device="cuda")

    def one_shot():
        qa.prefill(cache, p, q, k, v, cu, pos, S, out=out, ws=ws)

    def chunked():
        for cq, ck, cv, cp, ccu in chunks:
            qa.prefill(cache, p, cq, ck, cv, ccu, cp, C, out=cout, ws=cws)
    t1, _ = _graph_time_us(torch, one_shot)
    t4, _ = _graph_time_us(torch, chunked)
    return {"batch": B, "prompt": S, "chunk": C, "one_shot_us": round(t1, 2),
            "chunked_us": round(t4, 2),
            "device_error": qa.device_error(ws) | qa.device_error(cws)}


def profile_kernels(wl, torch, qa):
    """One pass of each hot kernel plus a copy of known size, for rocprofv3
    kernel-trace and counter runs: copy 256 MiB x3 (counter calibration),
    prefill of layer 0, one decode step over the 36 layers at context
    2048 + 65, one verify call, and the attention epilogue at 8192 tokens
    (GEMM) and at 4 tokens (streaming kernel)."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        qa.copy(src, dst)
    wl.prefill_layer(0)
    wl.dpos.fill_(wl.S + wl.steps // 2)
    for l in range(wl.L):
        wl.decode_layer(l)
    wl.verify()
    for T in (8192, 4):
        o = torch.randn(T, 4096, device="cuda").to(torch.bfloat16)
        w_o = (0.02 * torch.randn(2560, 4096, device="cuda")).to(torch.bfloat16)
        resid = torch.randn(T, 2560, device="cuda").to(torch.bfloat16)
        qa.attn_epilogue(o, w_o, resid, None, 1e-6)
    torch.cuda.synchronize()
    ctx = wl.S + wl.steps // 2 + 1
    print(json.dumps({
        "copy_bytes": n,
        "decode_ctx": ctx,
        "decode_algorithmic_bytes_per_launch":
            decode_bytes(wl.B, wl.Hq, wl.Hkv, ctx),
        "prefill_flops": prefill_flops(wl.B, wl.Hq, wl.S),
        "provenance": build_info()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the untimed extras (ragged-batch latency spread, "
                         "hidden-state RMSNorm rate)")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="run each hot kernel once (for rocprofv3) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path runs on one device's "
              f"share of the work; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W
    from prefill_attention_rmsnorm_amd import qa

    qa.lib()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    wl = Workload(torch, qa, W)
    if args.profile_kernels:
        profile_kernels(wl, torch, qa)
        return
    log("bench: capturing the decode-step graph")
    wl.capture_decode_step()

    def step(evs=None):
        if evs: evs[0].record()
        wl.prefill_all()
        if evs: evs[1].record()
        wl.decode_all()
        if evs: evs[2].record()
        wl.verify()
        if evs: evs[3].record()

    for i in range(args.warmup):
        log(f"bench: warmup step {i}")
        step()
    torch.cuda.synchronize()

    phase = {"prefill": 0.0, "decode": 0.0, "verify": 0.0}
    per_step = []
    t_start = time.perf_counter()
    for i in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(evs)
        torch.cuda.synchronize()
        p, d, v = (evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2]),
                   evs[2].elapsed_time(evs[3]))
        phase["prefill"] += p
        phase["decode"] += d
        phase["verify"] += v
        per_step.append(p + d + v)
        log(f"bench: step {i}: prefill {p:.3f} ms, decode {d:.3f} ms, "
            f"verify {v * 1e3:.1f} us")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # every workspace's device error word after the timed steps (a position
    # out of range, bad sequence offsets, or an in-launch merge that could not
    # prove its placement): nonzero means the timed outputs are not valid
    dev_err = {"prefill": qa.device_error(wl.pws), "decode": qa.device_error(wl.dws),
               "verify": qa.device_error(wl.vws)}
    K = args.steps
    ms_per_step = sum(per_step) / K
    pre_ms = phase["prefill"] / K
    dec_ms = phase["decode"] / K
    ver_us = phase["verify"] / K * 1e3

    B, Hq, Hkv, S, L, NS = wl.B, wl.Hq, wl.Hkv, wl.S, wl.L, wl.steps
    dec_us_step = dec_ms * 1e3 / NS
    step_bytes = sum(decode_bytes(B, Hq, Hkv, S + 1 + s) for s in range(NS)) \
        / NS * L
    dec_gbps = step_bytes / (dec_us_step * 1e-6) / 1e9
    pflops = prefill_flops(B, Hq, S)
    pre_tflops = pflops * L / (pre_ms * 1e-3) / 1e12

    # Live per-call durations from the timed region: a decode call is one
    # decode_kernel launch (B x Hkv = 32 pairs: partials merged inside it);
    # inside the captured step graph the calls
    # run back to back, so the phase time over (steps x layers) calls is the
    # average duration of one call on its stream (the position increment, one
    # tiny kernel per step, is included).
    dec_call_us = dec_us_step / L
    ctx_mean = S + 1 + (NS - 1) / 2.0
    dec_call_bytes = step_bytes / L
    dec_ach = dec_call_bytes / (dec_call_us * 1e-6) / 1e9
    pre_call_us = pre_ms * 1e3 / L
    pre_ach = pflops / (pre_call_us * 1e-6) / 1e12

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            t = json.load(f)
        if t.get("decode_source_sha") == build_info().get("decode_source_sha"):
            traffic = t.get("hbm_bytes_per_call")

    result = {
        "metric": METRIC,
        "value": round(dec_us_step, 3),
        "unit": "us/decode_step",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_4b_b4_s2048_36l", "batch": B,
                   "prompt_len": S, "decode_steps": NS, "layers": L,
                   "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": 128,
                   "verify": {"batch": wl.vB, "block": wl.vn,
                              "cache_slots": wl.vL0},
                   "parallelism": "none (1 GPU)"},
        "decode_us_per_step": round(dec_us_step, 3),
        "decode_GBps": round(dec_gbps, 1),
        "decode_frac_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "prefill_ms_36_layers": round(pre_ms, 4),
        "prefill_us_per_layer": round(pre_ms * 1e3 / L, 2),
        "prefill_TFLOPs": round(pre_tflops, 1),
        "prefill_frac_mfma_peak": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "verify_us": round(ver_us, 2),
        "roofline": {"kernel": "qa_decode call = decode_kernel<4,2,true> "
                               "(one launch, merge inside)", "bound": "hbm",
                     "achieved": round(dec_ach, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s",
                     "frac": round(dec_ach / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(dec_call_bytes),
                     "mean_context": ctx_mean,
                     "avg_launch_us": round(dec_call_us, 3),
                     "launches_timed": K * NS * L},
        "roofline_prefill": {"kernels": "qa_prefill call = kv_prologue_kernel"
                             " + prefill_attn_kernel<4>", "bound": "mfma",
                             "achieved": round(pre_ach, 1),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pre_ach / MFMA_BF16_PEAK_TFLOPS, 4),
                             "flops_per_launch": pflops,
                             "avg_launch_us": round(pre_call_us, 2)},
        "device_errors": dev_err,
        "wall_s_timed": round(wall, 3),
        "provenance": build_info(),
    }
    if not args.no_ragged:
        log("bench: ragged-batch latency spread (untimed)")
        result["ragged_spread"] = ragged_spread(torch, qa, W)
        log("bench: hidden-state RMSNorm, attention epilogue (untimed)")
        result["rmsnorm_hidden"] = rmsnorm_rate(torch, qa)
        result["attn_epilogue"] = epilogue_rate(torch, qa)
        log("bench: membw probe, rotated verify, small workloads, chunked prefill")
        probe = membw_probe(torch, qa)
        probe["decode_frac_of_probe"] = round(dec_ach / probe["GBps"], 4)
        result["membw_probe"] = probe
        result["verify_rotated"] = verify_rotated(torch, qa, W)
        result["latency_small"] = small_latency(torch, qa, W)
        result["chunked_prefill"] = chunked_prefill(torch, qa, W)
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (fp64 oracle, bounded sample)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)
    if any(dev_err.values()):
        log(f"bench: device error words are not zero: {dev_err}")
        sys.exit(3)


if __name__ == "__main__":
    main()
