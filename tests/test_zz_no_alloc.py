"""qa_decode_noalloc (decode on the library's own scratch array, for callers
that cannot allocate) against qa_decode with a workspace: the same kernels,
so outputs, LSE and cache bytes must be bit-identical.  Several calls in a
row share the one array: a full B=4 x 2048 step, then smaller inputs (fewer
splits, and a batch whose partials go through the merge kernel), then the
first case again, which also shows the merge counters came back to zero."""

import numpy as np
import pytest
import torch

import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import bits, new_cache, params, say

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, cap, lens, seed, max_ctx=None):
    say(f"no-alloc case: B={B} Hq={Hq} Hkv={Hkv} cap={cap} lens={lens}")
    max_ctx = max_ctx or cap
    ca, cb = new_cache(B, Hkv, cap), new_cache(B, Hkv, cap)
    for b, L in enumerate(lens):
        kk = W.normal_bf16((Hkv, L, 128), seed, b, 0, "cache_k").cuda()
        vv = W.normal_bf16((Hkv, L, 128), seed, b, 0, "cache_v").cuda()
        for c in (ca, cb):
            c.k[b, :, :L] = kk
            c.v[b, :, :L] = vv
    q = W.normal_bf16((B, Hq, 128), seed, 1, 0, "q").cuda()
    k = W.normal_bf16((B, Hkv, 128), seed, 1, 0, "k").cuda()
    v = W.normal_bf16((B, Hkv, 128), seed, 1, 0, "v").cuda()
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    p = params(Hq)
    lse_a = torch.empty((B, Hq), device="cuda")
    ref, _, ws = qa.decode(ca, p, q, k, v, pos, max_ctx, lse=lse_a)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse_b = torch.full((B, Hq), float("nan"), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    qa.decode_noalloc(cb, p, q, k, v, pos, max_ctx, out, lse=lse_b, dev_err=err)
    torch.cuda.synchronize()
    assert qa.device_error(ws) == 0
    assert int(err.item()) == 0
    assert np.array_equal(bits(out), bits(ref))
    assert torch.equal(lse_a, lse_b)
    assert np.array_equal(bits(ca.k), bits(cb.k))
    assert np.array_equal(bits(ca.v), bits(cb.v))


def test_noalloc_matches_decode_calls_in_a_row():
    w = W.get(2)
    big = (w.batch, w.n_q_heads, w.n_kv_heads, w.capacity, [2048, 2047, 1500, 3], 110)
    _case(*big)                                      # 32 pairs: merged in the launch
    _case(2, 32, 8, 300, [250, 17], 111)             # smaller: 16 pairs, fewer splits
    _case(3, 8, 2, 200, [150, 0, 199], 112)          # 6 pairs: merge kernel
    _case(*big)                                      # counters back at zero


def test_noalloc_reports_device_errors():
    B, Hq, Hkv, cap = 4, 8, 2, 64
    cache = new_cache(B, Hkv, cap)
    for b in range(B):
        cache.k[b, :, :10] = W.normal_bf16((Hkv, 10, 128), 113, b, 0, "cache_k").cuda()
        cache.v[b, :, :10] = W.normal_bf16((Hkv, 10, 128), 113, b, 0, "cache_v").cuda()
    q = W.normal_bf16((B, Hq, 128), 113, 1, 0, "q").cuda()
    k = W.normal_bf16((B, Hkv, 128), 113, 1, 0, "k").cuda()
    v = W.normal_bf16((B, Hkv, 128), 113, 1, 0, "v").cuda()
    pos = torch.tensor([10, 10, 64, 10], dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    qa.decode_noalloc(cache, params(Hq), q, k, v, pos, cap, out, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & qa.QA_DEVERR_POSITION
    assert torch.count_nonzero(out[2].float()) == 0
    assert torch.isfinite(out.float()).all()


def test_noalloc_rejects_oversized_layout():
    # B=64 x 8 kv heads at 32768 slots needs ~137 MB of partials: refused on
    # the host with QA_ERR_WORKSPACE, nothing launched
    c = qa.QaCache()
    assert qa.lib().qa_cache_alloc(qa.ctypes.byref(c), 64, 8, 32768, 128, qa.ctypes.c_void_p(0x10000),
                                   qa.ctypes.c_void_p(0x20000)) == 0
    p = qa.QaParams(32, 0.088, 1e6, 1e-6, None, None)
    f = qa.ctypes.c_void_p(0x30000)
    st = qa.lib().qa_decode_noalloc(qa.ctypes.byref(c), qa.ctypes.byref(p), f, f, f, f,
                                    64, 32768, f, None, None, None)
    assert st == -6, qa.lib().qa_last_error()
    assert b"16777216" in qa.lib().qa_last_error()
