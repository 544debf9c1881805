"""Debug mode and guard bands around outputs and workspaces.

Fail-closed checking (pegainfer PR #862, review thread):
- Debug mode (`qa_set_debug`, or QA_DEBUG=1 in the environment) makes every
  call synchronise and return QA_ERR_DEVICE when a kernel set a device error
  bit, instead of leaving the caller to read the error word.
- Guard bands: every output and workspace of a call is placed in the middle
  of a larger allocation whose margins hold a NaN pattern no kernel writes;
  after the call the margins must be bit-for-bit what they were.  This checks
  that no kernel writes outside the buffers it was given.
"""

import numpy as np
import pytest
import torch

import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import EPS, params, say

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements on each side (keeps 16-byte alignment for any dtype)
PATTERN = {torch.bfloat16: (torch.int16, 0x7FB5),
           torch.float32: (torch.int32, 0x7FB5A5A5),
           torch.uint8: (torch.uint8, 0xA5)}


def guarded(shape, dtype):
    """(full, inner): inner, of `shape`, sits between two margins of GUARD
    elements holding PATTERN[dtype]."""
    n = int(np.prod(shape))
    full = torch.empty(n + 2 * GUARD, dtype=dtype, device="cuda")
    view_t, pat = PATTERN[dtype]
    full.view(view_t).fill_(pat)
    return full, full[GUARD:GUARD + n].view(shape)


def check_guards(full, inner, what):
    torch.cuda.synchronize()
    view_t, pat = PATTERN[full.dtype]
    raw = full.view(view_t)
    n = inner.numel()
    for side, part in (("front", raw[:GUARD]), ("back", raw[GUARD + n:])):
        bad = int((part != pat).sum())
        assert bad == 0, f"{what}: {bad} guard elements overwritten ({side})"


def guarded_ws(op, B, Hq, Hkv, max_ctx, block_len=0):
    n = qa.workspace_bytes(op, B, Hq, Hkv, max_ctx, block_len)
    full, inner = guarded((n,), torch.uint8)
    qa._check(qa.lib().qa_workspace_init(qa._ptr(inner), n, None))
    return full, inner


def _prompts(B, Hq, Hkv, S, seed):
    T = B * S
    q = W.normal_bf16((T, Hq, 128), seed, 0, 0, "q").cuda()
    k = W.normal_bf16((T, Hkv, 128), seed, 0, 0, "k").cuda()
    v = W.normal_bf16((T, Hkv, 128), seed, 0, 0, "v").cuda()
    cu = torch.arange(0, T + 1, S, dtype=torch.int32, device="cuda")
    pos = torch.arange(S, dtype=torch.int32, device="cuda").repeat(B)
    return q, k, v, cu, pos


def test_guard_bands_every_entry_point():
    """Prefill (two q-tiles per pair and a ragged tail), decode with the merge
    inside the launch (8 pairs) and with the merge kernel (6 pairs), verify on
    the four-stage ring, the hidden-state norm and both epilogue kernels, each
    with its outputs and workspace inside guard bands."""
    for B, Hkv in ((4, 2), (3, 2)):
        Hq, S, cap = 8, 300, 320
        say(f"guards: prefill/decode/verify B={B} Hkv={Hkv} S={S}")
        cache = qa.Cache.empty(B, Hkv, cap)
        p = params(Hq)
        q, k, v, cu, pos = _prompts(B, Hq, Hkv, S, 90 + B)
        fo, out = guarded((B * S, Hq, 128), torch.bfloat16)
        fl, lse = guarded((B * S, Hq), torch.float32)
        fw, ws = guarded_ws(qa.QA_OP_PREFILL, B, Hq, Hkv, B * S)
        qa.prefill(cache, p, q, k, v, cu, pos, S, out=out, lse=lse, ws=ws)
        for f, t, w in ((fo, out, "prefill out"), (fl, lse, "prefill lse"),
                        (fw, ws, "prefill ws")):
            check_guards(f, t, w)
        assert qa.device_error(ws) == 0

        dq = W.normal_bf16((B, Hq, 128), 95, 0, 0, "q").cuda()
        dk = W.normal_bf16((B, Hkv, 128), 95, 0, 0, "k").cuda()
        dv = W.normal_bf16((B, Hkv, 128), 95, 0, 0, "v").cuda()
        dpos = torch.full((B,), S, dtype=torch.int32, device="cuda")
        fo, out = guarded((B, Hq, 128), torch.bfloat16)
        fl, lse = guarded((B, Hq), torch.float32)
        fw, ws = guarded_ws(qa.QA_OP_DECODE, B, Hq, Hkv, cap)
        for _ in range(3):  # the in-launch merge's counters sit at the workspace end
            qa.decode(cache, p, dq, dk, dv, dpos, cap, out=out, lse=lse, ws=ws)
        for f, t, w in ((fo, out, "decode out"), (fl, lse, "decode lse"),
                        (fw, ws, "decode ws")):
            check_guards(f, t, w)
        assert qa.device_error(ws) == 0

        n = 16
        vq = W.normal_bf16((B, n, Hq, 128), 96, 0, 0, "q").cuda()
        vk = W.normal_bf16((B, n, Hkv, 128), 96, 0, 0, "k").cuda()
        vv = W.normal_bf16((B, n, Hkv, 128), 96, 0, 0, "v").cuda()
        st = torch.full((B,), S, dtype=torch.int32, device="cuda")
        fo, out = guarded((B, n, Hq, 128), torch.bfloat16)
        fl, lse = guarded((B, n, Hq), torch.float32)
        fw, ws = guarded_ws(qa.QA_OP_VERIFY, B, Hq, Hkv, cap, n)
        qa.verify(cache, p, vq, vk, vv, st, cap, out=out, lse=lse, ws=ws)
        for f, t, w in ((fo, out, "verify out"), (fl, lse, "verify lse"),
                        (fw, ws, "verify ws")):
            check_guards(f, t, w)
        assert qa.device_error(ws) == 0

    for T in (4, 300, 600):  # the streaming kernel, the GEMM; both norm kernels
        say(f"guards: epilogue and norm T={T}")
        o = W.normal_bf16((T, 1024), 97, 0, 0, "hidden_x").cuda()
        w_o = W.normal_bf16((512, 1024), 97, 0, 0, "w_o", std=0.02).cuda()
        fr, res = guarded((T, 512), torch.bfloat16)
        res.copy_(W.normal_bf16((T, 512), 97, 0, 0, "hidden_res").cuda())
        fo, out = guarded((T, 512), torch.bfloat16)
        qa.attn_epilogue(o, w_o, res, None, EPS, out=out)
        check_guards(fr, res, "epilogue residual")
        check_guards(fo, out, "epilogue out")
        fo2, out2 = guarded((T, 512), torch.bfloat16)
        qa.rmsnorm_hidden(out, residual=res, eps=EPS, out=out2)
        check_guards(fo2, out2, "rmsnorm out")
        check_guards(fr, res, "rmsnorm residual")


def test_debug_mode_turns_device_errors_into_status():
    B, Hq, Hkv, cap = 2, 4, 1, 16
    cache = qa.Cache.empty(B, Hkv, cap)
    p = params(Hq)
    q = W.normal_bf16((B, Hq, 128), 98, 0, 0, "q").cuda()
    k = W.normal_bf16((B, Hkv, 128), 98, 0, 0, "k").cuda()
    v = W.normal_bf16((B, Hkv, 128), 98, 0, 0, "v").cuda()
    good = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    bad = torch.tensor([0, 16], dtype=torch.int32, device="cuda")  # past the cache
    qa.set_debug(True)
    try:
        ws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)
        qa.decode(cache, p, q, k, v, good, cap, ws=ws)  # clean: no error
        with pytest.raises(qa.QaError) as e:
            qa.decode(cache, p, q, k, v, bad, cap, ws=ws)
        assert "QA_ERR_DEVICE" in str(e.value) and "0x1" in str(e.value)
        # the word is left set for the caller; reading it clears it
        assert qa.device_error(ws) & qa.QA_DEVERR_POSITION
        qa.decode(cache, p, q, k, v, good, cap, ws=ws)
        # calls without an error word check only for HIP errors
        x = W.normal_bf16((3, 256), 98, 0, 0, "hidden_x").cuda()
        qa.rmsnorm_hidden(x, eps=EPS)
    finally:
        qa.set_debug(False)
    # debug mode off: the same bad call returns OK and only sets the word
    qa.decode(cache, p, q, k, v, bad, cap, ws=ws)
    assert qa.device_error(ws) & qa.QA_DEVERR_POSITION
