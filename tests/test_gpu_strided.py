"""GPU parity on KV caches that are not densely packed ("dryft-flash-infer"
agent guide, Where the wins are: a preallocated, correctly strided cache).

The cache is a strided view [B, Hkv, cap, 128] over a larger buffer: a padded
slot pitch and head pitch, a token-major buffer [B, cap, Hkv, 128] and a
slot-major one [cap, B, Hkv, 128].  Prefill, decode steps and a verify block
run on the view and are compared with the oracle; the cache bytes must equal
the oracle's and every byte of the buffer outside the view must keep its
sentinel."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import (EPS, NAN_BITS, THETA, bits, check_cache, compare, f64,
                          params, say, seq_index)

pytestmark = pytest.mark.gpu
PAD_BITS = 0x7FC3  # a second NaN pattern for bytes outside the view
SCALE = 1.0 / np.sqrt(128)


def _strided(layout, B, Hkv, cap):
    """(buffer_k, buffer_v, view_k, view_v) for one layout."""
    def buf(shape):
        return torch.full(shape, PAD_BITS, dtype=torch.int16,
                          device="cuda").view(torch.bfloat16)
    if layout == "padded":      # slot pitch 192, 3 spare slots per head
        bk, bv = buf((B, Hkv, cap + 3, 192)), buf((B, Hkv, cap + 3, 192))
        vk, vv = bk[:, :, :cap, :128], bv[:, :, :cap, :128]
    elif layout == "token_major":
        bk, bv = buf((B, cap, Hkv, 128)), buf((B, cap, Hkv, 128))
        vk, vv = bk.permute(0, 2, 1, 3), bv.permute(0, 2, 1, 3)
    elif layout == "slot_major":
        bk, bv = buf((cap, B, Hkv, 128)), buf((cap, B, Hkv, 128))
        vk, vv = bk.permute(1, 2, 0, 3), bv.permute(1, 2, 0, 3)
    else:
        raise ValueError(layout)
    vk.view(torch.int16).fill_(NAN_BITS)
    vv.view(torch.int16).fill_(NAN_BITS)
    return bk, bv, vk, vv


@pytest.mark.parametrize("layout", ["padded", "token_major", "slot_major"])
def test_strided_cache_prefill_decode_verify(layout):
    B, Hq, Hkv, cap = 3, 16, 4, 400
    lens = [300, 129, 64]
    seed = 60
    say(f"strided cache: layout={layout} B={B} Hq={Hq} Hkv={Hkv} cap={cap}")
    bk, bv, vk, vv = _strided(layout, B, Hkv, cap)
    cache = qa.Cache(vk, vv)
    if layout != "padded":
        assert cache.desc.stride_h != cap * 128  # not the dense descriptor
    oc = oracle.Cache.empty(B, Hkv, cap, 128)
    p = params(Hq)

    # prefill
    T = sum(lens)
    q = W.normal_bf16((T, Hq, 128), seed, 0, 0, "q")
    k = W.normal_bf16((T, Hkv, 128), seed, 0, 0, "k")
    v = W.normal_bf16((T, Hkv, 128), seed, 0, 0, "v")
    cu, pos = W.packed_layout(lens)
    out, _, ws = qa.prefill(cache, p, q.cuda(), k.cuda(), v.cuda(),
                            torch.from_numpy(cu).cuda(),
                            torch.from_numpy(pos).cuda(), max(lens))
    assert qa.device_error(ws) == 0
    ref, _, oc = oracle.prefill(oc, q.double().numpy(), k.double().numpy(),
                                v.double().numpy(), cu, pos, scale=SCALE,
                                theta=THETA, eps=EPS)
    compare(f64(out), ref, f"{layout} prefill")

    # decode steps
    dpos = np.array(lens, dtype=np.int32)
    dws = qa.workspace(qa.QA_OP_DECODE, B, Hq, Hkv, cap)
    for s in range(3):
        dq = W.normal_bf16((B, Hq, 128), seed, 1, s, "q")
        dk = W.normal_bf16((B, Hkv, 128), seed, 1, s, "k")
        dv = W.normal_bf16((B, Hkv, 128), seed, 1, s, "v")
        o, _, _ = qa.decode(cache, p, dq.cuda(), dk.cuda(), dv.cuda(),
                            torch.from_numpy(dpos).cuda(), cap, ws=dws)
        r, _, oc = oracle.decode(oc, dq.double().numpy(), dk.double().numpy(),
                                 dv.double().numpy(), dpos, scale=SCALE,
                                 theta=THETA, eps=EPS)
        compare(f64(o), r, f"{layout} decode step {s}")
        dpos = dpos + 1
    assert qa.device_error(dws) == 0

    # verify block
    n = 8
    vq = W.normal_bf16((B, n, Hq, 128), seed, 2, 0, "q")
    vk_ = W.normal_bf16((B, n, Hkv, 128), seed, 2, 0, "k")
    vv_ = W.normal_bf16((B, n, Hkv, 128), seed, 2, 0, "v")
    o, _, vws = qa.verify(cache, p, vq.cuda(), vk_.cuda(), vv_.cuda(),
                          torch.from_numpy(dpos).cuda(), cap)
    assert qa.device_error(vws) == 0
    r, _, oc = oracle.verify(oc, vq.double().numpy(), vk_.double().numpy(),
                             vv_.double().numpy(), dpos, scale=SCALE,
                             theta=THETA, eps=EPS)
    compare(f64(o), r, f"{layout} verify")

    check_cache(cache, oc, f"{layout} cache view")
    # nothing outside the view was touched
    inside = torch.zeros(bk.shape, dtype=torch.bool, device="cuda")
    if layout == "padded":
        inside[:, :, :cap, :128] = True
    else:
        inside[:] = True
    for buf in (bk, bv):
        outside = bits(buf)[~inside.cpu().numpy()]
        assert (outside == PAD_BITS).all(), f"{layout}: a byte outside the view changed"
