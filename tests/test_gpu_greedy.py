"""Synthetic greedy check through a random-init LM head.

"dryft-flash-infer" agent guide, Invariants: every emitted token must be the
greedy choice on the engine's own prefix or lie within 2.0 logits of the
argmax there, judged by a teacher-forced replay.  Here the engine is the HIP
attention path (plus a torch fp32 LM head on the GPU as test plumbing) and
the replay is the fp64 oracle on the engine's own tokens.  The LM head maps
the attention output through W_o [Hq*128, 2560], a final RMSNorm and
W_lm [2560, vocab]; without the norm the logits would be ~0.05 wide and the
margin vacuous.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from prefill_attention_rmsnorm_amd import qa

from .gpu_helpers import EPS, THETA, LMHead, f64, new_cache, params, say

pytestmark = pytest.mark.gpu
SCALE = 1.0 / np.sqrt(128)
MARGIN = 2.0


def _judge(logits_ref, toks, what):
    margins, exact = [], 0
    for lr, t in zip(logits_ref, toks):
        gap = float(lr.max() - lr[int(t)])
        margins.append(gap)
        exact += int(oracle.argmax_lowest(lr) == int(t))
        assert oracle.margin_ok(lr, int(t), MARGIN), f"{what}: token {t} is {gap} below"
    say(f"  {what}: {exact}/{len(toks)} exact argmax, worst gap {max(margins):.4f}")
    return exact, max(margins)


def test_tiny_closed_loop():
    w = W.get("tiny")
    Hq, Hkv, D, V = w.n_q_heads, w.n_kv_heads, w.hidden, w.vocab
    S, steps, cap = w.prompt_lens[0], w.decode_steps, w.capacity
    say(f"greedy tiny: prompt {S}, {steps} decode steps, vocab {V}")
    emb = W.normal_bf16((V, D), 0, 0, 0, "emb")
    w_q = W.normal_bf16((D, Hq * 128), 0, 0, 0, "w_q", std=0.02).float()
    w_k = W.normal_bf16((D, Hkv * 128), 0, 0, 0, "w_k", std=0.02).float()
    w_v = W.normal_bf16((D, Hkv * 128), 0, 0, 0, "w_v", std=0.02).float()
    head = LMHead(0, Hq, D, V)
    ids = W.rng(0, 0, 0, "ids").integers(0, V, S)

    def project(tok_ids):
        hdn = emb[torch.from_numpy(np.asarray(tok_ids))].float()
        n = hdn.shape[0]
        return ((hdn @ w_q).to(torch.bfloat16).reshape(n, Hq, 128),
                (hdn @ w_k).to(torch.bfloat16).reshape(n, Hkv, 128),
                (hdn @ w_v).to(torch.bfloat16).reshape(n, Hkv, 128))

    p = params(Hq)
    cache = new_cache(1, Hkv, cap)
    oc = oracle.Cache.empty(1, Hkv, cap, 128)
    q, k, v = project(ids)
    cu, pos = W.packed_layout([S])
    out, _, _ = qa.prefill(cache, p, q.cuda(), k.cuda(), v.cuda(),
                           torch.from_numpy(cu).cuda(),
                           torch.from_numpy(pos).cuda(), S)
    ref, _, oc = oracle.prefill(oc, q.double().numpy(), k.double().numpy(),
                                v.double().numpy(), cu, pos, scale=SCALE,
                                theta=THETA, eps=EPS)
    tok = int(head.gpu_tokens(out[-1:])[0])
    toks, refs = [tok], [head.ref_logits(ref[-1:])[0]]
    ws = qa.workspace(qa.QA_OP_DECODE, 1, Hq, Hkv, cap)
    for s in range(steps):
        q, k, v = project([tok])
        P = np.array([S + s], dtype=np.int32)
        out, _, _ = qa.decode(cache, p, q.cuda(), k.cuda(), v.cuda(),
                              torch.from_numpy(P).cuda(), cap, ws=ws)
        ref, _, oc = oracle.decode(oc, q.double().numpy(), k.double().numpy(),
                                   v.double().numpy(), P, scale=SCALE,
                                   theta=THETA, eps=EPS)
        tok = int(head.gpu_tokens(out)[0])
        toks.append(tok)
        refs.append(head.ref_logits(ref)[0])
    _judge(refs, toks, "tiny closed loop")


def test_verify_block_lm_margin():
    w = W.get(4)
    B, Hq, Hkv, n, L0, cap = (w.batch, w.n_q_heads, w.n_kv_heads,
                              w.verify_block, w.verify_start, w.capacity)
    say(f"greedy verify: B={B} block {n} after {L0} slots")
    cache = new_cache(B, Hkv, cap)
    oc = oracle.Cache.empty(B, Hkv, cap, 128)
    kk = W.normal_bf16((B, Hkv, L0, 128), 4, 0, 0, "cache_k")
    vv = W.normal_bf16((B, Hkv, L0, 128), 4, 0, 0, "cache_v")
    cache.k[:, :, :L0] = kk.cuda()
    cache.v[:, :, :L0] = vv.cuda()
    oc.k[:, :, :L0] = kk.double().numpy()
    oc.v[:, :, :L0] = vv.double().numpy()
    q = W.normal_bf16((B, n, Hq, 128), 4, 0, 0, "q")
    k = W.normal_bf16((B, n, Hkv, 128), 4, 0, 0, "k")
    v = W.normal_bf16((B, n, Hkv, 128), 4, 0, 0, "v")
    out, _, _ = qa.verify(cache, params(Hq), q.cuda(), k.cuda(), v.cuda(),
                          torch.full((B,), L0, dtype=torch.int32,
                                     device="cuda"), cap)
    ref, _, _ = oracle.verify(oc, q.double().numpy(), k.double().numpy(),
                              v.double().numpy(), [L0] * B, scale=SCALE,
                              theta=THETA, eps=EPS)
    head = LMHead(4, Hq, w.hidden, w.vocab)
    toks = head.gpu_tokens(out.reshape(B * n, Hq, 128))
    refs = head.ref_logits(ref.reshape(B * n, Hq, 128))
    _judge(refs, toks, "verify block")
