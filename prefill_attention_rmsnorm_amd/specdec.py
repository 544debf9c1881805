"""Exact speculative decoding around qa_verify (host-side loop).

"dryft-flash-infer" agent guide, Where the wins are (speculative decoding with
exact verification): a cheap drafter proposes tokens, the target model checks
a whole block of them in one pass, and only the tokens the target itself
would have chosen greedily are kept, so the output is the target's greedy
sequence whatever the drafter proposes.  The cache rewind is the caller's
(qa.h, qa_verify): rejected draft slots are simply overwritten later, since
every call writes a slot before any query reads it.

Per sequence b the loop keeps a length L_b (slots 0..L_b-1 of its cache row
hold the accepted tokens) and the target's greedy choice `nxt_b` for position
L_b, not yet in the cache.  One step:

1. block_b = [nxt_b, d_1, ..., d_{k-1}] (the drafter's k-1 proposals);
2. one qa_verify call writes the block's K/V at L_b .. L_b+k-1 and returns
   the attention output of every block position;
3. the target's greedy token after block position i is g_i (i < k);
4. a_b = the longest prefix with d_{i+1} == g_i; tokens nxt_b, d_1..d_{a_b}
   are accepted, and g_{a_b} becomes the new nxt_b (after a full accept, the
   bonus token);
5. L_b += a_b + 1.

The model around the attention (embedding and q/k/v projections, the layers
after attention, the LM head) is supplied by the caller as callables; this
module only runs the loop and the verify calls.
"""

from __future__ import annotations

from typing import Callable, List, Sequence

import torch

from . import qa


def accepted_prefix(draft: Sequence[int], target: Sequence[int]) -> int:
    """Largest a with draft[i] == target[i] for every i < a."""
    a = 0
    for d, t in zip(draft, target):
        if int(d) != int(t):
            break
        a += 1
    return a


def speculative_generate(cache: qa.Cache, params: qa.Params,
                         project: Callable, argmax: Callable,
                         drafter: Callable, lengths: List[int],
                         nxt: List[int], n_new: int, block: int,
                         max_ctx: int) -> List[List[int]]:
    """Generate n_new tokens per sequence by speculative blocks of `block`.

    cache/params: the target's KV cache (rows 0..B-1) and attention params.
    project(tokens [B][n]) -> (q, k, v) bf16 device tensors [B, n, H, 128]
      for the given tokens (their positions are implied by the cache state).
    argmax(out [B*n, Hq, 128]) -> list of B*n target tokens (greedy).
    drafter(b, emitted_b, k) -> k proposed tokens for sequence b.
    lengths[b]: slots already in the cache; nxt[b]: the target's greedy token
      for slot lengths[b].  Both lists are updated in place.
    Returns the tokens emitted per sequence (n_new each; the first is nxt).
    A sequence that has its n_new tokens stays in the batched verify calls
    until the others finish, without advancing, so max_ctx must cover the
    longest prompt + n_new + 2 * block - 1 slots.
    """
    B = len(lengths)
    if block < 1 or len(nxt) != B:
        raise ValueError("block >= 1 and one pending token per sequence")
    out_tokens: List[List[int]] = [[] for _ in range(B)]
    ws = qa.workspace(qa.QA_OP_VERIFY, B, params.desc.n_q_heads, cache.n_kv_heads,
                      max_ctx, block)
    while min(len(t) for t in out_tokens) < n_new:
        drafts = [list(drafter(b, out_tokens[b], block - 1))[:block - 1]
                  for b in range(B)]
        for d in drafts:
            if len(d) != block - 1:
                raise ValueError("the drafter must propose block - 1 tokens")
        blocks = [[nxt[b]] + drafts[b] for b in range(B)]
        if max(lengths) + block > max_ctx:
            raise ValueError("block would pass max_ctx")
        q, k, v = project(blocks)
        start = torch.tensor(lengths, dtype=torch.int32, device=q.device)
        o, _, _ = qa.verify(cache, params, q, k, v, start, max_ctx, ws=ws)
        g = argmax(o.reshape(B * block, params.desc.n_q_heads, qa.HEAD_DIM))
        for b in range(B):
            if len(out_tokens[b]) >= n_new:
                continue  # finished: its block sits past its length, unused
            gb = [int(x) for x in g[b * block:(b + 1) * block]]
            a = accepted_prefix(drafts[b], gb)
            out_tokens[b].extend(blocks[b][:a + 1])
            lengths[b] += a + 1
            nxt[b] = gb[a]
    return [t[:n_new] for t in out_tokens]
