"""CPU checks of the speculative-decoding loop's bookkeeping (acceptance,
bonus token, per-sequence lengths, cache rewind by overwrite) against plain
greedy decoding of a fake deterministic target."""

import numpy as np
import pytest
import torch

from prefill_attention_rmsnorm_amd import qa, specdec


def test_accepted_prefix():
    assert specdec.accepted_prefix([], []) == 0
    assert specdec.accepted_prefix([1, 2, 3], [1, 2, 3]) == 3
    assert specdec.accepted_prefix([1, 2, 3], [1, 5, 3]) == 1
    assert specdec.accepted_prefix([4], [1]) == 0


class FakeTarget:
    """A target whose greedy next token is a hash of the sequence so far.

    project() passes tokens through as q (one value per row); the fake
    verify writes them into a per-sequence slot table at start .. start+n-1,
    exactly where qa_verify writes K/V, and argmax() reads the slots
    0 .. position back, so a rejected draft left in the table would change
    the result if the loop ever read past its length."""

    V = 1000

    def __init__(self, B, cap):
        self.slots = np.full((B, cap), -1, dtype=np.int64)
        self.last = None

    def next_token(self, seq):
        h = 1469598103934665603
        for t in seq:
            h = ((h ^ int(t)) * 1099511628211) % (1 << 61)
        return h % self.V

    def project(self, toks):
        q = torch.tensor(toks, dtype=torch.float32)[..., None, None]
        q = q.expand(-1, -1, 1, qa.HEAD_DIM).contiguous()  # [B, n, 1, 128]
        return q, q, q

    def verify(self, cache, params, q, k, v, start, max_ctx, ws=None):
        B, n = q.shape[:2]
        st = start.tolist()
        for b in range(B):
            self.slots[b, st[b]:st[b] + n] = q[b, :, 0, 0].long().numpy()
        self.last = (st, n)
        return q, None, ws

    def argmax(self, o):
        st, n = self.last
        B = len(st)
        out = []
        for b in range(B):
            for i in range(n):
                seq = self.slots[b, :st[b] + i + 1]
                assert (seq >= 0).all(), "read an unwritten slot"
                out.append(self.next_token(seq))
        return out


@pytest.mark.parametrize("block", [1, 2, 5])
@pytest.mark.parametrize("quality", [0.0, 0.6, 1.0])
def test_loop_matches_plain_greedy(monkeypatch, block, quality):
    B, n_new = 3, 17
    prompts = [[5, 7, 9], [1], [2, 3, 4, 5, 6, 8]]
    tgt = FakeTarget(B, 64)
    for b, p in enumerate(prompts):
        tgt.slots[b, :len(p)] = p
    greedy = []
    for p in prompts:
        s = list(p)
        for _ in range(n_new):
            s.append(tgt.next_token(s))
        greedy.append(s[len(p):])
    rng = np.random.default_rng(int(quality * 10) + block)

    def drafter(b, emitted, k):  # each sequence drafts differently well
        i = len(emitted) + 1
        d = (greedy[b][i:i + k] + [0] * k)[:k]
        qb = quality if b != 1 else 1.0 - quality
        return [t if rng.random() < qb else (t + 1) % tgt.V for t in d]

    monkeypatch.setattr(qa, "verify", tgt.verify)
    monkeypatch.setattr(qa, "workspace", lambda *a, **kw: None)

    class P:
        class desc:
            n_q_heads = 1

    class C:
        n_kv_heads = 1

    lengths = [len(p) for p in prompts]
    nxt = [tgt.next_token(p) for p in prompts]
    out = specdec.speculative_generate(C, P, tgt.project, tgt.argmax, drafter,
                                       lengths, nxt, n_new, block, 64)
    assert out == greedy
    for b, p in enumerate(prompts):
        assert len(p) + n_new <= lengths[b] < len(p) + n_new + block
        assert list(tgt.slots[b, len(p):len(p) + n_new]) == greedy[b]
