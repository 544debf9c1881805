"""Plain fp64 definition of the GQA attention path (TEST INFRASTRUCTURE ONLY).

Nothing here is tiled, fused or reordered beyond what the definitions state;
library matmuls serve only as the dot-product step.  Every function names the
page passage it follows.  See the package docstring for what pins each one.

Shapes use the pages' problem statement ("htn.dryft.ai/docs", *What to
submit*): a batch of token sequences, each owning one row of a preallocated
cache ("dryft-flash-infer" agent guide, *Where the wins are*: "KV cache
layout").  Cache layout: [batch, kv_head, slot, head_dim], slot = absolute
position of the token.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even), done directly from fp64 so
# that no intermediate fp32 rounding can happen (double rounding would differ
# from a single RNE at about one value in 2^29).
# ---------------------------------------------------------------------------

_BF16_MIN_EXP = -133  # quantum of bf16 subnormals: 2^-126 * 2^-7


def bf16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even.

    Returns fp64 values that are exactly representable in bf16.  NaN stays
    NaN, +-inf stay, magnitudes that round past the largest finite bf16
    become inf (IEEE overflow under round-to-nearest).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    if np.any(fin):
        xf = x[fin]
        _, e = np.frexp(xf)  # xf = m * 2^e, 0.5 <= |m| < 1
        # 8 significant bits for normals; fixed quantum for subnormals
        qexp = np.maximum(e.astype(np.int64) - 8, _BF16_MIN_EXP)
        scaled = np.ldexp(xf, -qexp)  # exact: power-of-two scaling
        r = np.ldexp(np.round(scaled), qexp)  # np.round: half to even
        r = np.where(np.abs(r) >= 2.0**128, np.copysign(np.inf, r), r)
        out[fin] = r
    return out


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of ``bf16_round(x)`` (NaN -> 0x7FC0 | sign)."""
    r = bf16_round(x)
    with np.errstate(invalid="ignore", over="ignore"):
        f = r.astype(np.float32)  # exact for bf16-representable values
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(r)
    if np.any(nan):
        sign = (np.signbit(r[nan]).astype(np.uint16)) << 15
        bits[nan] = np.uint16(0x7FC0) | sign
    return bits


def bits_to_f64(bits) -> np.ndarray:
    """fp64 values of bf16 bit patterns (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Prologue: per-head RMSNorm, then rotary embedding.
# "dryft-flash-infer" agent guide, *Where the wins are* ("Fused kernels":
# RMSNorm and rotary embedding).  The forms are those of the pinned Qwen3
# implementation the guide's *intro* names (per-head q/k norm, rotate-half
# rotary with frequencies theta^(-2i/d)); the pages do not print them.
# ---------------------------------------------------------------------------


def rmsnorm(x, weight=None, eps: float = 1e-6) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * weight over the last axis (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """Rotation frequencies theta^(-2i/d), i = 0 .. d/2-1."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -(2.0 * i) / d)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding at absolute position(s) ``pos``.

    Pairs (i, i + d/2) turn by angle a_i = pos * theta^(-2i/d):
    x'[i] = x[i] cos a_i - x[i+d/2] sin a_i,
    x'[i+d/2] = x[i+d/2] cos a_i + x[i] sin a_i.
    ``pos`` broadcasts against x's leading axes.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    p = np.asarray(pos, dtype=np.float64)[..., None]
    a = p * rope_inv_freq(d, theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ---------------------------------------------------------------------------
# Attention: dense exact causal softmax attention ("dryft-flash-infer" agent
# guide, *Where the wins are*: no eviction, no approximate or sparse
# attention).
# ---------------------------------------------------------------------------


def attend_rows(q, K, V, scale: float, n_visible):
    """Softmax attention of query rows over the first ``n_visible[r]`` keys.

    q [n, d], K [m, d], V [m, d]; row r sees keys 0 .. n_visible[r]-1.
    Returns o [n, d] = sum_j softmax_j(scale q.K_j) V_j and the natural-log
    log-sum-exp of the scaled scores, lse [n].
    """
    q = np.asarray(q, dtype=np.float64)
    n_visible = np.asarray(n_visible, dtype=np.int64)
    if q.shape[0] == 0:
        return np.zeros((0, q.shape[1])), np.zeros((0,))
    if np.any(n_visible < 1):
        raise ValueError("every query must see at least one key")
    mv = int(n_visible.max())
    Kv = np.asarray(K, dtype=np.float64)[:mv]
    Vv = np.asarray(V, dtype=np.float64)[:mv]
    if np.isnan(Kv).any() or np.isnan(Vv).any():
        raise ValueError("a visible cache slot was never written")
    s = scale * (q @ Kv.T)
    vis = np.arange(mv)[None, :] < n_visible[:, None]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    o = (e @ Vv) / den
    lse = (m + np.log(den))[:, 0]
    return o, lse


@dataclass
class Cache:
    """Preallocated KV cache in fp64, NaN marking unwritten slots.

    k, v: [batch, n_kv_heads, capacity, head_dim].  Written entries hold
    bf16-representable values: what the cache stores and what a reader sees.
    """

    k: np.ndarray
    v: np.ndarray

    @staticmethod
    def empty(batch, n_kv_heads, capacity, head_dim) -> "Cache":
        shape = (batch, n_kv_heads, capacity, head_dim)
        return Cache(np.full(shape, np.nan), np.full(shape, np.nan))

    def copy(self) -> "Cache":
        return Cache(self.k.copy(), self.v.copy())


def _prologue_k(k, pos, theta, eps, k_w):
    """k' = RoPE(RMSNorm(k)) in fp64, then one RNE to bf16 for the cache."""
    return bf16_round(rope(rmsnorm(k, k_w, eps), pos, theta))


def write_kv(cache: Cache, k, v, seq, pos, *, theta, eps, k_w=None):
    """Cache writes of a call: K[seq[t], :, pos[t]] = bf16(k'), V = v.

    k/v [T, Hkv, d].  Returns the new cache (the input is not modified).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    cap = cache.k.shape[2]
    if len(pos) and (pos.min() < 0 or pos.max() >= cap):
        raise ValueError("position outside the cache")
    c = cache.copy()
    kp = _prologue_k(k, pos[:, None], theta, eps, k_w)  # [T, Hkv, d]
    for t in range(len(pos)):
        c.k[seq[t], :, pos[t]] = kp[t]
        c.v[seq[t], :, pos[t]] = v[t]
    return c


def attend_tokens(cache: Cache, q, seq, pos, *, scale, theta, eps, q_w=None,
                  rows=None):
    """Attention of tokens over the cache: token t, head h sees slots
    0..pos[t] of row seq[t], KV head h // G.

    q [T, Hq, d].  ``rows`` optionally restricts the work to a list of
    (t, h) pairs (the other outputs stay zero).  Returns out [T, Hq, d] and
    lse [T, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    T, Hq, d = q.shape
    Hkv = cache.k.shape[1]
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    G = Hq // Hkv
    out = np.zeros((T, Hq, d))
    lse = np.zeros((T, Hq))
    if rows is None:
        qp = rope(rmsnorm(q, q_w, eps), pos[:, None], theta)  # [T, Hq, d]
        for b in np.unique(seq):
            idx = np.nonzero(seq == b)[0]
            for h in range(Hq):
                o, l = attend_rows(qp[idx, h], cache.k[b, h // G],
                                   cache.v[b, h // G], scale, pos[idx] + 1)
                out[idx, h] = o
                lse[idx, h] = l
        return out, lse
    for t, h in rows:
        qp = rope(rmsnorm(q[t, h], q_w, eps), pos[t], theta)
        b = seq[t]
        o, l = attend_rows(qp[None], cache.k[b, h // G], cache.v[b, h // G],
                           scale, [pos[t] + 1])
        out[t, h] = o[0]
        lse[t, h] = l[0]
    return out, lse


def _forward(cache: Cache, q, k, v, seq, pos, *, scale, theta, eps,
             q_w=None, k_w=None):
    """Shared body of prefill / decode / verify for a flat list of tokens.

    Token t belongs to cache row seq[t] at slot pos[t].  All K/V writes of the
    call happen first, then every token attends to slots 0..pos[t] of its row
    (the cache holds post-RoPE K; V is neither normalised nor rotated).
    q [T, Hq, d], k/v [T, Hkv, d].  Returns (out [T, Hq, d], lse [T, Hq],
    new cache).
    """
    c = write_kv(cache, k, v, seq, pos, theta=theta, eps=eps, k_w=k_w)
    out, lse = attend_tokens(c, q, seq, pos, scale=scale, theta=theta,
                             eps=eps, q_w=q_w)
    return out, lse, c


def prefill(cache: Cache, q, k, v, cu_seqlens, positions, *, scale, theta,
            eps=1e-6, q_w=None, k_w=None):
    """Prompt prefill of a packed batch.

    "dryft-flash-infer" agent guide, *Where the wins are* ("Prefill").
    Sequence i owns tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 and cache row i;
    ``positions`` gives each token's absolute position (its cache slot).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    seq = np.zeros(T, dtype=np.int64)
    for i in range(len(cu) - 1):
        seq[cu[i]:cu[i + 1]] = i
    return _forward(cache, q, k, v, seq, positions, scale=scale, theta=theta,
                    eps=eps, q_w=q_w, k_w=k_w)


def decode(cache: Cache, q, k, v, positions, *, scale, theta, eps=1e-6,
           q_w=None, k_w=None):
    """One cached decode step: one new token per sequence at positions[b].

    "dryft-flash-infer" agent guide, *Invariants* (one token per sequence per
    step) and *Where the wins are* ("Per-step overhead", "KV cache layout").
    q [B, Hq, d], k/v [B, Hkv, d].
    """
    B = np.asarray(q).shape[0]
    return _forward(cache, q, k, v, np.arange(B), positions, scale=scale,
                    theta=theta, eps=eps, q_w=q_w, k_w=k_w)


def verify(cache: Cache, q, k, v, start_pos, *, scale, theta, eps=1e-6,
           q_w=None, k_w=None):
    """Exact verification of an n-token draft block per sequence.

    "dryft-flash-infer" agent guide, *Where the wins are* ("Speculative
    decoding with exact verification").  Token i of sequence b sits at
    position start_pos[b] + i and sees slots 0 .. start_pos[b] + i.
    q [B, n, Hq, d], k/v [B, n, Hkv, d].  Returns out [B, n, Hq, d],
    lse [B, n, Hq] and the new cache.
    """
    q = np.asarray(q, dtype=np.float64)
    B, n = q.shape[:2]
    start = np.asarray(start_pos, dtype=np.int64)
    seq = np.repeat(np.arange(B), n)
    pos = (start[:, None] + np.arange(n)[None, :]).reshape(-1)
    out, lse, c = _forward(
        cache, q.reshape(B * n, *q.shape[2:]),
        np.asarray(k, dtype=np.float64).reshape(B * n, *np.shape(k)[2:]),
        np.asarray(v, dtype=np.float64).reshape(B * n, *np.shape(v)[2:]),
        seq, pos, scale=scale, theta=theta, eps=eps, q_w=q_w, k_w=k_w)
    return out.reshape(B, n, *out.shape[1:]), lse.reshape(B, n, -1), c


# ---------------------------------------------------------------------------
# Greedy check.  "dryft-flash-infer" agent guide, *Invariants* (each token is
# the greedy choice on the engine's own prefix or within 2.0 logits of the
# argmax there) and *Numerics* (how the 2.0 margin was calibrated).
# ---------------------------------------------------------------------------


def lm_logits(o_flat, W_o, W_lm, eps: float = 1e-6, chunk: int = 16384):
    """logits = RMSNorm(o_flat @ W_o) @ W_lm in fp64.

    o_flat [n, Hq*d], W_o [Hq*d, hidden], W_lm [hidden, vocab].  The vocab
    axis is processed in column blocks only to bound host memory.
    """
    h = np.asarray(o_flat, dtype=np.float64) @ np.asarray(W_o, dtype=np.float64)
    h = rmsnorm(h, None, eps)
    W_lm = np.asarray(W_lm)
    V = W_lm.shape[1]
    out = np.empty((h.shape[0], V))
    for c0 in range(0, V, chunk):
        out[:, c0:c0 + chunk] = h @ W_lm[:, c0:c0 + chunk].astype(np.float64)
    return out


def margin_ok(logits_ref, token: int, margin: float = 2.0) -> bool:
    """True if ``token`` is within ``margin`` logits of the reference argmax."""
    lr = np.asarray(logits_ref, dtype=np.float64)
    return bool(lr[int(token)] >= lr.max() - margin)


def argmax_lowest(logits) -> int:
    """Greedy choice; ties go to the lowest token id."""
    lr = np.asarray(logits)
    return int(np.flatnonzero(lr == lr.max())[0])


__all__ = [
    "bf16_round", "bf16_bits", "bits_to_f64", "rmsnorm", "rope_inv_freq",
    "rope", "attend_rows", "Cache", "write_kv", "attend_tokens", "prefill",
    "decode", "verify",
    "lm_logits", "margin_ok", "argmax_lowest",
]
