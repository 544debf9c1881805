"""Pins for the oracle's attention and the prefill / decode / verify wrappers.

Closed forms and invariants fix the softmax-attention definition; torch's fp64
``scaled_dot_product_attention`` with an explicit bottom-right boolean mask is
the library special case; a 50-digit mpmath brute force re-derives the whole
prefill path (norm, rotation, bf16 cache, attention) on tiny shapes.
"""

import math

import mpmath
import numpy as np
import pytest
import torch

import oracle

THETA = 1.0e6
EPS = 1e-6


def _parse(s):
    return np.array([[float(t) for t in r.split()] for r in s.split(";")])


def test_hand_values(golden):
    for name, q, K, V, scale, o_exp, lse_exp in golden("attention_hand.txt"):
        qv = _parse(q)
        o, lse = oracle.attend_rows(qv, _parse(K), _parse(V), float(scale),
                                    [_parse(K).shape[0]])
        assert np.allclose(o[0], _parse(o_exp)[0], rtol=0, atol=1e-15), name
        assert abs(lse[0] - float(lse_exp)) < 1e-14, name


def test_single_visible_key_returns_v():
    g = np.random.default_rng(0)
    q, K, V = g.standard_normal((3, 16)), g.standard_normal((9, 16)), \
        g.standard_normal((9, 16))
    o, _ = oracle.attend_rows(q, K, V, 0.25, [1, 1, 1])
    assert np.array_equal(o, np.repeat(V[:1], 3, axis=0))


def test_uniform_v_and_zero_q():
    g = np.random.default_rng(1)
    K = g.standard_normal((50, 32))
    row = g.standard_normal(32)
    V = np.repeat(row[None], 50, axis=0)
    o, _ = oracle.attend_rows(g.standard_normal((4, 32)), K, V, 0.2,
                              [50, 10, 3, 1])
    assert np.allclose(o, row[None], rtol=1e-14, atol=1e-14)
    V2 = g.standard_normal((50, 32))
    o0, lse0 = oracle.attend_rows(np.zeros((2, 32)), K, V2, 0.2, [50, 7])
    assert np.allclose(o0[0], V2.mean(0), atol=1e-14)
    assert np.allclose(o0[1], V2[:7].mean(0), atol=1e-14)
    assert np.allclose(lse0, [math.log(50), math.log(7)], atol=1e-14)


def test_two_keys_sigmoid():
    g = np.random.default_rng(2)
    q, K, V = g.standard_normal(8), g.standard_normal((2, 8)), \
        g.standard_normal((2, 8))
    s = 0.3 * K @ q
    w1 = 1.0 / (1.0 + math.exp(-(s[0] - s[1])))
    o, _ = oracle.attend_rows(q[None], K, V, 0.3, [2])
    assert np.allclose(o[0], w1 * V[0] + (1 - w1) * V[1], atol=1e-15)


def test_shift_and_permutation_invariance():
    g = np.random.default_rng(3)
    q, K, V = g.standard_normal((5, 16)), g.standard_normal((30, 16)), \
        g.standard_normal((30, 16))
    o, lse = oracle.attend_rows(q, K, V, 0.25, [30] * 5)
    u = g.standard_normal(16)
    o2, lse2 = oracle.attend_rows(q, K + u, V, 0.25, [30] * 5)
    assert np.allclose(o, o2, atol=1e-13)
    assert np.allclose(lse2 - lse, 0.25 * q @ u, atol=1e-12)
    perm = g.permutation(30)
    o3, lse3 = oracle.attend_rows(q, K[perm], V[perm], 0.25, [30] * 5)
    assert np.allclose(o, o3, atol=1e-13) and np.allclose(lse, lse3,
                                                          atol=1e-13)


def test_lse_is_logsumexp():
    g = np.random.default_rng(4)
    q, K, V = g.standard_normal((1, 16)), g.standard_normal((20, 16)), \
        g.standard_normal((20, 16))
    _, lse = oracle.attend_rows(q, K, V, 0.5, [13])
    s = 0.5 * K[:13] @ q[0]
    mpmath.mp.dps = 40
    ref = mpmath.log(sum(mpmath.e ** mpmath.mpf(float(x)) for x in s))
    assert abs(lse[0] - float(ref)) < 1e-13


def test_unwritten_visible_slot_is_refused():
    K = np.full((4, 8), np.nan)
    with pytest.raises(ValueError):
        oracle.attend_rows(np.ones((1, 8)), K, K, 1.0, [2])


# ---------------------------------------------------------------- wrappers


def _rand_prefill(g, lens, Hq, Hkv, d, cap, start=None):
    T = sum(lens)
    q = oracle.bf16_round(g.standard_normal((T, Hq, d)))
    k = oracle.bf16_round(g.standard_normal((T, Hkv, d)))
    v = oracle.bf16_round(g.standard_normal((T, Hkv, d)))
    cu = np.concatenate([[0], np.cumsum(lens)])
    start = [0] * len(lens) if start is None else start
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(start, lens)])
    return q, k, v, cu, pos


def test_sdpa_fp64_special_case():
    g = np.random.default_rng(5)
    lens, Hq, Hkv, d = [7, 12], 4, 2, 16
    q, k, v, cu, pos = _rand_prefill(g, lens, Hq, Hkv, d, 16)
    cache = oracle.Cache.empty(2, Hkv, 16, d)
    out, lse, c = oracle.prefill(cache, q, k, v, cu, pos, scale=0.3,
                                 theta=THETA, eps=EPS)
    # re-derive q' directly; K'/V from the cache the oracle wrote
    qp = oracle.rope(oracle.rmsnorm(q, None, EPS), pos[:, None], THETA)
    for b, (s0, s1) in enumerate(zip(cu[:-1], cu[1:])):
        L = s1 - s0
        Qt = torch.from_numpy(qp[s0:s1].transpose(1, 0, 2).copy())  # [Hq,L,d]
        Kt = torch.from_numpy(c.k[b, :, :L].copy()).repeat_interleave(
            Hq // Hkv, 0)
        Vt = torch.from_numpy(c.v[b, :, :L].copy()).repeat_interleave(
            Hq // Hkv, 0)
        mask = torch.ones(L, L, dtype=torch.bool).tril()
        ref = torch.nn.functional.scaled_dot_product_attention(
            Qt, Kt, Vt, attn_mask=mask, scale=0.3)
        assert np.allclose(out[s0:s1].transpose(1, 0, 2), ref.numpy(),
                           rtol=0, atol=1e-12)


def test_bottom_right_alignment_with_prefix():
    # A block at positions 5..7 over a cache already holding slots 0..4 sees
    # slots 0..p: equal to SDPA with a bottom-right mask of shape [3, 8].
    g = np.random.default_rng(6)
    Hq, Hkv, d = 2, 1, 16
    q0, k0, v0, cu0, pos0 = _rand_prefill(g, [5], Hq, Hkv, d, 8)
    c0 = oracle.Cache.empty(1, Hkv, 8, d)
    _, _, c0 = oracle.prefill(c0, q0, k0, v0, cu0, pos0, scale=0.25,
                              theta=THETA, eps=EPS)
    q1, k1, v1, cu1, pos1 = _rand_prefill(g, [3], Hq, Hkv, d, 8, start=[5])
    out, _, c1 = oracle.prefill(c0, q1, k1, v1, cu1, pos1, scale=0.25,
                                theta=THETA, eps=EPS)
    qp = oracle.rope(oracle.rmsnorm(q1, None, EPS), pos1[:, None], THETA)
    Qt = torch.from_numpy(qp.transpose(1, 0, 2).copy())
    Kt = torch.from_numpy(c1.k[0, :, :8].copy()).repeat_interleave(Hq, 0)
    Vt = torch.from_numpy(c1.v[0, :, :8].copy()).repeat_interleave(Hq, 0)
    mask = torch.ones(3, 8, dtype=torch.bool).tril(diagonal=5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Qt, Kt, Vt, attn_mask=mask, scale=0.25)
    assert np.allclose(out.transpose(1, 0, 2), ref.numpy(), atol=1e-12)


def _brute_prefill_mp(q, k, v, scale, theta, eps):
    """Whole single-sequence prefill at 50 digits with plain loops."""
    mpmath.mp.dps = 50
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    half = d // 2

    def norm(x):
        ms = sum(mpmath.mpf(float(t)) ** 2 for t in x) / d
        r = mpmath.sqrt(ms + mpmath.mpf(eps))
        return [mpmath.mpf(float(t)) / r for t in x]

    def rot(x, p):
        y = [None] * d
        for i in range(half):
            a = p * mpmath.power(mpmath.mpf(theta), -mpmath.mpf(2 * i) / d)
            z = mpmath.mpc(x[i], x[i + half]) * mpmath.expj(a)
            y[i], y[i + half] = z.real, z.imag
        return y

    # cache: K rounded once to bf16 (rounding pinned in test_oracle_bf16)
    Kc = [[oracle.bf16_round(np.array([float(t) for t in rot(norm(k[t, g]), t)]))
           for t in range(T)] for g in range(Hkv)]
    out = np.zeros((T, Hq, d))
    for t in range(T):
        for h in range(Hq):
            qp = rot(norm(q[t, h]), t)
            g = h // G
            s = [mpmath.mpf(scale) * sum(qp[i] * mpmath.mpf(float(Kc[g][j][i]))
                                         for i in range(d)) for j in range(t + 1)]
            m = max(s)
            e = [mpmath.e ** (x - m) for x in s]
            den = sum(e)
            for i in range(d):
                out[t, h, i] = float(sum(e[j] * mpmath.mpf(float(v[j, g, i]))
                                         for j in range(t + 1)) / den)
    return out


def test_mpmath_brute_force_tiny():
    g = np.random.default_rng(7)
    T, Hq, Hkv, d = 5, 2, 1, 8
    q = oracle.bf16_round(g.standard_normal((T, Hq, d)))
    k = oracle.bf16_round(g.standard_normal((T, Hkv, d)))
    v = oracle.bf16_round(g.standard_normal((T, Hkv, d)))
    cache = oracle.Cache.empty(1, Hkv, 6, d)
    out, _, _ = oracle.prefill(cache, q, k, v, [0, T], np.arange(T),
                               scale=1 / math.sqrt(d), theta=THETA, eps=EPS)
    ref = _brute_prefill_mp(q, k, v, 1 / math.sqrt(d), THETA, EPS)
    assert np.allclose(out, ref, rtol=0, atol=1e-13)


def test_cache_contents():
    g = np.random.default_rng(8)
    q, k, v, cu, pos = _rand_prefill(g, [6, 3], 4, 2, 16, 8)
    cache = oracle.Cache.empty(2, 2, 8, 16)
    _, _, c = oracle.prefill(cache, q, k, v, cu, pos, scale=0.25,
                             theta=THETA, eps=EPS)
    # V is a copy, K is RNE(rope(norm(k))) which is bf16-representable
    assert np.array_equal(c.v[0, :, :6], v[0:6].transpose(1, 0, 2))
    assert np.array_equal(c.v[1, :, :3], v[6:9].transpose(1, 0, 2))
    assert np.array_equal(oracle.bf16_round(c.k[0, :, :6]), c.k[0, :, :6])
    assert np.isnan(c.k[0, :, 6:]).all() and np.isnan(c.v[1, :, 3:]).all()


def test_causality():
    g = np.random.default_rng(9)
    q, k, v, cu, pos = _rand_prefill(g, [10], 4, 1, 16, 10)
    cache = oracle.Cache.empty(1, 1, 10, 16)
    o1, _, _ = oracle.prefill(cache, q, k, v, cu, pos, scale=0.25,
                              theta=THETA, eps=EPS)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[6:] += 1.0
    k2[6:] -= 2.0
    v2[6:] *= 3.0
    o2, _, _ = oracle.prefill(cache, q2, k2, v2, cu, pos, scale=0.25,
                              theta=THETA, eps=EPS)
    assert np.array_equal(o1[:6], o2[:6])
    assert not np.allclose(o1[6:], o2[6:])


def test_gqa_equals_mha_with_repeated_kv():
    g = np.random.default_rng(10)
    Hq, Hkv, d = 8, 2, 16
    q, k, v, cu, pos = _rand_prefill(g, [9], Hq, Hkv, d, 9)
    o1, _, _ = oracle.prefill(oracle.Cache.empty(1, Hkv, 9, d), q, k, v, cu,
                              pos, scale=0.25, theta=THETA, eps=EPS)
    G = Hq // Hkv
    o2, _, _ = oracle.prefill(oracle.Cache.empty(1, Hq, 9, d), q,
                              np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                              cu, pos, scale=0.25, theta=THETA, eps=EPS)
    assert np.array_equal(o1, o2)


def test_decode_equals_prefill_row():
    g = np.random.default_rng(11)
    Hq, Hkv, d, S = 4, 2, 16, 12
    q, k, v, cu, pos = _rand_prefill(g, [S], Hq, Hkv, d, S)
    full, lse_f, _ = oracle.prefill(oracle.Cache.empty(1, Hkv, S, d), q, k, v,
                                    cu, pos, scale=0.25, theta=THETA, eps=EPS)
    t = S - 1
    _, _, c = oracle.prefill(oracle.Cache.empty(1, Hkv, S, d), q[:t], k[:t],
                             v[:t], [0, t], pos[:t], scale=0.25, theta=THETA,
                             eps=EPS)
    o, lse, _ = oracle.decode(c, q[t:], k[t:], v[t:], [t], scale=0.25,
                              theta=THETA, eps=EPS)
    assert np.allclose(o[0], full[t], atol=1e-14)
    assert np.allclose(lse[0], lse_f[t], atol=1e-13)


def test_verify_equals_sequential_decodes():
    g = np.random.default_rng(12)
    B, Hq, Hkv, d, L, n = 2, 4, 2, 16, 7, 4
    q0, k0, v0, cu, pos = _rand_prefill(g, [L, L], Hq, Hkv, d, L + n)
    _, _, c = oracle.prefill(oracle.Cache.empty(B, Hkv, L + n, d), q0, k0, v0,
                             cu, pos, scale=0.25, theta=THETA, eps=EPS)
    qb = oracle.bf16_round(g.standard_normal((B, n, Hq, d)))
    kb = oracle.bf16_round(g.standard_normal((B, n, Hkv, d)))
    vb = oracle.bf16_round(g.standard_normal((B, n, Hkv, d)))
    ov, lv, cv = oracle.verify(c, qb, kb, vb, [L, L], scale=0.25, theta=THETA,
                               eps=EPS)
    cs = c
    for i in range(n):
        o, l, cs = oracle.decode(cs, qb[:, i], kb[:, i], vb[:, i],
                                 [L + i, L + i], scale=0.25, theta=THETA,
                                 eps=EPS)
        assert np.allclose(ov[:, i], o, atol=1e-14)
        assert np.allclose(lv[:, i], l, atol=1e-13)
    assert np.array_equal(cs.k, cv.k, equal_nan=True)
    assert np.array_equal(cs.v, cv.v, equal_nan=True)


def test_packed_equals_separate():
    g = np.random.default_rng(13)
    lens, Hq, Hkv, d = [5, 11, 3], 4, 2, 16
    q, k, v, cu, pos = _rand_prefill(g, lens, Hq, Hkv, d, 12)
    out, lse, c = oracle.prefill(oracle.Cache.empty(3, Hkv, 12, d), q, k, v,
                                 cu, pos, scale=0.25, theta=THETA, eps=EPS)
    for b in range(3):
        s0, s1 = cu[b], cu[b + 1]
        o1, l1, c1 = oracle.prefill(oracle.Cache.empty(1, Hkv, 12, d),
                                    q[s0:s1], k[s0:s1], v[s0:s1],
                                    [0, s1 - s0], pos[s0:s1], scale=0.25,
                                    theta=THETA, eps=EPS)
        assert np.array_equal(out[s0:s1], o1) and np.array_equal(lse[s0:s1],
                                                                 l1)
        assert np.array_equal(c.k[b], c1.k[0], equal_nan=True)


def test_lse_merge_of_a_partition_equals_whole():
    # The identity split-K kernels rely on: for disjoint key sets A and B,
    # o = (e^{lA} oA + e^{lB} oB) / (e^{lA} + e^{lB}), lse = logaddexp(lA, lB).
    g = np.random.default_rng(14)
    q, K, V = g.standard_normal((3, 16)), g.standard_normal((40, 16)), \
        g.standard_normal((40, 16))
    o, l = oracle.attend_rows(q, K, V, 0.25, [40] * 3)
    oA, lA = oracle.attend_rows(q, K[:17], V[:17], 0.25, [17] * 3)
    oB, lB = oracle.attend_rows(q, K[17:], V[17:], 0.25, [23] * 3)
    M = np.maximum(lA, lB)
    wA, wB = np.exp(lA - M), np.exp(lB - M)
    om = (wA[:, None] * oA + wB[:, None] * oB) / (wA + wB)[:, None]
    assert np.allclose(om, o, atol=1e-14)
    assert np.allclose(np.logaddexp(lA, lB), l, atol=1e-14)


def test_row_sampling_matches_full():
    g = np.random.default_rng(15)
    q, k, v, cu, pos = _rand_prefill(g, [6, 9], 4, 2, 16, 10)
    seq = np.repeat([0, 1], [6, 9])
    c = oracle.write_kv(oracle.Cache.empty(2, 2, 10, 16), k, v, seq, pos,
                        theta=THETA, eps=EPS)
    full, lf = oracle.attend_tokens(c, q, seq, pos, scale=0.25, theta=THETA,
                                    eps=EPS)
    rows = [(0, 0), (5, 3), (6, 1), (14, 2)]
    part, lp = oracle.attend_tokens(c, q, seq, pos, scale=0.25, theta=THETA,
                                    eps=EPS, rows=rows)
    for t, h in rows:
        assert np.allclose(part[t, h], full[t, h], atol=1e-14)
        assert abs(lp[t, h] - lf[t, h]) < 1e-13
