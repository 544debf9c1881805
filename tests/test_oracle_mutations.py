"""Plant plausible mistakes in the oracle (CPU only) and check a pin fails.

Each mutation replaces one oracle function for the duration of a test and
runs the pins that should catch it; a pin that still passes would mean the
oracle is not pinned against that mistake.
"""

import numpy as np
import pytest

import oracle
import oracle.attention as A

from . import test_oracle_attention as TA
from . import test_oracle_rmsnorm as TN
from . import test_oracle_rope as TR
from .conftest import read_golden


def _rope_wrong_sign(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    a = np.asarray(pos, dtype=np.float64)[..., None] * A.rope_inv_freq(
        x.shape[-1], theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)


def _rope_interleaved(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = np.asarray(pos, dtype=np.float64)[..., None] * A.rope_inv_freq(d, theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x1 * c - x2 * s
    y[..., 1::2] = x2 * c + x1 * s
    return y


def _freq_wrong(d, theta):
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -i / d)


def _rmsnorm_eps_outside(x, weight=None, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    y = x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)
    return y if weight is None else y * weight


def _attend_sees_one_more(q, K, V, scale, n_visible):
    return _orig_attend(q, K, V, scale, np.minimum(
        np.asarray(n_visible) + 1, np.asarray(K).shape[0]))


def _prologue_no_rounding(k, pos, theta, eps, k_w):
    return A.rope(A.rmsnorm(k, k_w, eps), pos, theta)


_orig_attend = A.attend_rows


def _run_all(tests):
    failed = 0
    for t in tests:
        try:
            t()
        except (AssertionError, ValueError):
            failed += 1
    return failed


def _golden(fn):
    return lambda: fn(read_golden)


MUTATIONS = [
    ("rope_sign", {"rope": _rope_wrong_sign},
     [_golden(TR.test_hand_values), lambda: TR.test_complex_twin(128, 7)]),
    ("rope_interleaved", {"rope": _rope_interleaved},
     [_golden(TR.test_hand_values), lambda: TR.test_complex_twin(128, 7)]),
    ("rope_frequency", {"rope_inv_freq": _freq_wrong},
     [_golden(TR.test_hand_values), TR.test_frequencies_closed_form]),
    ("rmsnorm_eps_outside_root", {"rmsnorm": _rmsnorm_eps_outside},
     [_golden(TN.test_hand_values), TN.test_constant_vector]),
    ("causal_off_by_one", {"attend_rows": _attend_sees_one_more},
     [TA.test_single_visible_key_returns_v, TA.test_sdpa_fp64_special_case]),
    ("k_cache_not_rounded", {"_prologue_k": _prologue_no_rounding},
     [TA.test_mpmath_brute_force_tiny, TA.test_cache_contents]),
]


@pytest.mark.parametrize("name,patch,pins", MUTATIONS,
                         ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, patch, pins):
    for attr, fn in patch.items():
        monkeypatch.setattr(A, attr, fn)
        if hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, fn)
    assert _run_all(pins) >= 1, f"no pin caught mutation {name}"


# --- the attention epilogue (oracle/epilogue.py) -----------------------------

import oracle.epilogue as E  # noqa: E402

from . import test_oracle_epilogue as TE  # noqa: E402


def _proj_not_rounded(o_flat, w_o):
    return np.asarray(o_flat, dtype=np.float64) @ np.asarray(w_o, dtype=np.float64).T


def _proj_weight_transposed(o_flat, w_o):
    # the weight read as [in_dim, hidden] instead of one row per output
    return A.bf16_round(np.asarray(o_flat, dtype=np.float64) @ np.asarray(w_o, dtype=np.float64))


def _epilogue_norm_before_residual(o_flat, w_o, residual, weight=None, eps=1e-6):
    h = E.o_proj(o_flat, w_o)
    out, _ = E.rmsnorm_hidden(h, weight, eps)
    r = A.bf16_round(np.asarray(residual, dtype=np.float64) + h)
    return out, r, h


EPILOGUE_MUTATIONS = [
    ("projection_not_rounded", {"o_proj": _proj_not_rounded},
     [_golden(TE.test_hand_values), TE.test_projection_equals_exact_rational_sum]),
    ("projection_weight_transposed", {"o_proj": _proj_weight_transposed},
     [TE.test_projection_equals_exact_rational_sum, TE.test_matches_torch_bf16_linear_layer]),
    ("norm_before_residual", {"attn_epilogue": _epilogue_norm_before_residual},
     [_golden(TE.test_hand_values), TE.test_identity_and_zero_weights]),
]


@pytest.mark.parametrize("name,patch,pins", EPILOGUE_MUTATIONS,
                         ids=[m[0] for m in EPILOGUE_MUTATIONS])
def test_planted_epilogue_mistake_is_caught(monkeypatch, name, patch, pins):
    for attr, fn in patch.items():
        monkeypatch.setattr(E, attr, fn)
        monkeypatch.setattr(TE, attr, fn)
        if hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, fn)
    assert _run_all(pins) >= 1, f"no pin caught mutation {name}"
