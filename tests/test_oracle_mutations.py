"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutation replaces one oracle function with a plausible wrong variant (a
dropped term, a wrong sign or index, a transposed operand, a wrong axis) and
runs the pins; the test passes only if some pin raises."""
import numpy as np
import pytest

import oracle
from oracle import csa
from tests import test_oracle_attention as A
from tests import test_oracle_pins as P

_orig = {name: getattr(csa, name) for name in ("pool", "rope", "rms_norm", "index_score", "topk", "attend",
                                                "window_positions", "sparse_attn")}


def _pool_wrong_axis(gates, values):
    g = np.asarray(gates, float)
    v = np.asarray(values, float)
    keep = g != -np.inf
    e = np.where(keep, np.exp(np.where(keep, g, 0) - np.max(np.where(keep, g, 0), axis=1, keepdims=True)), 0)
    p = e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)   # softmax over channels
    return np.sum(np.where(keep, p * v, 0), axis=0)


def _pool_zero_instead_of_minus_inf(gates, values):
    g = np.where(np.asarray(gates, float) == -np.inf, 0.0, gates)
    v = np.where(np.isfinite(values), values, 0.0)
    return _orig["pool"](g, v)


def _rope_sign(x, pos, rope_dim, base=10000.0, inverse=False):
    return _orig["rope"](x, pos, rope_dim, base, inverse=not inverse)


def _rope_half_split(x, pos, rope_dim, base=10000.0, inverse=False):
    x = np.array(x, float, copy=True)
    if rope_dim == 0:
        return x
    d, h = x.shape[-1], rope_dim // 2
    th = base ** (-2.0 * np.arange(h) / rope_dim)
    a = np.asarray(pos, float)[..., None] * th
    c, s = np.cos(a), np.sin(a) * (-1 if inverse else 1)
    lo, hi = x[..., d - rope_dim:d - h].copy(), x[..., d - h:].copy()
    x[..., d - rope_dim:d - h] = lo * c - hi * s
    x[..., d - h:] = lo * s + hi * c
    return x


def _rms_no_sqrt(y, gamma, eps):
    y = np.asarray(y, float)
    return y / (np.mean(y * y, axis=-1, keepdims=True) + eps) * gamma


def _index_no_relu(q_idx, w, idx_cache, n_vis):
    k = np.asarray(idx_cache, float)
    out = np.full(k.shape[0], -np.inf)
    m = min(n_vis, k.shape[0])
    out[:m] = (k[:m] @ np.asarray(q_idx, float).T) @ np.asarray(w, float)
    return out


def _index_w_reversed(q_idx, w, idx_cache, n_vis):
    return _orig["index_score"](q_idx, np.asarray(w)[::-1], idx_cache, n_vis)


def _topk_ties_high(scores, n_valid, k):
    s = np.asarray(scores, float)[:n_valid]
    cand = np.nonzero(s != -np.inf)[0]
    order = np.lexsort((-cand, -s[cand]))
    chosen = np.sort(cand[order[:k]])
    out = np.full(k, -1, np.int64)
    out[:chosen.size] = chosen
    return out


def _attend_sink_scaled(q, rows, sink, scale):
    return _orig["attend"](q, rows, np.asarray(sink) * scale, scale)


def _attend_no_scale(q, rows, sink, scale):
    return _orig["attend"](q, rows, sink, 1.0)


def _attend_sink_dropped(q, rows, sink, scale):
    return _orig["attend"](q, rows, np.full(np.shape(sink), -np.inf), scale)


def _window_excludes_self(t, window):
    return list(range(max(0, t - window), t))


def _sparse_no_inverse_rope(q, cmp, sel, win_rows, sink, scale, pos, rope_dim, rope_base=10000.0):
    return _orig["sparse_attn"](q, cmp, sel, win_rows, sink, scale, pos, 0, rope_base)


MUTATIONS = {
    "pool_softmax_over_channels": ("pool", _pool_wrong_axis),
    "pool_zero_padding_for_missing_group": ("pool", _pool_zero_instead_of_minus_inf),
    "rope_wrong_sign": ("rope", _rope_sign),
    "rope_half_split_pairs": ("rope", _rope_half_split),
    "rmsnorm_without_sqrt": ("rms_norm", _rms_no_sqrt),
    "indexer_without_relu": ("index_score", _index_no_relu),
    "indexer_head_weights_misindexed": ("index_score", _index_w_reversed),
    "topk_ties_to_higher_index": ("topk", _topk_ties_high),
    "sink_scaled_like_logits": ("attend", _attend_sink_scaled),
    "logit_scale_dropped": ("attend", _attend_no_scale),
    "sink_dropped": ("attend", _attend_sink_dropped),
    "window_excludes_self": ("window_positions", _window_excludes_self),
    "no_inverse_rope_on_output": ("sparse_attn", _sparse_no_inverse_rope),
}

PINS = [
    P.test_pooled_scalar_7_4_pool, P.test_minus_inf_candidates_are_never_read,
    P.test_equal_gates_give_the_arithmetic_mean, P.test_pool_matches_scalar_brute_force,
    P.test_rms_norm_unit_rms_and_scale_invariance, P.test_rope_matches_complex_rotation,
    P.test_rope_large_position_angle_in_float64,
    A.test_sink_closed_form, A.test_sink_limits_and_textbook_softmax,
    A.test_attention_matches_torch_sdpa_with_sink_column, A.test_index_score_brute_force_and_mask,
    A.test_topk_brute_force_and_minus_inf, A.test_full_topk_equals_dense_attention,
    A.test_inverse_rope_on_output_undoes_a_rotated_single_row, A.test_window_positions,
    lambda: A.test_topk_matches_stable_argsort(64, 64, 8),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(csa, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin in PINS:
        pin()
