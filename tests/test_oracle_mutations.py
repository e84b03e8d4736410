"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutation replaces one oracle function with a plausible wrong variant (a
dropped term, a wrong sign or index, a transposed operand, a wrong axis) and
runs the pins; the test passes only if some pin raises."""
import numpy as np
import pytest

import oracle
from oracle import csa
from oracle import projection, quant
from tests import test_oracle_attention as A
from tests import test_oracle_pins as P
from tests import test_oracle_projection as Q
from tests import test_oracle_quant as QT

_orig = {name: getattr(csa, name) for name in ("pool", "rope", "rms_norm", "index_score", "topk", "attend",
                                                "window_positions", "sparse_attn", "entry_from_rows")}


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


def _entry_rope_before_norm(e, ratio, gates, values, gamma, rope_dim, rope_base=10000.0, eps=1e-6):
    y = csa.pool(gates, values)
    y = csa.rope(y, e * ratio, rope_dim, rope_base)
    return csa.rms_norm(y, gamma, eps)


def _entry_rope_at_group_end(e, ratio, gates, values, gamma, rope_dim, rope_base=10000.0, eps=1e-6):
    y = csa.rms_norm(csa.pool(gates, values), gamma, eps)
    return csa.rope(y, (e + 1) * ratio - 1, rope_dim, rope_base)


def _rms_eps_outside_root(y, gamma, eps):
    y = np.asarray(y, float)
    return y / (np.sqrt(np.mean(y * y, axis=-1, keepdims=True)) + eps) * gamma


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


_orig_proj = {name: getattr(projection, name) for name in ("q_path", "grouped_down", "out_proj")}


def _q_no_latent_norm(x, wq_a, gamma_q, wq_b, heads, head_dim, pos, rope_dim, rope_base=10000.0, eps=1e-6):
    x = np.asarray(x, float)
    q = ((x @ np.asarray(wq_a, float).T) * gamma_q @ np.asarray(wq_b, float).T).reshape(*x.shape[:-1], heads, head_dim)
    q = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps)
    return csa.rope(q, np.broadcast_to(np.asarray(pos)[..., None], q.shape[:-1]), rope_dim, rope_base)


def _q_norm_over_all_heads(x, wq_a, gamma_q, wq_b, heads, head_dim, pos, rope_dim, rope_base=10000.0, eps=1e-6):
    x = np.asarray(x, float)
    qr = csa.rms_norm(x @ np.asarray(wq_a, float).T, gamma_q, eps)
    q = qr @ np.asarray(wq_b, float).T
    q = (q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps)).reshape(*x.shape[:-1], heads, head_dim)
    return csa.rope(q, np.broadcast_to(np.asarray(pos)[..., None], q.shape[:-1]), rope_dim, rope_base)


def _q_rope_on_leading_dims(x, wq_a, gamma_q, wq_b, heads, head_dim, pos, rope_dim, rope_base=10000.0, eps=1e-6):
    q = _orig_proj["q_path"](x, wq_a, gamma_q, wq_b, heads, head_dim, np.zeros_like(np.asarray(pos)), rope_dim,
                             rope_base, eps)
    flipped = q[..., ::-1].copy()             # rotate the first rope_dim dims instead of the last
    p = np.broadcast_to(np.asarray(pos)[..., None], q.shape[:-1])
    return csa.rope(flipped, p, rope_dim, rope_base)[..., ::-1]


def _grouped_interleaved_heads(o, wo_a, groups):
    o = np.asarray(o, float)
    H = o.shape[-2]
    perm = np.argsort(np.arange(H) % groups, kind="stable")   # group g = heads g, g+G, g+2G, ...
    return _orig_proj["grouped_down"](o[..., perm, :], wo_a, groups)


def _grouped_transposed_weight(o, wo_a, groups):
    o = np.asarray(o, float)
    og = o.reshape(*o.shape[:-2], groups, -1)
    w = np.asarray(wo_a, float)
    return np.einsum("...gd,gdr->...gr", og, w.reshape(w.shape[0], w.shape[2], w.shape[1]))


def _out_proj_without_up(o, wo_a, wo_b, groups):
    r = projection.grouped_down(o, wo_a, groups)
    y = r.reshape(*r.shape[:-2], -1)
    return y[..., :np.asarray(wo_b).shape[0]]


_orig_quant = {name: getattr(quant, name) for name in ("block_scale_exp", "_nearest_code", "quantize_row",
                                                        "e4m3_decode")}


def _scale_clips_like_floor(block, fmt_max):
    a = float(np.max(np.abs(block)))
    if a == 0.0:
        return -127
    return int(np.floor(np.log2(a))) - int(np.floor(np.log2(fmt_max)))   # the max may exceed the format


def _ties_away_from_zero(y, codes, values, sign_bit):
    y = np.asarray(y, float)
    d = np.abs(y[..., None] - values)
    best = np.min(d, axis=-1, keepdims=True)
    score = (d == best) * (4 + 2 * (((codes & sign_bit) != 0) == np.signbit(y)[..., None]) + np.abs(values) /
                           (1 + np.max(np.abs(values))))
    return codes[np.argmax(score, axis=-1)]


def _row_nibbles_swapped(v, rope_dim):
    row = _orig_quant["quantize_row"](v, rope_dim)
    lat = np.asarray(v).shape[-1] - rope_dim
    row[:lat // 2] = ((row[:lat // 2] & 15) << 4) | (row[:lat // 2] >> 4)
    return row


def _e4m3_bias_8(code):
    return _orig_quant["e4m3_decode"](code) / 2.0


MUTATIONS = {
    "quant_scale_may_clip": ("block_scale_exp", _scale_clips_like_floor),
    "quant_ties_away_from_zero": ("_nearest_code", _ties_away_from_zero),
    "quant_row_nibbles_swapped": ("quantize_row", _row_nibbles_swapped),
    "quant_e4m3_exponent_bias_8": ("e4m3_decode", _e4m3_bias_8),
    "q_path_latent_norm_dropped": ("q_path", _q_no_latent_norm),
    "q_path_norm_over_all_heads": ("q_path", _q_norm_over_all_heads),
    "q_path_rope_on_leading_dims": ("q_path", _q_rope_on_leading_dims),
    "out_proj_groups_interleave_heads": ("grouped_down", _grouped_interleaved_heads),
    "out_proj_down_weight_transposed": ("grouped_down", _grouped_transposed_weight),
    "out_proj_up_projection_dropped": ("out_proj", _out_proj_without_up),
    "pool_softmax_over_channels": ("pool", _pool_wrong_axis),
    "pool_zero_padding_for_missing_group": ("pool", _pool_zero_instead_of_minus_inf),
    "rope_wrong_sign": ("rope", _rope_sign),
    "rope_half_split_pairs": ("rope", _rope_half_split),
    "rmsnorm_without_sqrt": ("rms_norm", _rms_no_sqrt),
    "rmsnorm_eps_outside_the_root": ("rms_norm", _rms_eps_outside_root),
    "entry_rope_before_gain_scaled_norm": ("entry_from_rows", _entry_rope_before_norm),
    "entry_rotated_at_its_last_token": ("entry_from_rows", _entry_rope_at_group_end),
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
    P.test_entry_pool_norm_gain_rope_order_hand_worked,
    P.test_rope_large_position_angle_in_float64,
    A.test_sink_closed_form, A.test_sink_limits_and_textbook_softmax,
    A.test_attention_matches_torch_sdpa_with_sink_column, A.test_index_score_brute_force_and_mask,
    A.test_topk_brute_force_and_minus_inf, A.test_full_topk_equals_dense_attention,
    A.test_inverse_rope_on_output_undoes_a_rotated_single_row, A.test_window_positions,
    lambda: A.test_topk_matches_stable_argsort(64, 64, 8),
    Q.test_grouped_projection_is_a_block_diagonal_matmul, Q.test_each_group_reads_only_its_own_heads,
    Q.test_q_path_matches_torch_rms_norm_and_complex_rotation,
    Q.test_q_heads_have_unit_rms_and_rope_spares_the_leading_dims, Q.test_low_rank_query_is_a_two_step_product,
    QT.test_e4m3_codes_match_torch_float8_e4m3fn, QT.test_e4m3_rounding_matches_torch_conversion,
    QT.test_e2m1_midpoints_round_to_the_even_code, QT.test_hand_worked_row,
    lambda: QT.test_block_scale_is_the_smallest_without_clipping("e2m1", 6.0),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    mod = projection if attr in _orig_proj else (quant if attr in _orig_quant else csa)
    monkeypatch.setattr(mod, attr, fn)
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
