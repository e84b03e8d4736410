"""Causality pins of the oracle: prefill == streaming, emission schedule, the
3/4/8 boundary pattern, causal edits, decode == full recompute (no GPU)."""
import copy

import numpy as np
import pytest

import oracle
import synth
from oracle import csa, pipeline
from tests.conftest import read_golden


def _rows(T, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, d)), rng.standard_normal((T, d))


@pytest.mark.parametrize("ratio,overlap", [(4, 1), (2, 1), (4, 0), (128, 0)])
def test_prefill_equals_streaming_bitwise(ratio, overlap):
    """"把推导变成可以检查的程序": whole-span and per-token pooling agree; in
    float64 the two schedules give bit-identical entries."""
    T = 3 * ratio + 1
    kv, gate = _rows(T, 16, ratio)
    gamma = 1 + 0.1 * np.random.default_rng(1).standard_normal(16)
    full = oracle.compress(kv, gate, gamma, ratio, overlap, 8)
    sc = oracle.StreamingCompressor(gamma, ratio, overlap, 8)
    for t in range(T):
        sc.push(t, kv[t], gate[t])
    assert read_golden("lab_checks.txt")["prefill_equals_streaming"] == ["True"]
    assert len(sc.cache) == full.shape[0] == T // ratio
    assert np.array_equal(np.stack(sc.cache), full)


def test_emission_schedule_ratio_2():
    g = read_golden("emission_schedule.txt")
    r, T = int(g["ratio"][0]), int(g["tokens"][0])
    kv, gate = _rows(T, 4, 2)
    sc = oracle.StreamingCompressor(np.ones(4), r, 1, 0)
    emitted = [t for t in range(T) if sc.push(t, kv[t], gate[t]) is not None]
    assert emitted == [int(v) for v in g["emit_at"]]
    assert len(sc.cache) == int(g["entries_after_tokens"][0])
    assert [oracle.visible(t, r) for t in range(T)] == [0, 1, 1, 2, 2, 3]


def test_entries_appear_at_group_ends_ratio_4():
    kv, gate = _rows(12, 4, 3)
    sc = oracle.StreamingCompressor(np.ones(4), 4, 1, 0)
    assert [t for t in range(12) if sc.push(t, kv[t], gate[t]) is not None] == [3, 7, 11]


# ---------------------------------------------------------------------------
# Tiny configuration end to end
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def tiny():
    cfg = synth.TINY
    return cfg, synth.tiny_inputs(cfg)


def test_tiny_decode_equals_prefill(tiny):
    """"4 Profiling" (V4.1 lab): streaming decode equals a full recompute under
    a 1e-9 threshold.  Prefill of 16 tokens followed by 4 streamed tokens is
    compared with a prefill of all 20 tokens."""
    cfg, inp = tiny
    T = cfg.T_prefill + cfg.T_decode
    full = pipeline.tiny_prefill(inp, cfg, T)
    st = pipeline.tiny_stream(inp, cfg, T)
    thr = float(read_golden("lab_checks.txt")["decode_vs_recompute_threshold"][0])
    assert np.array_equal(st["kv_cache"], full["kv_cache"])
    assert np.array_equal(st["idx_cache"], full["idx_cache"])
    for t in range(T):
        assert np.array_equal(st["sel"][t], full["sel"][t])
        assert np.max(np.abs(st["out"][t] - full["out"][t])) < thr


def test_causal_edit_leaves_earlier_rows_unchanged(tiny):
    """"3 Giải pháp" (V4.1 lab): editing the last token leaves every earlier
    output row exactly unchanged."""
    cfg, inp = tiny
    T = 12
    base = pipeline.tiny_prefill(inp, cfg, T)
    edited = copy.deepcopy(inp)
    for key in ("kv", "gate", "k_idx", "g_idx"):
        edited[key][T - 1] += 0.5
    for key in ("q", "q_idx", "w"):
        edited[key][T - 1] *= -1
    new = pipeline.tiny_prefill(edited, cfg, T)
    diff_before = max(np.max(np.abs(new["out"][t] - base["out"][t])) for t in range(T - 1))
    assert diff_before == float(read_golden("lab_checks.txt")["earlier_rows_after_edit"][0])
    assert np.max(np.abs(new["out"][T - 1] - base["out"][T - 1])) > 1e-6


def _pipeline_with_visibility(inp, cfg, T, vis_fn):
    """The tiny prefill with a replaced visibility rule (a planted mistake)."""
    saved = csa.visible
    try:
        csa.visible = vis_fn
        return pipeline.tiny_prefill(inp, cfg, T)
    finally:
        csa.visible = saved


def test_boundary_pattern_3_4_8(tiny):
    """"短输入一致，长输入开始偏：检查边界": an off-by-one visibility rule agrees
    with the correct one for tokens 1-3, departs at token 4, agrees for 5-7
    and departs again at token 8."""
    cfg, inp = tiny
    g = read_golden("boundary_pattern.txt")
    T = int(g["tokens"][0])
    good = pipeline.tiny_prefill(inp, cfg, T)
    bad = _pipeline_with_visibility(inp, cfg, T, lambda t, r: t // r)
    pattern = [int(np.max(np.abs(good["out"][t] - bad["out"][t])) > 0) for t in range(T)]
    assert pattern == [int(v) for v in g["pattern"]]


def test_leaky_visibility_differs_from_token_1(tiny):
    """A rule that exposes partial groups (ceil) leaks in-group future tokens."""
    cfg, inp = tiny
    good = pipeline.tiny_prefill(inp, cfg, 8)
    saved = csa.compress

    def leaky_compress(kv, gate, gamma, ratio, overlap, rope_dim, rope_base=10000.0, eps=1e-6, **kw):
        n = -(-kv.shape[0] // ratio) if ratio > 1 else kv.shape[0]
        pad = n * ratio - kv.shape[0]
        kvp = np.concatenate([kv, np.zeros((pad, kv.shape[1]))])
        gp = np.concatenate([gate, np.full((pad, kv.shape[1]), -np.inf)])
        return saved(kvp, gp, gamma, ratio, overlap, rope_dim, rope_base, eps)

    try:
        csa.compress = leaky_compress
        bad = _pipeline_with_visibility(inp, cfg, 8, lambda t, r: -(-(t + 1) // r))
    finally:
        csa.compress = saved
    assert np.max(np.abs(good["out"][0] - bad["out"][0])) > 0


def test_zero_padded_first_group_differs_from_token_4(tiny):
    """Replacing the -inf previous gates of entry 0 by zero-valued, zero-gated
    padding rows (a plausible mistake) changes entry 0 and hence token 4."""
    cfg, inp = tiny
    good = pipeline.tiny_prefill(inp, cfg, 8)
    saved = csa.entry_candidates
    saved_entry = csa.compress_entry

    def padded_entry(e, kv, gate, kv_prev, gate_prev, gamma, ratio, overlap, rope_dim, rope_base, eps):
        if e == 0 and overlap:
            zk = np.zeros((ratio, kv.shape[1]))
            kv2 = np.concatenate([zk, kv]); g2 = np.concatenate([zk, gate])
            out = saved_entry(1, kv2, g2, kv2, g2, gamma, ratio, overlap, rope_dim, rope_base, eps)
            # undo the position shift of the fake entry 1: rotate back by r
            return oracle.rope(oracle.rope(out, ratio, rope_dim, rope_base, inverse=True), 0, rope_dim, rope_base)
        return saved_entry(e, kv, gate, kv_prev, gate_prev, gamma, ratio, overlap, rope_dim, rope_base, eps)

    try:
        csa.compress_entry = padded_entry
        bad = pipeline.tiny_prefill(inp, cfg, 8)
    finally:
        csa.compress_entry = saved_entry
        csa.entry_candidates = saved
    diffs = [np.max(np.abs(good["out"][t] - bad["out"][t])) for t in range(8)]
    assert all(d == 0 for d in diffs[:3]) and diffs[3] > 0
