"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times (its own workload objects, one step through the C ABI), checked
on sampled sequences / queries that the float64 oracle computes one by one.

Sequences and queries are sampled; each sampled one is checked in full:
the compressed entry appended by the step, every index score of the row,
the top-k set (bit-exact up to swaps within 1e-3 relative of the k-th score)
and the attention output (max-abs 2e-2, mean-abs 2e-3), the latter on rows
whose top-k set is exactly the oracle's."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_attn, assert_bf16_matches, assert_normwise, host, progress, topk_set_check

pytestmark = pytest.mark.gpu

f64 = synth.bf16_to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_06_amd as csa
    csa.lib()


@pytest.fixture(autouse=True)
def _name(request):
    progress(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _step(wl):
    import bench
    bench.run_step(wl, 0)
    torch.cuda.synchronize()


def _new_entry(cfg, s, gamma, role):
    """The oracle's entry n_vis-1 from the sequence's staging ring rows."""
    e = s.n_vis - 1
    prev, cur = oracle.entry_candidates(e, cfg.ratio, cfg.overlap)
    slots = [t % synth.staging_rows(cfg) for t in prev + cur]
    if role == "kv":
        g, v, rd = s.gate_stage, s.kv_stage, cfg.rope_dim
    else:
        g, v, rd = s.gi_stage, s.ki_stage, cfg.rope_dim_idx
    return oracle.entry_from_rows(e, cfg.ratio, f64(g[slots]), f64(v[slots]), gamma, rd, cfg.rope_base, cfg.eps)


def _stored(entry):
    """The entry as the bf16 cache holds it."""
    return oracle.round_bf16(entry)


def _check_decode(wl, samples):
    cfg = wl.cfg
    shared = synth.decode_shared(cfg)
    scale = 1.0 / math.sqrt(cfg.D)
    kv_gpu = wl.kv[0]
    out = host(wl.out)
    if cfg.csa:
        scores = wl.scores.cpu().numpy()[:, 0]
        sel = wl.sel.cpu().numpy()[:, 0]
        idx_gpu = wl.idx_cache[0]
    swaps = 0
    for b in samples:
        s = wl.seqs[b]
        e = s.n_vis - 1
        emitted = (s.pos + 1) % cfg.ratio == 0
        win = np.stack([f64(s.win[p % cfg.window]) for p in oracle.window_positions(s.pos, cfg.window)])
        q = f64(s.q)
        if emitted:
            want_kv = _new_entry(cfg, s, shared["gamma"], "kv")
            assert_bf16_matches(host(kv_gpu[b, e])[None], want_kv[None], what=f"b={b} new KV entry")
        if not cfg.csa:
            cmp = f64(synth.kv_cache_rows(cfg, b, s.n_vis))
            if emitted:
                cmp[e] = _stored(want_kv)
            want = oracle.hca_attn(q, cmp, s.n_vis, win, shared["sink"], scale, s.pos, cfg.rope_dim, cfg.rope_base)
            assert_attn(out[b, 0], want, what=f"b={b} HCA output")
            continue
        idx_cache = f64(synth.idx_cache_rows(cfg, b, s.n_vis))
        if emitted:
            want_i = _new_entry(cfg, s, shared["gamma_idx"], "idx")
            assert_bf16_matches(host(idx_gpu[b, e])[None], want_i[None], what=f"b={b} new index entry")
            idx_cache[e] = _stored(want_i)
        want_s = oracle.index_score(f64(s.q_idx), s.w, idx_cache, s.n_vis)
        got_s = scores[b]
        assert np.all(np.isneginf(got_s[s.n_vis:])), f"b={b}: invisible entries must be -inf"
        assert_normwise(got_s[:s.n_vis][None], want_s[None], what=f"b={b} index scores")
        want_sel = oracle.topk(want_s, s.n_vis, cfg.k)
        swaps += topk_set_check(sel[b][None], want_s[None], want_sel[None], cfg.k)
        if set(sel[b]) == set(want_sel):
            picked = [int(i) for i in want_sel if i >= 0]
            rows = f64(synth.kv_cache_rows_at(cfg, b, picked)) if picked else np.zeros((0, cfg.D))
            if emitted and e in picked:
                rows[picked.index(e)] = _stored(want_kv)
            o = oracle.sparse_attn(q, rows, np.arange(len(picked)), win, shared["sink"], scale, s.pos,
                                   cfg.rope_dim, cfg.rope_base)
            assert_attn(out[b, 0], o, what=f"b={b} CSA output")
    return swaps


def test_csa_decode_64k():
    import bench
    wl = bench.DecodeWorkload(synth.CSA_DECODE_64K, "cuda", copies=1)
    progress("csa_decode_64k: step")
    _step(wl)
    assert _check_decode(wl, [0, 3, 7]) <= 1


def test_csa_decode_64k_k1024():
    """The 64K-context decode with the larger model's top-k of 1024."""
    import bench
    wl = bench.DecodeWorkload(synth.CSA_DECODE_64K_K1024, "cuda", copies=1)
    progress("csa_decode_64k_k1024: step")
    _step(wl)
    assert _check_decode(wl, [0, 5]) <= 1


def test_hca_decode_1m():
    import bench
    wl = bench.DecodeWorkload(synth.HCA_DECODE_1M, "cuda", copies=1)
    progress("hca_decode_1m: step")
    _step(wl)
    _check_decode(wl, [0, 1, 2, 3])


def test_csa_decode_1m_lengths_mix():
    """The 1M-context CSA decode with per-sequence lengths U[512K, 1M], all 32
    sequences as the bench runs them (caches of 262,144 rows each); four
    sequences are checked against the oracle."""
    import bench
    wl = bench.DecodeWorkload(synth.CSA_DECODE_1M, "cuda", copies=1)
    assert len(set(int(n) for n in wl.lengths)) > 16
    progress("csa_decode_1m: step")
    _step(wl)
    assert _check_decode(wl, [0, 7, 19, 31]) <= 1


def test_csa_prefill_8k():
    import bench
    cfg = synth.CSA_PREFILL_8K
    wl = bench.PrefillWorkload(cfg, "cuda", copies=1)
    progress("csa_prefill_8k: step")
    _step(wl)
    shared = synth.decode_shared(cfg)
    inp = synth.prefill_inputs(cfg, q_rows=[])
    kvc = oracle.compress(f64(inp["kv"]), f64(inp["gate"]), shared["gamma"], cfg.ratio, cfg.overlap, cfg.rope_dim,
                          cfg.rope_base, cfg.eps)
    idc = oracle.compress(f64(inp["k_idx"]), f64(inp["g_idx"]), shared["gamma_idx"], cfg.ratio, cfg.overlap,
                          cfg.rope_dim_idx, cfg.rope_base, cfg.eps)
    assert_bf16_matches(host(wl.kv_cache)[0], kvc, what="KV cache")
    assert_bf16_matches(host(wl.idx_cache)[0], idc, what="index cache")
    # the caches are stored as bfloat16: scoring and attention read them so
    kvc, idc = oracle.round_bf16(kvc), oracle.round_bf16(idc)
    rng = np.random.default_rng(8)
    samples = sorted(set([0, 1, 3, 4, 7, 127, 128, 511, 2048, 4095, 8190, 8191] +
                         list(rng.integers(0, cfg.S, 6))))
    qin = synth.prefill_inputs(cfg, q_rows=samples)
    scores = wl.scores.cpu().numpy()[0]
    sel = wl.sel.cpu().numpy()[0]
    out = host(wl.out[0, samples])
    win = f64(inp["win"])
    swaps = 0
    for j, t in enumerate(samples):
        n_vis = oracle.visible(t, cfg.ratio)
        want_s = oracle.index_score(f64(qin["q_idx"][j]), qin["w"][j], idc, n_vis)
        assert_normwise(scores[t][None], want_s[None], what=f"t={t} scores")
        want_sel = oracle.topk(want_s, n_vis, cfg.k)
        swaps += topk_set_check(sel[t][None], want_s[None], want_sel[None], cfg.k)
        if set(sel[t]) == set(want_sel):
            o = oracle.sparse_attn(f64(qin["q"][j]), kvc, want_sel, np.stack(
                [win[p] for p in oracle.window_positions(t, cfg.window)]), shared["sink"], 1 / math.sqrt(cfg.D), t,
                cfg.rope_dim, cfg.rope_base)
            assert_attn(out[j], o, what=f"t={t} output")
    assert swaps <= 2
