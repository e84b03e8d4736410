"""Whole-path compositions of the float64 oracle steps (test infrastructure).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
use this module.  It strings the per-step definitions of ``oracle.csa``
together in the order the pages give them
([V4-Flash walkthrough] "压缩条目必须等整组完成后才可见" for the emission and
visibility rule, "少读 KV 之前，Indexer 仍要给历史打分" for scoring and top-k,
"局部和压缩记忆，共用一次归一化" for the joint softmax).
"""
from __future__ import annotations

import numpy as np

from . import csa


def csa_query(q, q_idx, w, kv_cache, idx_cache, n_vis, win_rows, sink, k, scale,
              pos, rope_dim, rope_base=10000.0):
    """One CSA query: score visible entries, pick the top-k, attend.

    Returns (scores (N,), selection (k,), output (H, D)).
    """
    scores = csa.index_score(q_idx, w, idx_cache, n_vis)
    sel = csa.topk(scores, n_vis, k)
    out = csa.sparse_attn(q, kv_cache, sel, win_rows, sink, scale, pos, rope_dim, rope_base)
    return scores, sel, out


def window_rows(win_by_pos, t, window):
    """Window rows of a query at t from per-position rows (positions 0..t)."""
    return np.stack([win_by_pos[p] for p in csa.window_positions(t, window)])


def tiny_prefill(inp, cfg, T):
    """Prefill of the first T tokens of the tiny CSA configuration.

    Every compressed entry of the span is built at once; each query then uses
    its own visibility (t+1)//r.  Window rows are the per-token rows
    normalised and rotated at their own position, i.e. the compressor at
    ratio 1 without overlap.  Returns a dict of per-token arrays.
    """
    kv = np.asarray(inp["kv"][:T], np.float64)
    gate = np.asarray(inp["gate"][:T], np.float64)
    ki = np.asarray(inp["k_idx"][:T], np.float64)
    gi = np.asarray(inp["g_idx"][:T], np.float64)
    kv_cache = csa.compress(kv, gate, inp["gamma"], cfg.ratio, cfg.overlap, cfg.rope_dim,
                            cfg.rope_base, cfg.eps)
    idx_cache = csa.compress(ki, gi, inp["gamma_idx"], cfg.ratio, cfg.overlap,
                             cfg.rope_dim_idx, cfg.rope_base, cfg.eps)
    win = csa.compress(kv, np.zeros_like(kv), inp["gamma_win"], 1, 0, cfg.rope_dim,
                       cfg.rope_base, cfg.eps)
    scale = 1.0 / np.sqrt(cfg.D)
    res = dict(kv_cache=kv_cache, idx_cache=idx_cache, win=win, scores=[], sel=[], out=[])
    for t in range(T):
        n_vis = csa.visible(t, cfg.ratio)
        s, sel, o = csa_query(inp["q"][t], inp["q_idx"][t], inp["w"][t], kv_cache, idx_cache,
                              n_vis, window_rows(win, t, cfg.window), inp["sink"], cfg.k,
                              scale, t, cfg.rope_dim, cfg.rope_base)
        res["scores"].append(s)
        res["sel"].append(sel)
        res["out"].append(o)
    return res


def tiny_stream(inp, cfg, T):
    """The same T tokens fed one at a time, as decode would see them.

    Compressors emit an entry only when a group completes; each query reads
    the caches as they stand after its own token was pushed.  Returns per-token
    outputs, selections and the final caches.
    """
    kvc = csa.StreamingCompressor(inp["gamma"], cfg.ratio, cfg.overlap, cfg.rope_dim,
                                  cfg.rope_base, cfg.eps)
    idc = csa.StreamingCompressor(inp["gamma_idx"], cfg.ratio, cfg.overlap, cfg.rope_dim_idx,
                                  cfg.rope_base, cfg.eps)
    wc = csa.StreamingCompressor(inp["gamma_win"], 1, 0, cfg.rope_dim, cfg.rope_base, cfg.eps)
    scale = 1.0 / np.sqrt(cfg.D)
    res = dict(sel=[], out=[], scores=[])
    for t in range(T):
        kvc.push(t, inp["kv"][t], inp["gate"][t])
        idc.push(t, inp["k_idx"][t], inp["g_idx"][t])
        wc.push(t, inp["kv"][t], np.zeros_like(inp["kv"][t]))
        n_vis = len(kvc.cache)
        d, di = cfg.D, cfg.D_I
        kv_cache = np.stack(kvc.cache) if kvc.cache else np.zeros((0, d))
        idx_cache = np.stack(idc.cache) if idc.cache else np.zeros((0, di))
        s, sel, o = csa_query(inp["q"][t], inp["q_idx"][t], inp["w"][t], kv_cache, idx_cache,
                              n_vis, window_rows(wc.cache, t, cfg.window), inp["sink"], cfg.k,
                              scale, t, cfg.rope_dim, cfg.rope_base)
        res["scores"].append(s)
        res["sel"].append(sel)
        res["out"].append(o)
    res["kv_cache"] = np.stack(kvc.cache)
    res["idx_cache"] = np.stack(idc.cache)
    return res
