"""Pins of the oracle's indexer, top-k and attention (no GPU): closed forms of
the sink, library routines (stable argsort, torch SDPA in float64), GEMV
special cases and brute-force loops."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import csa, pipeline


# ---------------------------------------------------------------------------
# Sink
# ---------------------------------------------------------------------------
def test_sink_closed_form():
    """"局部和压缩记忆，共用一次归一化": the sink adds to the denominator only,
    so o_sink = (1 - p_sink) * o_nosink with p_sink = sigmoid(s - lse(l))."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 16))
    rows = rng.standard_normal((7, 16))
    sink = np.array([0.3, -2.0, 4.0])
    scale = 0.25
    with_sink = oracle.attend(q, rows, sink, scale)
    no_sink = oracle.attend(q, rows, np.full(3, -np.inf), scale)
    logits = q @ rows.T * scale
    lse = np.log(np.sum(np.exp(logits), axis=1))
    p_sink = 1.0 / (1.0 + np.exp(-(sink - lse)))
    assert np.allclose(with_sink, (1 - p_sink)[:, None] * no_sink, atol=1e-14)


def test_sink_limits_and_textbook_softmax():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 8))
    rows = rng.standard_normal((5, 8))
    no_sink = oracle.attend(q, rows, np.full(2, -np.inf), 1.0)
    logits = q @ rows.T
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(no_sink, p @ rows, atol=1e-14)
    assert np.allclose(oracle.attend(q, rows, np.full(2, 1e4), 1.0), 0, atol=1e-300)
    # no candidate at all: only the sink, output zero
    assert np.array_equal(oracle.attend(q, np.zeros((0, 8)), np.zeros(2), 1.0), np.zeros((2, 8)))


def test_attention_matches_torch_sdpa_with_sink_column():
    """Library routine: the sink is an extra key with a zero value whose logit
    is the sink (an additive float mask); SDPA in float64 on the CPU."""
    rng = np.random.default_rng(13)
    H, D, C = 4, 32, 9
    q = rng.standard_normal((H, D))
    rows = rng.standard_normal((C, D))
    sink = rng.standard_normal(H)
    scale = 1 / math.sqrt(D)
    keys = np.concatenate([rows, np.zeros((1, D))])
    mask = np.zeros((H, 1, C + 1))
    mask[:, 0, C] = sink
    tq = torch.tensor(q).reshape(1, H, 1, D)
    tk = torch.tensor(keys).reshape(1, 1, C + 1, D).expand(1, H, C + 1, D)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tk, attn_mask=torch.tensor(mask)[None], scale=scale)
    assert np.allclose(oracle.attend(q, rows, sink, scale), ref.numpy().reshape(H, D), atol=1e-13)


# ---------------------------------------------------------------------------
# Indexer
# ---------------------------------------------------------------------------
def test_index_score_gemv_special_case():
    """One head, w = 1, non-negative dot products: a plain GEMV."""
    rng = np.random.default_rng(14)
    k = np.abs(rng.standard_normal((50, 16)))
    q = np.abs(rng.standard_normal((1, 16)))
    s = oracle.index_score(q, np.ones(1), k, 50)
    assert np.allclose(s, np.dot(k, q[0]), atol=1e-13)


def test_index_score_brute_force_and_mask():
    rng = np.random.default_rng(15)
    H, D, N, vis = 3, 8, 12, 9
    q = rng.standard_normal((H, D))
    w = rng.standard_normal(H)
    k = rng.standard_normal((N, D))
    s = oracle.index_score(q, w, k, vis)
    for e in range(N):
        if e >= vis:
            assert s[e] == -np.inf
            continue
        acc = 0.0
        for h in range(H):
            dot = sum(q[h, d] * k[e, d] for d in range(D))
            acc += w[h] * max(dot, 0.0)
        assert s[e] == pytest.approx(acc, abs=1e-13)
    # negative dot products are cut by the ReLU: a head whose dots are all
    # negative contributes nothing whatever its weight
    s2 = oracle.index_score(np.stack([q[0], -np.abs(k).sum(0)]), np.array([w[0], 1e6]), np.abs(k), N)
    assert np.allclose(s2, oracle.index_score(q[:1], w[:1], np.abs(k), N), atol=1e-13)


# ---------------------------------------------------------------------------
# Top-k
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,n_valid,k", [(64, 64, 8), (64, 40, 8), (64, 5, 8), (300, 300, 300), (20, 0, 4)])
def test_topk_matches_stable_argsort(n, n_valid, k):
    s = synth.topk_scores(99, 1, n, tie_frac=0.3)[0].astype(np.float64)
    got = oracle.topk(s, n_valid, k)
    order = np.argsort(-s[:n_valid], kind="stable")       # ties keep index order
    want = np.sort(order[:k])
    assert np.array_equal(got[:want.size], want)
    assert np.all(got[want.size:] == -1)


def test_topk_brute_force_and_minus_inf():
    s = np.array([1.0, 3.0, 3.0, -np.inf, 2.0, 3.0, -np.inf])
    assert list(oracle.topk(s, 7, 2)) == [1, 2]
    assert list(oracle.topk(s, 7, 5)) == [0, 1, 2, 4, 5]
    assert list(oracle.topk(s, 7, 7)) == [0, 1, 2, 4, 5, -1, -1]
    ranked = sorted(range(7), key=lambda j: (-s[j], j))
    assert list(oracle.topk(s, 7, 3)) == sorted(ranked[:3])


# ---------------------------------------------------------------------------
# Whole path: top-k covering every entry == dense attention == HCA
# ---------------------------------------------------------------------------
def test_full_topk_equals_dense_attention():
    """When k >= visible entries, CSA reads every visible entry: the result
    equals the HCA formula and a dense SDPA over window + all entries."""
    rng = np.random.default_rng(16)
    H, D, rd, N, W, t = 4, 32, 8, 10, 4, 45
    q = rng.standard_normal((H, D))
    cmp = rng.standard_normal((N, D))
    win = rng.standard_normal((W, D))
    sink = rng.standard_normal(H)
    qi = rng.standard_normal((2, 16))
    ki = rng.standard_normal((N, 16))
    n_vis = oracle.visible(t, 4)
    assert n_vis >= N
    _, sel, o_csa = pipeline.csa_query(q, qi, rng.standard_normal(2), cmp, ki, N, win, sink, 16,
                                       0.2, t, rd)
    assert np.array_equal(sel[:N], np.arange(N))
    o_hca = oracle.hca_attn(q, cmp, N, win, sink, 0.2, t, rd)
    assert np.allclose(o_csa, o_hca, atol=1e-14)
    keys = np.concatenate([win, cmp, np.zeros((1, D))])
    mask = np.zeros((1, H, 1, keys.shape[0]))
    mask[0, :, 0, -1] = sink
    tk = torch.tensor(keys).reshape(1, 1, -1, D).expand(1, H, -1, D)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q).reshape(1, H, 1, D), tk, tk,
                                                           attn_mask=torch.tensor(mask), scale=0.2)
    ref = oracle.rope(ref.numpy().reshape(H, D), t, rd, inverse=True)
    assert np.allclose(o_csa, ref, atol=1e-13)


def test_inverse_rope_on_output_undoes_a_rotated_single_row():
    """With one candidate and a sink of -inf the output is that row; a row
    rotated at the query position comes back unrotated."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal(64)
    row = oracle.rope(x, 77, 16)
    o = oracle.sparse_attn(rng.standard_normal((2, 64)), row[None], np.array([0]), np.zeros((0, 64)),
                           np.full(2, -np.inf), 1.0, 77, 16)
    assert np.allclose(o, np.stack([x, x]), atol=1e-13)


def test_window_positions():
    assert oracle.window_positions(0, 128) == [0]
    assert oracle.window_positions(5, 4) == [2, 3, 4, 5]
    assert oracle.window_positions(200, 128) == list(range(73, 201))
