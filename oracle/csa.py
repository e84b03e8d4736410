"""Float64 CPU oracle for the CSA / HCA compressed-KV attention path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and this module imports
nothing from the product path.

Every function is the plain definition of one step, written in float64 with
NumPy, in the order and notation of the pages it follows.  Sources are cited
by page title and section:

* [V4-Flash walkthrough] "DeepSeek-V4-Flash 架构：一个 token 的旅程"
  (hs-black.github.io/posts/deepseek-v4-flash/).
* [V4.1 lab] "Lab tổng hợp DeepSeek-V4.1-Flash"
  (openarchlab.com, dsv41-end-to-end-lab).
* [LLM Atlas] "LLM Atlas: DeepSeek" (llm-atlas.k1412.top/deepseek/),
  §19 "V4 / HETEROGENEOUS STATE MACHINE".

Readings taken where the pages are silent (each one is listed, with its
reason, in the design notes of the repository):

* RoPE rotates interleaved pairs (2i, 2i+1) of the trailing ``rope_dim``
  channels by ``pos * base**(-2i/rope_dim)``; the inverse rotation uses the
  negated angle.
* A compressed entry ``e`` of ratio ``r`` sits at position ``e * r``.
* RMSNorm is ``y / sqrt(mean(y**2) + eps) * gamma``.
* Candidates whose gate is -inf (the previous group of entry 0) are left out
  of the softmax; their weight is exactly zero and their value is never read.
* The indexer applies ReLU to each head's dot product; the 1/sqrt scale lives
  in ``w`` only.
* Attention logits are ``q . kv * scale``; K and V are the same row; the sink
  is a raw logit that enters the denominator only.
* The sliding window holds positions ``max(0, t-W+1) .. t`` (self included).
* Top-k keeps the k largest finite scores among the visible entries, ties to
  the lower index; the result is returned as an ascending index list padded
  with -1.

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import numpy as np

NEG_INF = float("-inf")


# ---------------------------------------------------------------------------
# Positional rotation and normalisation
# ---------------------------------------------------------------------------
def rope(x, pos, rope_dim, base=10000.0, inverse=False):
    """Rotate the trailing ``rope_dim`` channels of ``x`` at position ``pos``.

    [V4-Flash walkthrough, "低秩 Q：两次矩阵乘法接起来"]: only the last 64 of
    the 512 query channels are rotated.  [LLM Atlas §19]: rotary position is
    encoded on part of the dimensions only.  The pair convention, the base
    and the angle are the readings stated in the module header.  ``pos`` is a
    scalar or an integer array of shape ``x.shape[:-1]``.  ``inverse=True``
    applies the transpose rotation, used on the attention output
    [V4-Flash walkthrough, "输出投影也分组，并且降低中间维度"].
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return x
    d = x.shape[-1]
    half = rope_dim // 2
    i = np.arange(half, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / rope_dim)
    angle = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(angle), np.sin(angle)
    if inverse:
        sin = -sin
    tail = x[..., d - rope_dim:]
    even = tail[..., 0::2].copy()
    odd = tail[..., 1::2].copy()
    tail[..., 0::2] = even * cos - odd * sin
    tail[..., 1::2] = even * sin + odd * cos
    return x


def round_bf16(x):
    """Value of x after storage as bfloat16 (round to nearest, ties to even).

    The compressed caches of the bf16 workloads are stored as bfloat16: the
    8 exponent bits of float32 and its top 7 fraction bits.  x is first
    rounded to float32 (nearest even), then the low 16 bits of that float32
    are rounded away (nearest even).  Finite inputs only.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    keep = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & 1) == 1))
    keep = (keep + up.astype(np.uint64)) & 0xFFFF
    return (keep.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rms_norm(y, gamma, eps):
    """RMSNorm over the last axis, ``y / sqrt(mean(y^2) + eps) * gamma``.

    [V4-Flash walkthrough, "压缩是逐通道的 learned pooling"]: pooled entries
    are RMS-normalised before the rotation.
    """
    y = np.asarray(y, dtype=np.float64)
    ms = np.mean(y * y, axis=-1, keepdims=True)
    return y / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


# ---------------------------------------------------------------------------
# Compressor
# ---------------------------------------------------------------------------
def pool(gates, values):
    """Per-channel learned softmax pooling of one candidate list (pre-norm).

    [V4-Flash walkthrough, "压缩是逐通道的 learned pooling"]: the softmax runs
    along the token axis, separately for every channel.
    [V4-Flash walkthrough, "一个通道，逐项算出压缩结果"]: a candidate whose
    gate is -inf gets weight zero.  Such candidates are dropped from the list
    before the softmax, so their value is never multiplied.

    gates, values: (C, D) arrays (C candidates).  Returns (D,).
    """
    g = np.asarray(gates, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    keep = g != NEG_INF                                   # (C, D)
    with np.errstate(invalid="ignore"):
        m = np.max(np.where(keep, g, NEG_INF), axis=0)    # per-channel max
        e = np.where(keep, np.exp(g - m), 0.0)            # softmax numerators
        num = np.sum(np.where(keep, e * v, 0.0), axis=0)
    den = np.sum(e, axis=0)
    out = np.zeros(g.shape[1], dtype=np.float64)
    np.divide(num, den, out=out, where=den > 0)
    return out


def entry_candidates(e, ratio, overlap):
    """Token indices pooled into compressed entry ``e``.

    Returns (previous-role tokens, current-role tokens).  The current group of
    entry e is tokens [e*r, (e+1)*r); with overlap, the previous group
    [(e-1)*r, e*r) is added, and for e == 0 that group does not exist (its
    gates are -inf) [V4-Flash walkthrough, "一个通道，逐项算出压缩结果"].
    """
    cur = list(range(e * ratio, (e + 1) * ratio))
    prev = list(range((e - 1) * ratio, e * ratio)) if (overlap and e >= 1) else []
    return prev, cur


def compress_entry(e, kv, gate, kv_prev, gate_prev, gamma, ratio, overlap,
                   rope_dim, rope_base, eps):
    """One compressed entry: pool, then RMSNorm, then RoPE at position e*r.

    [V4-Flash walkthrough, "压缩是逐通道的 learned pooling"].  ``kv``/``gate``
    are (T, D) per-token rows of the current role; ``kv_prev``/``gate_prev``
    those of the previous role (they may be the same arrays).
    """
    prev, cur = entry_candidates(e, ratio, overlap)
    g = [gate_prev[t] for t in prev] + [gate[t] for t in cur]
    v = [kv_prev[t] for t in prev] + [kv[t] for t in cur]
    return entry_from_rows(e, ratio, np.stack(g), np.stack(v), gamma, rope_dim, rope_base, eps)


def entry_from_rows(e, ratio, gates, values, gamma, rope_dim, rope_base=10000.0, eps=1e-6):
    """Entry e from its candidate rows (previous group first, then current).

    Pool, RMSNorm, then RoPE at the entry position e*ratio
    [V4-Flash walkthrough, "压缩是逐通道的 learned pooling"].
    """
    y = pool(gates, values)
    y = rms_norm(y, gamma, eps)
    return rope(y, e * ratio, rope_dim, rope_base)


def compress(kv, gate, gamma, ratio, overlap, rope_dim, rope_base=10000.0,
             eps=1e-6, kv_prev=None, gate_prev=None, n_entries=None):
    """All compressed entries of one sequence, computed as in prefill.

    [V4-Flash walkthrough, "压缩条目必须等整组完成后才可见"]: prefill may build
    every entry of the span at once; entry e exists once tokens up to
    (e+1)*r - 1 are present.  Returns (n_entries, D), n_entries defaulting to
    T // r.
    """
    kv = np.asarray(kv, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    kv_prev = kv if kv_prev is None else np.asarray(kv_prev, dtype=np.float64)
    gate_prev = gate if gate_prev is None else np.asarray(gate_prev, dtype=np.float64)
    n = kv.shape[0] // ratio if n_entries is None else n_entries
    out = np.zeros((n, kv.shape[1]), dtype=np.float64)
    for e in range(n):
        out[e] = compress_entry(e, kv, gate, kv_prev, gate_prev, gamma, ratio,
                                overlap, rope_dim, rope_base, eps)
    return out


class StreamingCompressor:
    """Token-by-token compressor that only ever sees tokens <= t.

    [V4-Flash walkthrough, "压缩条目必须等整组完成后才可见"]: when
    ``(t+1) % ratio == 0`` the completed group is pooled into cache slot
    ``t // ratio``; before that, nothing of the group is visible.
    """

    def __init__(self, gamma, ratio, overlap, rope_dim, rope_base=10000.0, eps=1e-6):
        self.gamma, self.ratio, self.overlap = gamma, ratio, overlap
        self.rope_dim, self.rope_base, self.eps = rope_dim, rope_base, eps
        self.kv, self.gate, self.kv_prev, self.gate_prev = [], [], [], []
        self.cache = []

    def push(self, t, kv_t, gate_t, kv_prev_t=None, gate_prev_t=None):
        """Append token t; returns the slot index emitted at t, or None."""
        assert t == len(self.kv)
        self.kv.append(np.asarray(kv_t, dtype=np.float64))
        self.gate.append(np.asarray(gate_t, dtype=np.float64))
        self.kv_prev.append(self.kv[-1] if kv_prev_t is None else np.asarray(kv_prev_t, dtype=np.float64))
        self.gate_prev.append(self.gate[-1] if gate_prev_t is None else np.asarray(gate_prev_t, dtype=np.float64))
        if (t + 1) % self.ratio != 0:
            return None
        e = t // self.ratio
        assert e == len(self.cache)
        self.cache.append(compress_entry(e, self.kv, self.gate, self.kv_prev, self.gate_prev,
                                         self.gamma, self.ratio, self.overlap,
                                         self.rope_dim, self.rope_base, self.eps))
        return e


def visible(t, ratio):
    """Number of compressed entries a query at position t may read.

    [V4-Flash walkthrough, "压缩条目必须等整组完成后才可见"]: (t+1) // ratio.
    """
    return (t + 1) // ratio


# ---------------------------------------------------------------------------
# Indexer and top-k
# ---------------------------------------------------------------------------
def index_score(q_idx, w, idx_cache, n_vis):
    """Indexer score of every compressed entry for one query.

    [V4-Flash walkthrough, "少读 KV 之前，Indexer 仍要给历史打分"]: 64 heads of
    dim 128 score a single shared 128-d index cache with signed per-head
    weights w.  [V4.1 lab, "3 Giải pháp"]: a ReLU acts on each head's dot
    product before the weighting.  Entries at or beyond ``n_vis`` get -inf.

    q_idx: (H_I, D_I); w: (H_I,); idx_cache: (N, D_I).  Returns (N,).
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(idx_cache, dtype=np.float64)
    n = k.shape[0]
    out = np.full(n, NEG_INF, dtype=np.float64)
    m = min(n_vis, n)
    if m > 0:
        dots = k[:m] @ q_idx.T             # (m, H_I)
        out[:m] = np.maximum(dots, 0.0) @ w
    return out


def topk(scores, n_valid, k):
    """The k best visible entries of one score row.

    [V4-Flash walkthrough, "少读 KV 之前，Indexer 仍要给历史打分"]: top-k picks
    the entries the main attention reads.  [LLM Atlas §19]: the Flash model
    uses k = 512.  Order: larger score first, ties to the lower index; -inf
    scores are never picked.  Returns int64 (k,) ascending, padded with -1.
    """
    s = np.asarray(scores, dtype=np.float64)[:n_valid]
    cand = np.nonzero(s != NEG_INF)[0]
    order = np.lexsort((cand, -s[cand]))   # primary: -score; secondary: index
    chosen = np.sort(cand[order[:k]])
    out = np.full(k, -1, dtype=np.int64)
    out[:chosen.size] = chosen
    return out


# ---------------------------------------------------------------------------
# Joint-softmax attention with a sink
# ---------------------------------------------------------------------------
def window_positions(t, window):
    """Positions of the sliding window of a query at t: max(0,t-W+1) .. t."""
    return list(range(max(0, t - window + 1), t + 1))


def attend(q, rows, sink, scale):
    """Softmax attention of H query heads over one shared K=V row set.

    [V4-Flash walkthrough, "局部和压缩记忆，共用一次归一化"]: window entries and
    compressed entries form one candidate set under one normalisation; the
    per-head sink adds to the denominator and carries no value.

    q: (H, D); rows: (C, D); sink: (H,).  Returns (H, D) before the inverse
    rotation.
    """
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64).reshape(-1, q.shape[1])
    sink = np.asarray(sink, dtype=np.float64)
    logits = (q @ rows.T) * scale                       # (H, C)
    if rows.shape[0]:
        m = np.maximum(logits.max(axis=1), sink)
    else:
        m = sink.copy()
    p = np.exp(logits - m[:, None])
    denom = p.sum(axis=1) + np.exp(sink - m)
    return (p @ rows) / denom[:, None]


def sparse_attn(q, cmp, sel, win_rows, sink, scale, pos, rope_dim, rope_base=10000.0):
    """CSA attention of one query: window rows plus the selected entries.

    [V4-Flash walkthrough, "局部和压缩记忆，共用一次归一化"] and
    ["输出投影也分组，并且降低中间维度"]: after the joint softmax the output is
    rotated back by the query position.  ``sel`` holds entry indices, -1
    entries are skipped.  ``win_rows`` is (W', D), the window rows in position
    order.
    """
    cmp = np.asarray(cmp, dtype=np.float64)
    picked = [cmp[i] for i in np.asarray(sel).ravel() if i >= 0]
    rows = list(np.asarray(win_rows, dtype=np.float64).reshape(-1, cmp.shape[1])) + picked
    rows = np.stack(rows) if rows else np.zeros((0, cmp.shape[1]))
    o = attend(q, rows, sink, scale)
    return rope(o, pos, rope_dim, rope_base, inverse=True)


def hca_attn(q, cmp, n_vis, win_rows, sink, scale, pos, rope_dim, rope_base=10000.0):
    """HCA attention of one query: window rows plus every visible entry.

    [LLM Atlas §19]: HCA keeps all compressed entries and skips the top-k.
    """
    return sparse_attn(q, cmp, np.arange(n_vis), win_rows, sink, scale, pos,
                       rope_dim, rope_base)
