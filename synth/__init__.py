"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the attention path's arithmetic.  It only draws
Gaussian numbers, scales rows to unit RMS (a distribution recipe: such rows
are uniform on the sphere of radius sqrt(D)), draws the linear projections of
a Gaussian hidden state for the tiny configuration, and rounds float32 to
bfloat16 bit patterns (round to nearest even).

Every tensor comes from its own stream,
``PCG64(SeedSequence(0, spawn_key=(config_id, tensor_id, b, chunk)))``, so any
sequence ``b`` and any row chunk of a large cache can be regenerated alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CHUNK_ROWS = 16384  # rows per independently seeded chunk of a cache


# ---------------------------------------------------------------------------
# Workload configurations (shapes follow the pages' model: 64 query heads of
# dim 512 on one shared K=V head with RoPE on the trailing 64 dims; a 64x128
# indexer; window 128; top-k 512; CSA ratio 4 with overlap, HCA ratio 128).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    cid: int
    kind: str            # "tiny", "decode" or "prefill"
    B: int
    H: int = 64
    D: int = 512
    rope_dim: int = 64
    H_I: int = 64
    D_I: int = 128
    rope_dim_idx: int = 64
    window: int = 128
    k: int = 512
    ratio: int = 4
    overlap: int = 1
    csa: bool = True     # False: HCA (all visible entries, no indexer)
    S: int = 1           # query tokens per sequence in this call
    ctx: int = 0         # decode: context length N (query at position N-1)
    ctx_lo: int = 0      # decode with a length mix: N_b ~ U{ctx_lo .. ctx}
    T_prefill: int = 0   # tiny: prefill tokens
    T_decode: int = 0    # tiny: streamed decode tokens
    d_model: int = 0     # tiny: hidden width of the projected inputs
    eps: float = 1e-6
    rope_base: float = 10000.0
    dtype: str = "bf16"
    kv4: bool = False    # compressed KV cache stored quantised (FP4 latent, FP8 RoPE tail)
    page_rows: int = 0   # decode: caches held in a shared page pool of pages of this many rows (0: contiguous)


TINY = Config("tiny_csa", 0, "tiny", B=1, H=2, D=32, rope_dim=8, H_I=2, D_I=16,
              rope_dim_idx=8, window=4, k=4, ratio=4, overlap=1, T_prefill=16,
              T_decode=4, d_model=64, dtype="f32")
CSA_DECODE_64K = Config("csa_decode_64k", 1, "decode", B=8, ctx=65536)
HCA_DECODE_1M = Config("hca_decode_1m", 2, "decode", B=4, ctx=1048576, ratio=128,
                       overlap=0, csa=False)
CSA_PREFILL_8K = Config("csa_prefill_8k", 3, "prefill", B=1, S=8192)
CSA_DECODE_1M = Config("csa_decode_1m", 4, "decode", B=32, ctx=1048576, ctx_lo=524288)
# the 64K-context decode with the Pro model's selection width, top-k 1024 ("LLM Atlas:
# DeepSeek", section 19)
CSA_DECODE_64K_K1024 = Config("csa_decode_64k_k1024", 5, "decode", B=8, ctx=65536, k=1024)

# one whole attention block at decode: the low-rank query path, the CSA path
# of csa_decode_64k and the grouped output projection (the Flash widths of
# ProjDims below)
ATTN_BLOCK_DECODE_64K = Config("attn_block_decode_64k", 6, "block", B=8, ctx=65536)

# the two decode workloads with the quantised compressed-KV cache ("Lab tổng hợp
# DeepSeek-V4.1-Flash", section "3 Giải pháp": FP4 E2M1 latent, FP8 E4M3 tail)
CSA_DECODE_64K_KV4 = Config("csa_decode_64k_kv4", 7, "decode", B=8, ctx=65536, kv4=True)
HCA_DECODE_1M_KV4 = Config("hca_decode_1m_kv4", 8, "decode", B=4, ctx=1048576, ratio=128, overlap=0, csa=False,
                           kv4=True)
# the long-context decode with its length mix served from paged caches ("LLM
# Atlas: DeepSeek", section 19: serving cost depends on the sequence-length mix
# and the allocator): the same seeded draw as csa_decode_1m (same stream id),
# its rows in one shared pool of 256-row pages handed out by the page allocator
CSA_DECODE_1M_PAGED = Config("csa_decode_1m_paged", 4, "decode", B=32, ctx=1048576, ctx_lo=524288, page_rows=256)

CONFIGS = {c.name: c for c in (TINY, CSA_DECODE_64K, HCA_DECODE_1M, CSA_PREFILL_8K, CSA_DECODE_1M,
                               CSA_DECODE_64K_K1024, ATTN_BLOCK_DECODE_64K, CSA_DECODE_64K_KV4, HCA_DECODE_1M_KV4,
                               CSA_DECODE_1M_PAGED)}

# tensor ids of the seeded streams
T_X, T_WKV, T_WG, T_WKI, T_WGI, T_WQ, T_WQI, T_WW = 0, 1, 2, 3, 4, 5, 6, 7
T_KV, T_GATE, T_KI, T_GI, T_Q, T_QI, T_W, T_SINK = 10, 11, 12, 13, 14, 15, 16, 17
T_GAMMA, T_GAMMA_I, T_KVCACHE, T_IDXCACHE, T_WIN, T_LEN, T_SCORES, T_SEL = 20, 21, 22, 23, 24, 25, 26, 27
T_GAMMA_W = 28
T_XM, T_WQA, T_GAMMA_Q, T_WQB, T_WOA, T_WOB = 30, 31, 32, 33, 34, 35


# Widths of the projections on either side of the attention (the Flash model:
# "DeepSeek-V4-Flash 架构：一个 token 的旅程", sections "低秩 Q：两次矩阵乘法接起来"
# and "输出投影也分组，并且降低中间维度").
@dataclass(frozen=True)
class ProjDims:
    d_model: int = 4096
    q_rank: int = 1024
    groups: int = 8
    o_rank: int = 1024


FLASH_PROJ = ProjDims()


def stream(cid, tid, b=0, chunk=0):
    """Independent PCG64 stream for (config, tensor, sequence, chunk)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(0, spawn_key=(cid, tid, b, chunk))))


# ---------------------------------------------------------------------------
# bfloat16 helpers (storage format only)
# ---------------------------------------------------------------------------
def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits):
    return bf16_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------------------
# Row distributions
# ---------------------------------------------------------------------------
def gaussian(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def unit_rms(rng, shape):
    """Gaussian rows scaled to unit RMS along the last axis (float32)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= 1.0 / np.sqrt(np.mean(np.square(x, dtype=np.float64), axis=-1, keepdims=True)).astype(np.float32)
    return x


def cache_rows(cid, tid, b, rows, d, lo=0):
    """Rows [lo, rows) of a unit-RMS cache of sequence b, bf16 bits (rows-lo, d).

    Chunk c covers rows [c*CHUNK_ROWS, (c+1)*CHUNK_ROWS) and has its own stream,
    so a row range can be regenerated without drawing the rows before it.
    """
    out = np.empty((rows - lo, d), dtype=np.uint16)
    c0, c1 = lo // CHUNK_ROWS, (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    for c in range(c0, c1):
        a, z = c * CHUNK_ROWS, min((c + 1) * CHUNK_ROWS, rows)
        blk = bf16_bits(unit_rms(stream(cid, tid, b, c), (CHUNK_ROWS, d)))
        s0, s1 = max(a, lo), z
        out[s0 - lo:s1 - lo] = blk[s0 - a:s1 - a]
    return out


def cache_rows_at(cid, tid, b, index, d):
    """Rows at the given indices of the same cache (each chunk drawn once)."""
    index = np.asarray(index, dtype=np.int64)
    out = np.empty((index.size, d), dtype=np.uint16)
    for c in np.unique(index // CHUNK_ROWS):
        blk = bf16_bits(unit_rms(stream(cid, tid, b, int(c)), (CHUNK_ROWS, d)))
        sel = np.nonzero(index // CHUNK_ROWS == c)[0]
        out[sel] = blk[index[sel] - c * CHUNK_ROWS]
    return out


# ---------------------------------------------------------------------------
# Tiny configuration: per-token rows projected from a Gaussian hidden state
# ---------------------------------------------------------------------------
def tiny_inputs(cfg=TINY):
    """x ~ N(0,1)[T, d_model]; projections ~ N(0, 1/d_model); sink ~ N(0,1).

    Returns float32 arrays: kv, gate (T, D); k_idx, g_idx (T, D_I); q
    (T, H, D) and q_idx (T, H_I, D_I) with every head at unit RMS; w (T, H_I)
    scaled by 1/sqrt(D_I)/sqrt(H_I); sink (H,); gammas (1 + 0.1 N(0,1)).
    """
    T = cfg.T_prefill + cfg.T_decode
    d = cfg.d_model
    cid = cfg.cid
    x = gaussian(stream(cid, T_X), (T, d)).astype(np.float64)

    def proj(tid, n):
        return gaussian(stream(cid, tid), (d, n)).astype(np.float64) / np.sqrt(d)

    kv = x @ proj(T_WKV, cfg.D)
    gate = x @ proj(T_WG, cfg.D)
    k_idx = x @ proj(T_WKI, cfg.D_I)
    g_idx = x @ proj(T_WGI, cfg.D_I)
    q = (x @ proj(T_WQ, cfg.H * cfg.D)).reshape(T, cfg.H, cfg.D)
    q /= np.sqrt(np.mean(q * q, axis=-1, keepdims=True))
    q_idx = (x @ proj(T_WQI, cfg.H_I * cfg.D_I)).reshape(T, cfg.H_I, cfg.D_I)
    q_idx /= np.sqrt(np.mean(q_idx * q_idx, axis=-1, keepdims=True))
    w = (x @ proj(T_WW, cfg.H_I)) / np.sqrt(cfg.D_I) / np.sqrt(cfg.H_I)
    sink = gaussian(stream(cid, T_SINK), (cfg.H,))
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return dict(
        kv=f(kv), gate=f(gate), k_idx=f(k_idx), g_idx=f(g_idx), q=f(q), q_idx=f(q_idx),
        w=f(w), sink=f(sink),
        gamma=f(1.0 + 0.1 * gaussian(stream(cid, T_GAMMA), (cfg.D,))),
        gamma_idx=f(1.0 + 0.1 * gaussian(stream(cid, T_GAMMA_I), (cfg.D_I,))),
        gamma_win=f(1.0 + 0.1 * gaussian(stream(cid, T_GAMMA_W), (cfg.D,))),
    )


# ---------------------------------------------------------------------------
# Decode configurations
# ---------------------------------------------------------------------------
def decode_lengths(cfg):
    """Context length N_b of every sequence (query at position N_b - 1)."""
    if cfg.ctx_lo:
        return stream(cfg.cid, T_LEN).integers(cfg.ctx_lo, cfg.ctx, size=cfg.B, endpoint=True).astype(np.int64)
    return np.full(cfg.B, cfg.ctx, dtype=np.int64)


def decode_capacity(cfg):
    """Compressed-cache rows allocated per sequence."""
    return cfg.ctx // cfg.ratio


def staging_rows(cfg):
    """Per-token rows kept for the compressor: (1 + overlap) groups."""
    return (1 + cfg.overlap) * cfg.ratio


@dataclass
class DecodeSeq:
    """Inputs of one decode query (sequence b), bf16 as uint16 bits."""
    b: int
    pos: int
    n_vis: int
    q: np.ndarray         # (H, D)
    q_idx: np.ndarray     # (H_I, D_I) (CSA only)
    w: np.ndarray         # (H_I,) float32 (CSA only)
    win: np.ndarray       # (window, D): ring slots, slot = p % window
    kv_stage: np.ndarray  # (R, D): slot = token % R, R = staging_rows
    gate_stage: np.ndarray
    ki_stage: np.ndarray  # (R, D_I) (CSA only)
    gi_stage: np.ndarray
    extra: dict = field(default_factory=dict)


def decode_seq(cfg, b, lengths=None):
    """Query-side inputs and compressor staging rows of sequence b."""
    lengths = decode_lengths(cfg) if lengths is None else lengths
    n = int(lengths[b])
    pos = n - 1
    cid = cfg.cid
    R = staging_rows(cfg)
    rq = stream(cid, T_Q, b)
    q = bf16_bits(unit_rms(rq, (cfg.H, cfg.D)))
    win = bf16_bits(unit_rms(stream(cid, T_WIN, b), (cfg.window, cfg.D)))
    kv_stage = bf16_bits(gaussian(stream(cid, T_KV, b), (R, cfg.D)))
    gate_stage = bf16_bits(gaussian(stream(cid, T_GATE, b), (R, cfg.D)))
    if cfg.csa:
        q_idx = bf16_bits(unit_rms(stream(cid, T_QI, b), (cfg.H_I, cfg.D_I)))
        w = (gaussian(stream(cid, T_W, b), (cfg.H_I,)) / np.sqrt(cfg.D_I) / np.sqrt(cfg.H_I)).astype(np.float32)
        ki_stage = bf16_bits(gaussian(stream(cid, T_KI, b), (R, cfg.D_I)))
        gi_stage = bf16_bits(gaussian(stream(cid, T_GI, b), (R, cfg.D_I)))
    else:
        q_idx = np.zeros((0, 0), np.uint16)
        w = np.zeros((0,), np.float32)
        ki_stage = gi_stage = np.zeros((0, 0), np.uint16)
    return DecodeSeq(b=b, pos=pos, n_vis=n // cfg.ratio, q=q, q_idx=q_idx, w=w, win=win,
                     kv_stage=kv_stage, gate_stage=gate_stage, ki_stage=ki_stage, gi_stage=gi_stage)


def decode_shared(cfg):
    """Per-layer parameters: sink (H,), compressor gammas."""
    cid = cfg.cid
    return dict(
        sink=gaussian(stream(cid, T_SINK), (cfg.H,)),
        gamma=(1.0 + 0.1 * gaussian(stream(cid, T_GAMMA), (cfg.D,))).astype(np.float32),
        gamma_idx=(1.0 + 0.1 * gaussian(stream(cid, T_GAMMA_I), (cfg.D_I,))).astype(np.float32),
    )


def kv_cache_rows(cfg, b, rows, lo=0):
    """Pre-filled compressed KV cache rows [lo, rows) of sequence b (bf16 bits)."""
    return cache_rows(cfg.cid, T_KVCACHE, b, rows, cfg.D, lo)


def kv_cache_rows_at(cfg, b, index):
    """Pre-filled compressed KV cache rows at the given indices of sequence b."""
    return cache_rows_at(cfg.cid, T_KVCACHE, b, index, cfg.D)


def idx_cache_rows(cfg, b, rows, lo=0):
    """Pre-filled compressed index-key cache rows [lo, rows) of sequence b."""
    return cache_rows(cfg.cid, T_IDXCACHE, b, rows, cfg.D_I, lo)


# ---------------------------------------------------------------------------
# Prefill configuration
# ---------------------------------------------------------------------------
def prefill_inputs(cfg, b=0, q_rows=None):
    """Per-token inputs of one prefill sequence (bf16 bits unless noted).

    kv, gate (S, D) and k_idx, g_idx (S, D_I) ~ N(0,1); win (S, D), the
    per-token window rows, at unit RMS; q (S, H, D) and q_idx (S, H_I, D_I)
    with unit-RMS heads; w (S, H_I) float32 ~ N(0,1)/sqrt(D_I)/sqrt(H_I).
    ``q_rows`` restricts the query-side tensors to the given token indices
    (each token's query rows come from their own chunk stream).
    """
    cid, S = cfg.cid, cfg.S
    out = dict(
        kv=bf16_bits(gaussian(stream(cid, T_KV, b), (S, cfg.D))),
        gate=bf16_bits(gaussian(stream(cid, T_GATE, b), (S, cfg.D))),
        k_idx=bf16_bits(gaussian(stream(cid, T_KI, b), (S, cfg.D_I))),
        g_idx=bf16_bits(gaussian(stream(cid, T_GI, b), (S, cfg.D_I))),
        win=cache_rows(cid, T_WIN, b, S, cfg.D),
    )
    rows = np.arange(S) if q_rows is None else np.asarray(q_rows)
    qc = 256  # query tokens per seeded chunk
    q = np.empty((rows.size, cfg.H, cfg.D), np.uint16)
    qi = np.empty((rows.size, cfg.H_I, cfg.D_I), np.uint16)
    w = np.empty((rows.size, cfg.H_I), np.float32)
    chunks = {}
    for j, t in enumerate(rows):
        c = int(t) // qc
        if c not in chunks:
            chunks = {c: (
                bf16_bits(unit_rms(stream(cid, T_Q, b, c), (qc, cfg.H, cfg.D))),
                bf16_bits(unit_rms(stream(cid, T_QI, b, c), (qc, cfg.H_I, cfg.D_I))),
                (gaussian(stream(cid, T_W, b, c), (qc, cfg.H_I)) / np.sqrt(cfg.D_I) / np.sqrt(cfg.H_I)).astype(np.float32),
            )}
        cq, cqi, cw = chunks[c]
        q[j], qi[j], w[j] = cq[int(t) % qc], cqi[int(t) % qc], cw[int(t) % qc]
    out.update(q=q, q_idx=qi, w=w)
    return out


# ---------------------------------------------------------------------------
# Stand-alone top-k inputs
# ---------------------------------------------------------------------------
def topk_scores(cid, R, N, tie_frac=0.05, b=0):
    """float32 scores (R, N) ~ N(0,1) with a share of exact ties planted."""
    rng = stream(cid, T_SCORES, b)
    s = rng.standard_normal((R, N), dtype=np.float32)
    n_tie = int(tie_frac * N)
    if n_tie:
        for r in range(R):
            src = rng.integers(0, N, size=n_tie)
            dst = rng.integers(0, N, size=n_tie)
            s[r, dst] = s[r, src]
    return s


def random_selection(cid, n_vis, k, b=0, t=0):
    """A valid top-k shaped selection: distinct visible entries, ascending, -1 padded."""
    rng = stream(cid, T_SEL, b, t)
    m = min(k, n_vis)
    sel = np.sort(rng.choice(n_vis, size=m, replace=False)) if m else np.zeros(0, np.int64)
    out = np.full(k, -1, np.int32)
    out[:m] = sel
    return out


# ---------------------------------------------------------------------------
# Projection weights and hidden states (random init of the Flash widths)
# ---------------------------------------------------------------------------
def proj_weights(cid, H=64, D=512, dims=FLASH_PROJ):
    """bf16 bits of the query-path and output-projection weights, each drawn
    N(0, 1/fan_in); the latent's RMSNorm gain 1 + 0.1 N(0,1) (float32).

    wq_a (q_rank, d_model), wq_b (H*D, q_rank), wo_a (groups, o_rank,
    H*D/groups), wo_b (d_model, groups*o_rank)."""
    def w(tid, shape, fan_in):
        x = gaussian(stream(cid, tid), shape)
        x *= np.float32(1.0 / np.sqrt(fan_in))
        return bf16_bits(x)
    hd = H * D
    return dict(
        wq_a=w(T_WQA, (dims.q_rank, dims.d_model), dims.d_model),
        gamma_q=(1.0 + 0.1 * gaussian(stream(cid, T_GAMMA_Q), (dims.q_rank,))).astype(np.float32),
        wq_b=w(T_WQB, (hd, dims.q_rank), dims.q_rank),
        wo_a=w(T_WOA, (dims.groups, dims.o_rank, hd // dims.groups), hd // dims.groups),
        wo_b=w(T_WOB, (dims.d_model, dims.groups * dims.o_rank), dims.groups * dims.o_rank),
    )


def hidden_states(cid, M, d_model, b=0):
    """Token hidden states x ~ N(0, 1), (M, d_model) bf16 bits."""
    return bf16_bits(gaussian(stream(cid, T_XM, b), (M, d_model)))
