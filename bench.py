#!/usr/bin/env python3
"""Benchmark of the CSA / HCA compressed-KV attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload csa_decode_64k] [--extra ...]

A step is one pass of the whole path over one batch of synthetic inputs that
are already resident in HBM:
  decode (CSA):  append the completed group to both compressed caches (KV and
                 index keys), score every visible entry, top-k, sparse attention
  decode (HCA):  append to the compressed KV cache, attention over all entries
  prefill (CSA): compress every group of both roles, score, top-k, attention
Each step reads its caches from one of 16 copies in rotation, so the 256 MiB
Infinity Cache cannot serve the stream.  Steps are replayed from HIP graphs
(one graph per copy).  Per-kernel durations are measured with HIP events in an
eager pass queued behind a GPU spin (so launches run back to back).

Prints ONE JSON line (rank 0).  The CPU baseline is the float64 oracle run on
a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "decode query-tokens/s + achieved HBM GB/s at 64K/1M ctx; prefill indexer MFMA util"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
COPIES = 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="csa_decode_64k", choices=sorted(synth.CONFIGS))
    ap.add_argument("--extra", default="hca_decode_1m,csa_decode_1m,csa_prefill_8k,csa_decode_64k_k1024,"
                    "attn_block_decode_64k,csa_decode_64k_kv4,hca_decode_1m_kv4,csa_decode_1m_paged",
                    help="comma-separated secondary workloads measured after the main one ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-only", default="", help="profiling aid: replay only this kernel's graphs")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="counter reference: copy MIB MiB device-to-device 8 times and exit")
    return ap.parse_args()


def copy_probe(mib):
    """A plain copy of known size, to scale the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_copy": n * 4, "copies": 8}), flush=True)


# ---------------------------------------------------------------------------
# Device workloads
# ---------------------------------------------------------------------------
def _bf16(bits, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def _f32(x, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def _fill_cache(dst, cid, tid, rows, device):
    """dst[b, :rows[b]] = the seeded cache rows of sequence b, drawn chunk by
    chunk on a thread pool (the generator releases the GIL while drawing)."""
    from concurrent.futures import ThreadPoolExecutor
    d = dst.shape[-1]
    jobs = [(b, c) for b in range(dst.shape[0]) for c in range((int(rows[b]) + synth.CHUNK_ROWS - 1) // synth.CHUNK_ROWS)]

    def one(job):
        b, c = job
        lo, hi = c * synth.CHUNK_ROWS, min((c + 1) * synth.CHUNK_ROWS, int(rows[b]))
        blk = synth.cache_rows(cid, tid, b, hi, d, lo)
        dst[b, lo:hi] = _bf16(blk, device)

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
        list(ex.map(one, jobs))


class DecodeWorkload:
    """One decode step for B sequences (CSA or HCA) on rotated cache copies."""

    def __init__(self, cfg, device, copies=COPIES, batch=None):
        import torch
        lengths = synth.decode_lengths(cfg)
        if batch is not None:  # the first `batch` sequences of the workload's draw
            import dataclasses
            cfg = dataclasses.replace(cfg, B=batch)
            lengths = lengths[:batch]
        self.cfg, self.device = cfg, device
        B, D, DI = cfg.B, cfg.D, cfg.D_I
        self.lengths = lengths
        self.Ncap = synth.decode_capacity(cfg)
        self.R = synth.staging_rows(cfg)
        self.seqs = [synth.decode_seq(cfg, b, self.lengths) for b in range(B)]
        shared = synth.decode_shared(cfg)
        self.pos_np = np.array([s.pos for s in self.seqs], np.int32)
        self.n_vis = np.array([s.n_vis for s in self.seqs], np.int64)
        self.pos = torch.from_numpy(self.pos_np).to(device)
        self.pos2 = self.pos.view(B, 1)
        self.sink = _f32(shared["sink"], device)
        self.gamma = _f32(shared["gamma"], device)
        self.gamma_idx = _f32(shared["gamma_idx"], device)
        self.q = _bf16(np.stack([s.q for s in self.seqs])[:, None], device)
        self.win = _bf16(np.stack([s.win for s in self.seqs]), device)
        self.kv_stage = _bf16(np.stack([s.kv_stage for s in self.seqs]), device)
        self.gate_stage = _bf16(np.stack([s.gate_stage for s in self.seqs]), device)
        # caches: the first copy from the seeded generator (the visible rows of
        # every sequence; rows past them are never read and stay zero), the
        # others device copies
        self.copies = copies if cfg.ctx_lo == 0 else 1
        kv0 = torch.zeros((B, self.Ncap, D), dtype=torch.bfloat16, device=device)
        _fill_cache(kv0, cfg.cid, synth.T_KVCACHE, self.n_vis, device)
        if cfg.kv4:  # the quantised cache of the same rows (quantised by the library itself)
            import compressed_sparse_attention_06_amd as csa
            self.kv_row_bytes = csa.csa_kv4_row_bytes(D, cfg.rope_dim)
            q0 = torch.empty((B, self.Ncap, self.kv_row_bytes), dtype=torch.uint8, device=device)
            csa.csa_kv4_quantize(kv0, q0, rope_dim=cfg.rope_dim)
            del kv0
            kv0 = q0
        else:
            self.kv_row_bytes = D * 2
        self.kv = [kv0] + [kv0.clone() for _ in range(self.copies - 1)]
        self.out = torch.empty((B, 1, cfg.H, D), dtype=torch.float32, device=device)
        if cfg.csa:
            self.q_idx = _bf16(np.stack([s.q_idx for s in self.seqs])[:, None], device)
            self.w = _f32(np.stack([s.w for s in self.seqs])[:, None], device)
            self.ki_stage = _bf16(np.stack([s.ki_stage for s in self.seqs]), device)
            self.gi_stage = _bf16(np.stack([s.gi_stage for s in self.seqs]), device)
            ic0 = torch.zeros((B, self.Ncap, DI), dtype=torch.bfloat16, device=device)
            _fill_cache(ic0, cfg.cid, synth.T_IDXCACHE, self.n_vis, device)
            self.idx_cache = [ic0] + [ic0.clone() for _ in range(self.copies - 1)]
            self.scores = torch.empty((B, 1, self.Ncap), dtype=torch.float32, device=device)
            self.sel = torch.empty((B, 1, cfg.k), dtype=torch.int32, device=device)
            import compressed_sparse_attention_06_amd as csa
            self.ws_topk = torch.empty(max(1, csa.csa_topk_workspace_size(B, self.Ncap, cfg.k)), dtype=torch.uint8,
                                       device=device)
            self.ws_attn = torch.empty(max(1, csa.csa_sparse_attn_workspace_size(B, 1, cfg.H, D, cfg.k, cfg.window)),
                                       dtype=torch.uint8, device=device)
        else:
            import compressed_sparse_attention_06_amd as csa
            self.ws_attn = torch.empty(max(1, csa.hca_attn_workspace_size(B, 1, cfg.H, D, self.Ncap, cfg.window)),
                                       dtype=torch.uint8, device=device)
        # compressor workspaces: zero-filled once, one per role (the roles may run concurrently)
        self.ws_ckv = torch.zeros(max(16, csa.csa_compress_workspace_size(B, D, cfg.ratio, cfg.overlap)),
                                  dtype=torch.uint8, device=device)
        self.ws_cidx = torch.zeros(max(16, csa.csa_compress_workspace_size(B, cfg.D_I, cfg.ratio, cfg.overlap)),
                                   dtype=torch.uint8, device=device)
        torch.cuda.synchronize()

    # A decode step stays on one stream: in a replayed graph, a fork to a side
    # stream and the join before the attention cost more (about 10 us) than
    # the KV-role compressor they would hide.
    side_kernels = ()

    # the kernels of one step, as (name, callable) in launch order
    def launches(self, c):
        import compressed_sparse_attention_06_amd as csa
        cfg = self.cfg
        c = c % self.copies
        scale = 1.0 / math.sqrt(cfg.D)
        kv_job = dict(kv=self.kv_stage, gate=self.gate_stage, gamma=self.gamma, out=self.kv[c], ratio=cfg.ratio,
                      overlap=cfg.overlap, rope_dim=cfg.rope_dim, rope_base=cfg.rope_base, eps=cfg.eps, pos=self.pos,
                      ws=self.ws_ckv)
        if cfg.csa:
            # both cache appends (KV entries, index keys) in one compressor launch
            idx_job = dict(kv=self.ki_stage, gate=self.gi_stage, gamma=self.gamma_idx, out=self.idx_cache[c],
                           ratio=cfg.ratio, overlap=cfg.overlap, rope_dim=cfg.rope_dim_idx, rope_base=cfg.rope_base,
                           eps=cfg.eps, pos=self.pos, ws=self.ws_cidx)
            L = [
                ("compress", lambda: csa.csa_compress_jobs([kv_job, idx_job])),
                ("index_score", lambda: csa.csa_index_score(self.q_idx, self.w, self.idx_cache[c], self.pos2,
                                                            self.scores, ratio=cfg.ratio)),
                ("topk", lambda: csa.csa_topk(self.scores.view(cfg.B, self.Ncap), None, cfg.k,
                                              self.sel.view(cfg.B, cfg.k), ws=self.ws_topk)),
                ("sparse_attn", lambda: csa.csa_sparse_attn(
                    self.q, self.kv[c], self.sel, self.win, self.pos2, self.sink, self.out, window=cfg.window,
                    scale=scale, rope_dim=cfg.rope_dim, rope_base=cfg.rope_base, ws=self.ws_attn)),
            ]
        else:
            L = [
                ("compress", lambda: csa.csa_compress(**kv_job)),
                ("hca_attn", lambda: csa.hca_attn(
                    self.q, self.kv[c], self.win, self.pos2, self.sink, self.out, ratio=cfg.ratio, window=cfg.window,
                    scale=scale, rope_dim=cfg.rope_dim, rope_base=cfg.rope_base, ws=self.ws_attn)),
            ]
        return L

    def queries(self):
        return self.cfg.B

    def dominant(self):
        return "index_score" if self.cfg.csa else "hca_attn"

    def algorithmic(self):
        """Algorithmic HBM bytes of each kernel of one step (and flops)."""
        cfg, B = self.cfg, self.cfg.B
        D, DI, H, HI = cfg.D, cfg.D_I, cfg.H, cfg.H_I
        emit = int(np.sum((self.pos_np + 1) % cfg.ratio == 0))
        rows_in = (1 + cfg.overlap) * cfg.ratio
        vis = self.n_vis
        win = np.minimum(cfg.window, self.pos_np + 1)
        rb = self.kv_row_bytes  # a compressed KV row: 1 KiB in bf16, 304 B quantised
        by = {"compress": emit * (2 * rows_in * D * 2 + rb) + D * 4}
        fl = {}
        if cfg.csa:
            by["compress"] += emit * (2 * rows_in * DI * 2 + DI * 2) + DI * 4
            by["index_score"] = int(np.sum(vis * DI * 2) + B * (HI * DI * 2 + HI * 4) + B * self.Ncap * 4)
            fl["index_score"] = int(np.sum(vis) * HI * DI * 2)
            by["topk"] = int(B * self.Ncap * 4 + B * cfg.k * 4)
            sel = np.minimum(vis, cfg.k)
            by["sparse_attn"] = int(np.sum(sel * rb + win * D * 2) + B * (H * D * 2 + cfg.k * 4 + H * D * 4))
            fl["sparse_attn"] = int(np.sum(sel + win) * H * D * 4)
        else:
            by["hca_attn"] = int(np.sum(vis * rb + win * D * 2) + B * (H * D * 2 + H * D * 4))
            fl["hca_attn"] = int(np.sum(vis + win) * H * D * 4)
        return by, fl

    def unit(self):
        return "per visible index row: 256 B read (64x128 heads: 16,384 flop)" if self.cfg.csa else \
            f"per attended KV row: {self.kv_row_bytes:,} B read (64 heads x 512: 131,072 flop)"

    def describe(self):
        cfg = self.cfg
        d = dict(workload=cfg.name, batch=cfg.B, context=int(cfg.ctx) if not cfg.ctx_lo else
                 [int(cfg.ctx_lo), int(cfg.ctx)], compressed_entries=int(np.max(self.n_vis)), ratio=cfg.ratio,
                 heads=cfg.H, head_dim=cfg.D, rope_dim=cfg.rope_dim, window=cfg.window, cache_copies=self.copies,
                 kv_cache="fp4 e2m1 latent + fp8 e4m3 rope tail, 304 B/row" if cfg.kv4 else "bf16, 1024 B/row")
        if cfg.csa:
            d.update(index_heads=cfg.H_I, index_dim=cfg.D_I, top_k=cfg.k)
        return d


class BlockWorkload(DecodeWorkload):
    """One whole attention block at decode: the low-rank query path
    (csa_q_proj) makes the queries the CSA step attends with, the CSA decode
    step runs as in DecodeWorkload (its attention output in bf16), and the
    grouped output projection (csa_out_proj) maps it back to the model width.
    The 200 MiB of projection weights rotate over 4 copies, so the Infinity
    Cache cannot serve them either."""

    WEIGHT_COPIES = 4

    def __init__(self, cfg, device, copies=COPIES, batch=None):
        import torch
        import compressed_sparse_attention_06_amd as csa
        super().__init__(cfg, device, copies=copies, batch=batch)
        dims = synth.FLASH_PROJ
        self.dims = dims
        B, H, D = self.cfg.B, self.cfg.H, self.cfg.D
        wts = synth.proj_weights(self.cfg.cid, H, D, dims)
        self.gamma_q = _f32(wts["gamma_q"], device)
        self.wcopies = self.WEIGHT_COPIES
        self.wts = {}
        for name in ("wq_a", "wq_b", "wo_a", "wo_b"):
            w0 = _bf16(wts[name], device)
            self.wts[name] = [w0] + [w0.clone() for _ in range(self.wcopies - 1)]
        self.x = _bf16(synth.hidden_states(self.cfg.cid, B, dims.d_model), device)
        self.q = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=device)   # made by the query path
        self.out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=device)  # attention output
        self.y = torch.empty((B, dims.d_model), dtype=torch.float32, device=device)
        self.ws_q = torch.empty(csa.csa_q_proj_workspace_size(B, dims.d_model, dims.q_rank, H, D), dtype=torch.uint8,
                                device=device)
        self.ws_o = torch.empty(csa.csa_out_proj_workspace_size(B, H, D, dims.groups, dims.o_rank, dims.d_model),
                                dtype=torch.uint8,
                                device=device)
        self.pos_flat = self.pos.view(B)
        torch.cuda.synchronize()

    def launches(self, c):
        import compressed_sparse_attention_06_amd as csa
        cfg, w = self.cfg, self.wts
        cw = c % self.wcopies
        L = [("q_proj", lambda: csa.csa_q_proj(self.x, w["wq_a"][cw], self.gamma_q, w["wq_b"][cw], self.pos_flat,
                                               self.q.view(cfg.B, cfg.H, cfg.D), rope_dim=cfg.rope_dim,
                                               rope_base=cfg.rope_base, eps=cfg.eps, ws=self.ws_q))]
        L += super().launches(c)
        L.append(("out_proj", lambda: csa.csa_out_proj(self.out.view(cfg.B, cfg.H, cfg.D), w["wo_a"][cw],
                                                       w["wo_b"][cw], self.y, ws=self.ws_o)))
        return L

    def dominant(self):
        return "out_proj"

    def algorithmic(self):
        by, fl = super().algorithmic()
        cfg, d, B = self.cfg, self.dims, self.cfg.B
        HD = cfg.H * cfg.D
        by["sparse_attn"] -= B * HD * 2      # the attention output is bf16 here
        by["q_proj"] = 2 * (d.q_rank * d.d_model + HD * d.q_rank) + B * d.d_model * 2 + B * 4 + d.q_rank * 4 + B * HD * 2
        by["out_proj"] = 2 * (d.groups * d.o_rank * (HD // d.groups) + d.d_model * d.groups * d.o_rank) + \
            B * HD * 2 + B * d.d_model * 4
        fl["q_proj"] = 2 * B * (d.q_rank * d.d_model + HD * d.q_rank)
        fl["out_proj"] = 2 * B * (d.o_rank * HD + d.d_model * d.groups * d.o_rank)
        return by, fl

    def unit(self):
        return "per projection weight: 2 B read (8 tokens: 16 flop)"

    def describe(self):
        d = super().describe()
        d.update(d_model=self.dims.d_model, q_rank=self.dims.q_rank, out_groups=self.dims.groups,
                 out_rank=self.dims.o_rank, weight_copies=self.wcopies)
        return d


class PagedDecodeWorkload(DecodeWorkload):
    """The decode step with both compressed caches in shared page pools.

    The page allocator (csa_page_pool) starts from a shuffled free list and
    hands pages out a round at a time to every sequence that still needs one,
    as concurrent sequences growing together would get them; each sequence
    holds the pages its visible entries (and this step's append) need, so the
    pools hold the visible rows only instead of every sequence's full
    capacity.  The kernels are the paged entry points; the seeded rows are the
    contiguous workload's."""

    def __init__(self, cfg, device, copies=COPIES, batch=None):
        import torch
        import compressed_sparse_attention_06_amd as csa
        super().__init__(cfg, device, copies=copies, batch=batch)
        cfg, B, pr = self.cfg, self.cfg.B, self.cfg.page_rows
        self.page_rows = pr
        self.max_pages = (self.Ncap + pr - 1) // pr
        need = np.maximum(self.n_vis, self.pos_np // cfg.ratio + 1)   # entries this step may touch
        pages = (need + pr - 1) // pr
        self.pool_pages = int(pages.sum())
        self.alloc = csa.PagePool(self.pool_pages)
        free = self.alloc.alloc(self.pool_pages)
        self.alloc.release(np.random.default_rng(cfg.cid).permutation(free))
        tab = np.full((B, self.max_pages), -1, np.int32)
        for rnd in range(int(pages.max())):
            for b in range(B):
                if rnd < pages[b]:
                    self.alloc.reserve(tab[b], pr, int(min(need[b], (rnd + 1) * pr)))
        assert self.alloc.available() == 0
        self.table_np = tab
        self.table = torch.from_numpy(tab).to(device)

        def paginate(caches):
            out = []
            for cache in caches:
                W = cache.shape[2]
                pool = torch.zeros((self.pool_pages * pr, W), dtype=cache.dtype, device=device)
                for b in range(B):
                    n = int(pages[b])
                    dst = (torch.from_numpy(tab[b, :n]).to(device).long()[:, None] * pr +
                           torch.arange(pr, device=device)[None]).view(-1)
                    rows = min(n * pr, self.Ncap)
                    pool[dst[:rows]] = cache[b, :rows]
                out.append(pool)
            return out

        self.kv = paginate(self.kv)
        if cfg.csa:
            self.idx_cache = paginate(self.idx_cache)
            self.scores = torch.empty((B, 1, self.max_pages * pr), dtype=torch.float32, device=device)
            self.ws_topk = torch.empty(max(1, csa.csa_topk_workspace_size(B, self.max_pages * pr, cfg.k)),
                                       dtype=torch.uint8, device=device)
        torch.cuda.synchronize()

    def launches(self, c):
        import compressed_sparse_attention_06_amd as csa
        cfg, pr = self.cfg, self.page_rows
        c = c % self.copies
        scale = 1.0 / math.sqrt(cfg.D)
        N = self.max_pages * pr
        kv_job = dict(kv=self.kv_stage, gate=self.gate_stage, gamma=self.gamma, pool=self.kv[c], pages=self.table,
                      page_rows=pr, ratio=cfg.ratio, overlap=cfg.overlap, rope_dim=cfg.rope_dim,
                      rope_base=cfg.rope_base, eps=cfg.eps, pos=self.pos, ws=self.ws_ckv)
        if not cfg.csa:
            return [("compress", lambda: csa.csa_compress_paged(**kv_job)),
                    ("hca_attn", lambda: csa.hca_attn_paged(
                        self.q, self.kv[c], self.table, self.win, self.pos2, self.sink, self.out, page_rows=pr,
                        ratio=cfg.ratio, window=cfg.window, scale=scale, rope_dim=cfg.rope_dim,
                        rope_base=cfg.rope_base, ws=self.ws_attn))]
        idx_job = dict(kv=self.ki_stage, gate=self.gi_stage, gamma=self.gamma_idx, pool=self.idx_cache[c],
                       pages=self.table, page_rows=pr, ratio=cfg.ratio, overlap=cfg.overlap,
                       rope_dim=cfg.rope_dim_idx, rope_base=cfg.rope_base, eps=cfg.eps, pos=self.pos, ws=self.ws_cidx)
        return [
            ("compress", lambda: csa.csa_compress_paged_jobs([kv_job, idx_job])),
            ("index_score", lambda: csa.csa_index_score_paged(self.q_idx, self.w, self.idx_cache[c], self.pos2,
                                                              self.scores, self.table, page_rows=pr,
                                                              ratio=cfg.ratio)),
            ("topk", lambda: csa.csa_topk(self.scores.view(cfg.B, N), None, cfg.k, self.sel.view(cfg.B, cfg.k),
                                          ws=self.ws_topk)),
            ("sparse_attn", lambda: csa.csa_sparse_attn_paged(
                self.q, self.kv[c], self.table, self.sel, self.win, self.pos2, self.sink, self.out, page_rows=pr,
                window=cfg.window, scale=scale, rope_dim=cfg.rope_dim, rope_base=cfg.rope_base, ws=self.ws_attn)),
        ]

    def algorithmic(self):
        """The contiguous step's bytes plus the page-table entries read: one
        per page of visible index rows, one per selected or attended row."""
        by, fl = super().algorithmic()
        cfg = self.cfg
        N = self.max_pages * self.page_rows
        vis = self.n_vis
        if cfg.csa:
            by["index_score"] += int(np.sum((vis + self.page_rows - 1) // self.page_rows) * 4)
            by["index_score"] += int(cfg.B * (N - self.Ncap) * 4)
            by["topk"] += int(cfg.B * (N - self.Ncap) * 4)
            by["sparse_attn"] += int(np.sum(np.minimum(vis, cfg.k)) * 4)
        else:
            by["hca_attn"] += int(np.sum((vis + self.page_rows - 1) // self.page_rows) * 4)
        return by, fl

    def describe(self):
        d = super().describe()
        d.update(page_rows=self.page_rows, pool_pages=self.pool_pages,
                 pool_gib=round(self.pool_pages * self.page_rows * (self.kv_row_bytes +
                                                                    (self.cfg.D_I * 2 if self.cfg.csa else 0)) /
                                2 ** 30, 2),
                 contiguous_gib=round(self.cfg.B * self.Ncap * (self.kv_row_bytes +
                                                                (self.cfg.D_I * 2 if self.cfg.csa else 0)) / 2 ** 30,
                                      2))
        return d


class PrefillWorkload:
    """CSA prefill of S tokens: compress all groups, score, top-k, attention."""

    def __init__(self, cfg, device, copies=2):
        import torch
        import compressed_sparse_attention_06_amd as csa
        self.cfg, self.device = cfg, device
        S, D, DI = cfg.S, cfg.D, cfg.D_I
        inp = synth.prefill_inputs(cfg)
        self.copies = copies
        self.Nc = S // cfg.ratio
        self.kv = _bf16(inp["kv"][None], device)
        self.gate = _bf16(inp["gate"][None], device)
        self.ki = _bf16(inp["k_idx"][None], device)
        self.gi = _bf16(inp["g_idx"][None], device)
        self.win = _bf16(inp["win"][None], device)
        q = _bf16(inp["q"][None], device)
        qi = _bf16(inp["q_idx"][None], device)
        self.q = [q] + [q.clone() for _ in range(copies - 1)]
        self.q_idx = [qi] + [qi.clone() for _ in range(copies - 1)]
        self.w = _f32(inp["w"][None], device)
        shared = synth.decode_shared(cfg)
        self.sink = _f32(shared["sink"], device)
        self.gamma = _f32(shared["gamma"], device)
        self.gamma_idx = _f32(shared["gamma_idx"], device)
        self.pos = torch.arange(S, dtype=torch.int32, device=device)[None]
        self.kv_cache = torch.empty((1, self.Nc, D), dtype=torch.bfloat16, device=device)
        self.idx_cache = torch.empty((1, self.Nc, DI), dtype=torch.bfloat16, device=device)
        self.scores = torch.empty((1, S, self.Nc), dtype=torch.float32, device=device)
        self.sel = torch.empty((1, S, cfg.k), dtype=torch.int32, device=device)
        self.out = torch.empty((1, S, cfg.H, D), dtype=torch.bfloat16, device=device)
        self.ws_topk = torch.empty(max(1, csa.csa_topk_workspace_size(S, self.Nc, cfg.k)), dtype=torch.uint8,
                                   device=device)
        self.ws_attn = torch.empty(max(1, csa.csa_sparse_attn_workspace_size(1, S, cfg.H, D, cfg.k, cfg.window)),
                                   dtype=torch.uint8, device=device)
        self.ws_ckv = torch.zeros(max(16, csa.csa_compress_workspace_size(self.Nc, D, cfg.ratio, cfg.overlap)),
                                  dtype=torch.uint8, device=device)
        self.ws_cidx = torch.zeros(max(16, csa.csa_compress_workspace_size(self.Nc, DI, cfg.ratio, cfg.overlap)),
                                   dtype=torch.uint8, device=device)
        torch.cuda.synchronize()

    # the KV-role compressor feeds only the attention: it runs beside the index
    # chain (a prefill step is long enough for the fork and join to pay off)
    side_kernels = ("compress_kv",)
    join_before = "sparse_attn"

    def launches(self, c):
        import compressed_sparse_attention_06_amd as csa
        cfg, S = self.cfg, self.cfg.S
        c = c % self.copies
        return [
            ("compress_kv", lambda: csa.csa_compress(self.kv, self.gate, self.gamma, self.kv_cache, ratio=cfg.ratio,
                                                     overlap=cfg.overlap, rope_dim=cfg.rope_dim, eps=cfg.eps,
                                                     ws=self.ws_ckv)),
            ("compress_idx", lambda: csa.csa_compress(self.ki, self.gi, self.gamma_idx, self.idx_cache,
                                                      ratio=cfg.ratio, overlap=cfg.overlap,
                                                      rope_dim=cfg.rope_dim_idx, eps=cfg.eps, ws=self.ws_cidx)),
            ("index_score", lambda: csa.csa_index_score(self.q_idx[c], self.w, self.idx_cache, self.pos,
                                                        self.scores, ratio=cfg.ratio)),
            ("topk", lambda: csa.csa_topk(self.scores.view(S, self.Nc), None, cfg.k, self.sel.view(S, cfg.k),
                                          ws=self.ws_topk)),
            ("sparse_attn", lambda: csa.csa_sparse_attn(self.q[c], self.kv_cache, self.sel, self.win, self.pos,
                                                        self.sink, self.out, window=cfg.window,
                                                        scale=1.0 / math.sqrt(cfg.D), rope_dim=cfg.rope_dim,
                                                        ws=self.ws_attn)),
        ]

    def queries(self):
        return self.cfg.S

    def dominant(self):
        return "index_score"

    def algorithmic(self):
        cfg, S = self.cfg, self.cfg.S
        D, DI, H, HI, r = cfg.D, cfg.D_I, cfg.H, cfg.H_I, cfg.ratio
        t = np.arange(S)
        vis = (t + 1) // r
        win = np.minimum(cfg.window, t + 1)
        sel = np.minimum(vis, cfg.k)
        # compulsory HBM bytes: every input read once, every output written
        # once; the attention's gathers of selected rows (each query re-reads
        # up to 640 rows of a 2 MiB cache, ~4.8 GB in all) are served from L2
        # and the Infinity Cache and are reported apart (gathered_bytes)
        by = {"compress_kv": S * D * 2 * 2 + self.Nc * D * 2, "compress_idx": S * DI * 2 * 2 + self.Nc * DI * 2,
              "index_score": S * HI * DI * 2 + S * HI * 4 + self.Nc * DI * 2 + S * self.Nc * 4,
              "topk": S * self.Nc * 4 + S * cfg.k * 4,
              "sparse_attn": int(S * H * D * 2 * 2 + self.Nc * D * 2 + S * D * 2 + S * cfg.k * 4)}
        fl = {"index_score": int(np.sum(vis)) * HI * DI * 2, "sparse_attn": int(np.sum(sel + win)) * H * D * 4}
        self.gathered_bytes = int(np.sum(sel + win) * D * 2)
        return by, fl

    def unit(self):
        return "per visible (query, entry) pair: 64 heads x 128 dims = 16,384 flop"

    def describe(self):
        cfg = self.cfg
        return dict(workload=cfg.name, batch=1, tokens=cfg.S, compressed_entries=self.Nc, ratio=cfg.ratio,
                    heads=cfg.H, head_dim=cfg.D, index_heads=cfg.H_I, index_dim=cfg.D_I, top_k=cfg.k,
                    window=cfg.window, query_copies=self.copies)


def make_workload(name, device):
    cfg = synth.CONFIGS[name]
    if cfg.kind == "decode":
        return PagedDecodeWorkload(cfg, device) if cfg.page_rows else DecodeWorkload(cfg, device)
    if cfg.kind == "block":
        return BlockWorkload(cfg, device)
    if cfg.kind == "prefill":
        return PrefillWorkload(cfg, device)
    raise SystemExit(f"{name} is a parity-test configuration, not a bench workload")


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------
def _spin(ms):
    """Keep the GPU busy for about `ms` so that what follows is queued back to back."""
    import torch
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))


def run_step(wl, c, only=None, side=None):
    """Enqueue one step.  Kernels the workload marks independent (the KV-role
    compressor of a prefill step, needed only by the attention) go to the
    `side` stream and are joined back before the first kernel that reads them."""
    import torch
    launches = wl.launches(c)
    forked = [n for n in getattr(wl, "side_kernels", ()) if only is None]
    if side is None or not forked:
        for name, fn in launches:
            if only is None or name == only:
                fn()
        return
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        for name, fn in launches:
            if name in forked:
                fn()
    for name, fn in launches:
        if name in forked:
            continue
        if name == wl.join_before:
            main.wait_stream(side)
        fn()


def capture_graphs(wl, n, only=None):
    import torch
    graphs = []
    side = torch.cuda.Stream()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(n):
            run_step(wl, c, only, side)
        s.wait_stream(side)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for c in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(wl, c, only, side)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_steps(wl, steps, warmup, only=None):
    """Replay `steps` one-step graphs between events; returns per-step ms."""
    import torch
    graphs = capture_graphs(wl, min(wl.copies, max(steps, 1)), only)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    _spin(20)
    ev[0].record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    total = ev[0].elapsed_time(ev[steps])
    return per, total


def time_kernels(wl, steps):
    """Per-kernel durations (ms) from HIP events around each eager launch."""
    import torch
    names = [n for n, _ in wl.launches(0)]
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for n in names}
    for i in range(2):
        for _, fn in wl.launches(i):
            fn()
    torch.cuda.synchronize()
    _spin(60)
    for i in range(steps):
        for n, fn in wl.launches(i):
            a, b = ev[n][i]
            a.record()
            fn()
            b.record()
    torch.cuda.synchronize()
    return {n: np.array([a.elapsed_time(b) for a, b in ev[n]]) for n in names}


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------
def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline_decode(wl, seconds):
    import oracle
    from oracle import pipeline
    cfg = wl.cfg
    f64 = synth.bf16_to_f64
    shared = synth.decode_shared(cfg)
    prepared = []
    for s in wl.seqs:
        d = dict(seq=s)
        d["kv"] = f64(synth.kv_cache_rows(cfg, s.b, s.n_vis))
        if cfg.kv4:  # the rows the quantised cache stands for (oracle quantiser), one sequence
            from oracle import quant
            d["kv"] = np.stack([quant.dequantize_row(quant.quantize_row(r, cfg.rope_dim), cfg.D, cfg.rope_dim)
                                for r in d["kv"]])
        if cfg.csa:
            d["idx"] = f64(synth.idx_cache_rows(cfg, s.b, s.n_vis))
        prepared.append(d)
        if len(prepared) * s.n_vis > 2_000_000 or cfg.kv4:
            break

    def one(d):
        s = d["seq"]
        e = s.n_vis - 1
        scale = 1.0 / math.sqrt(cfg.D)
        emit = (s.pos + 1) % cfg.ratio == 0
        prev, cur = oracle.entry_candidates(e, cfg.ratio, cfg.overlap)
        toks = prev + cur                     # staging ring slot = token % R
        if emit:
            rows = lambda st: f64(st[[t % wl.R for t in toks]])
            d["kv"][e] = oracle.entry_from_rows(e, cfg.ratio, rows(s.gate_stage), rows(s.kv_stage), shared["gamma"],
                                                cfg.rope_dim, cfg.rope_base, cfg.eps)
            if cfg.kv4:
                from oracle import quant
                d["kv"][e] = quant.dequantize_row(quant.quantize_row(d["kv"][e], cfg.rope_dim), cfg.D, cfg.rope_dim)
        win = np.stack([f64(s.win[p % cfg.window]) for p in oracle.window_positions(s.pos, cfg.window)])
        q = d["q_override"] if "q_override" in d else f64(s.q)
        if cfg.csa:
            if emit:
                d["idx"][e] = oracle.entry_from_rows(e, cfg.ratio, rows(s.gi_stage), rows(s.ki_stage),
                                                     shared["gamma_idx"], cfg.rope_dim_idx, cfg.rope_base, cfg.eps)
            return pipeline.csa_query(q, f64(s.q_idx), s.w, d["kv"], d["idx"], s.n_vis, win, shared["sink"],
                                      cfg.k, scale, s.pos, cfg.rope_dim, cfg.rope_base)[2]
        return oracle.hca_attn(q, d["kv"], s.n_vis, win, shared["sink"], scale, s.pos, cfg.rope_dim, cfg.rope_base)

    block = isinstance(wl, BlockWorkload)
    if block:
        from oracle import projection
        wts = synth.proj_weights(cfg.cid, cfg.H, cfg.D, wl.dims)
        wf = {k: (f64(v) if v.dtype == np.uint16 else v) for k, v in wts.items()}
        xs = f64(synth.hidden_states(cfg.cid, cfg.B, wl.dims.d_model))
        inner = one

        def one(d):  # noqa: F811 -- the block: query path, the CSA step, output projection
            s = d["seq"]
            q = projection.q_path(xs[s.b], wf["wq_a"], wf["gamma_q"], wf["wq_b"], cfg.H, cfg.D, s.pos,
                                  cfg.rope_dim, cfg.rope_base, cfg.eps)
            d["q_override"] = q
            o = inner(d)
            projection.out_proj(o, wf["wo_a"], wf["wo_b"], wl.dims.groups)

    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        one(prepared[n % len(prepared)])
        n += 1
    dt = time.perf_counter() - t0
    what = ("query path, compress the completed group, score, top-k, attend, output projection" if block else
            "compress the completed group, score, top-k, attend")
    return dict(value=n / dt, unit="query-tokens/s", cores=cpu_threads(), kind="oracle",
                sample=f"{n} decode queries of {cfg.name} (sequences 0..{len(prepared) - 1} in turn, float64 "
                       f"NumPy oracle: {what}), {dt:.1f} s")


def cpu_baseline_prefill(wl, seconds):
    import oracle
    from oracle import pipeline
    cfg = wl.cfg
    f64 = synth.bf16_to_f64
    shared = synth.decode_shared(cfg)
    inp = synth.prefill_inputs(cfg, q_rows=np.arange(cfg.S - 256, cfg.S))
    t0 = time.perf_counter()
    kvc = oracle.compress(f64(inp["kv"]), f64(inp["gate"]), shared["gamma"], cfg.ratio, cfg.overlap, cfg.rope_dim)
    idc = oracle.compress(f64(inp["k_idx"]), f64(inp["g_idx"]), shared["gamma_idx"], cfg.ratio, cfg.overlap,
                          cfg.rope_dim_idx)
    win = f64(inp["win"])
    n = 0
    qs = np.arange(cfg.S - 256, cfg.S)
    while time.perf_counter() - t0 < seconds and n < qs.size:
        t = int(qs[n])
        pipeline.csa_query(f64(inp["q"][n]), f64(inp["q_idx"][n]), inp["w"][n], kvc, idc, oracle.visible(t, 4),
                           pipeline.window_rows(win, t, cfg.window), shared["sink"], cfg.k, 1 / math.sqrt(cfg.D),
                           t, cfg.rope_dim)
        n += 1
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="query-tokens/s", cores=cpu_threads(), kind="oracle",
                sample=f"compress all {cfg.S} tokens (both roles) + {n} of the last 256 queries of {cfg.name} "
                       f"(score 2048 entries, top-k, attend), float64 NumPy oracle, {dt:.1f} s")


def cpu_baseline(wl, seconds):
    if isinstance(wl, PrefillWorkload):
        return cpu_baseline_prefill(wl, seconds)
    return cpu_baseline_decode(wl, seconds)


# ---------------------------------------------------------------------------
def time_dominant(wl, dom, launches=16, reps=5):
    """Average duration (ms) of one launch of the dominant kernel: `launches`
    back-to-back launches of it alone (the workload's own launch closures,
    rotating over its input copies) captured in one graph, replayed `reps`
    times between HIP events on the stream the graph runs on; the best
    replay counts.  Unlike an event pair around one eager launch, this
    leaves out the event and dispatch overhead around each launch (about
    2 us), which is not the kernel's time."""
    import torch
    fns = [fn for c in range(launches) for n, fn in wl.launches(c) if n == dom]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for fn in fns:  # warm
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    best = None
    with torch.cuda.stream(s):
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            _spin(2)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            t = a.elapsed_time(b) / len(fns)
            best = t if best is None else min(best, t)
    torch.cuda.synchronize()
    return best


def measure(wl, steps, warmup, only=None):
    per, total = time_steps(wl, steps, warmup, only)
    ms = total / steps
    kern = time_kernels(wl, steps)
    by, fl = wl.algorithmic()
    dom = wl.dominant()
    dom_ms = time_dominant(wl, dom)
    res = dict(ms_per_step=ms, per=per, kern={n: float(np.mean(v)) * 1e3 for n, v in kern.items()},
               step_bytes=int(sum(by.values())), by=by, fl=fl, dom=dom, dom_ms=dom_ms,
               dom_eager_ms=float(np.mean(kern[dom])))
    return res


KERNEL_SOURCE = {"q_proj": "proj.hip", "out_proj": "proj.hip",
                 "index_score": "index_score.hip", "topk": "topk.hip", "sparse_attn": "attn.hip",
                 "hca_attn": "attn.hip", "compress": "compress.hip", "compress_kv": "compress.hip",
                 "compress_idx": "compress.hip"}


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of this workload (profiles/*_<workload>.md: FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy), or None when there is none or the
    kernel source has changed since the counters were taken."""
    v = _profile_field(workload, kernel, "traffic_bytes_per_launch")
    return None if v is None else int(v)


def _source_hash(kernel):
    import hashlib
    csrc = os.path.join(ROOT, "compressed_sparse_attention_06_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[kernel], "common.h", "kernels.h", "rope_math.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _profile_field(workload, kernel, key):
    """A numeric field of the committed profile summary of `workload` whose
    traffic_kernel is `kernel`, if its source hash matches the current source."""
    import glob
    want = _source_hash(kernel)
    for path in glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}.md")):
        fields = {}
        with open(path) as fh:
            for line in fh:
                if ":" in line and line.split(":", 1)[0] in ("traffic_kernel", key, "source_sha256"):
                    k, v = line.split(":", 1)
                    fields[k] = v.strip()
        if fields.get("traffic_kernel") == kernel and fields.get("source_sha256") == want and key in fields:
            return float(fields[key])
    return None


def roofline(wl, m):
    dom, t = m["dom"], m["dom_ms"] * 1e-3
    timing = dict(kernel_us=round(m["dom_ms"] * 1e3, 2), kernel_us_eager=round(m["dom_eager_ms"] * 1e3, 2))
    if isinstance(wl, PrefillWorkload):
        ach = m["fl"][dom] / t / 1e12
        return dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4), traffic=measured_traffic(wl.cfg.name, dom), kernel=dom,
                    **timing, algorithmic_flops=m["fl"][dom], per_unit=wl.unit())
    ach = m["by"][dom] / t / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4),
                traffic=measured_traffic(wl.cfg.name, dom), kernel=dom, **timing, algorithmic_bytes=m["by"][dom],
                per_unit=wl.unit())


def measured_mfma_util(workload, kernel):
    """Matrix-core busy fraction of `kernel` from the committed rocprofv3
    counter summary (SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles), or None when
    there is none or the kernel source changed since it was taken."""
    return _profile_field(workload, kernel, "mfma_busy_frac")


def summary(wl, m):
    q = wl.queries()
    per = m["per"] * 1e3
    extra = {}
    if isinstance(wl, PrefillWorkload):
        t_attn = m["kern"]["sparse_attn"] * 1e-6
        extra = dict(indexer_mfma_util=round(m["fl"]["index_score"] / (m["dom_ms"] * 1e-3) / 1e12 /
                                             MFMA_BF16_PEAK_TFLOPS, 4),
                     indexer_mfma_busy_counters=measured_mfma_util(wl.cfg.name, "index_score"),
                     attn_gathered_rows_gbs=round(wl.gathered_bytes / t_attn / 1e9, 1))
    return dict(**extra,query_tokens_per_s=round(q / (m["ms_per_step"] * 1e-3), 1), ms_per_step=round(m["ms_per_step"], 5),
                step_us_p50=round(float(np.percentile(per, 50)), 2), step_us_p95=round(float(np.percentile(per, 95)), 2),
                step_us_p99=round(float(np.percentile(per, 99)), 2),
                hbm_gbs_step=round(m["step_bytes"] / (m["ms_per_step"] * 1e-3) / 1e9, 1),
                kernels_us={n: round(v, 2) for n, v in m["kern"].items()}, roofline=roofline(wl, m),
                config=wl.describe())


def note(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path runs on a single MI355X; --gpus above 1 is not supported",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    import compressed_sparse_attention_06_amd as csa
    csa.lib()
    dev = torch.device("cuda:0")
    t_setup = time.time()
    wl = make_workload(args.workload, dev)
    setup_s = time.time() - t_setup
    note(f"{args.workload}: inputs resident in HBM after {setup_s:.1f} s")
    only = args.kernel_only or None
    m = measure(wl, args.steps, args.warmup, only)
    note(f"{args.workload}: {m['ms_per_step'] * 1e3:.2f} us/step")
    main_sum = summary(wl, m)
    line = dict(metric=METRIC, value=main_sum["query_tokens_per_s"], unit="query-tokens/s", n_gpus=1,
                steps=args.steps, warmup=args.warmup, ms_per_step=main_sum["ms_per_step"], higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic", config=main_sum["config"],
                roofline=main_sum["roofline"])
    for key in ("hbm_gbs_step", "step_us_p50", "step_us_p95", "step_us_p99", "kernels_us"):
        line[key] = main_sum[key]
    line["setup_s"] = round(setup_s, 1)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        note(f"cpu baseline: {line['cpu_baseline']['value']:.2f} {line['cpu_baseline']['unit']}")
    del wl
    torch.cuda.empty_cache()
    extras = {}
    for name in [x for x in args.extra.split(",") if x and x != args.workload]:
        w2 = make_workload(name, dev)
        note(f"{name}: inputs resident")
        m2 = measure(w2, args.steps, args.warmup)
        note(f"{name}: {m2['ms_per_step'] * 1e3:.2f} us/step")
        extras[name] = summary(w2, m2)
        # (a paged workload computes what its contiguous twin does: the
        # oracle's sample is the same kind of work, timed again here)
        if not args.no_cpu_baseline:
            extras[name]["cpu_baseline"] = cpu_baseline(w2, args.cpu_seconds / 2)
            note(f"{name} cpu baseline: {extras[name]['cpu_baseline']['value']:.2f} query-tokens/s")
        del w2
        torch.cuda.empty_cache()
    if extras:
        line["secondary"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
