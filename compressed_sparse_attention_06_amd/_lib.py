"""ctypes binding of libcsa.so: argument marshalling only.

Every function takes torch tensors that live in device memory, passes their
data pointers, sizes and torch's current HIP stream to the C entry point of
the same name, and raises ``CsaError`` on a non-zero status.  All arithmetic
happens in the HIP kernels; there is no fallback path.  When the library has
not been built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

CSA_F32, CSA_BF16, CSA_KV4 = 0, 1, 2
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape or dtype", -3: "HIP runtime error",
          -4: "workspace too small", -5: "out of pages"}

_c_int, _c_i64, _c_f, _c_sz, _c_p = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class CompressJob(ctypes.Structure):
    """csa_compress_job of include/csa.h: the arguments of one csa_compress call."""
    _fields_ = [("kv", _c_p), ("gate", _c_p), ("kv_prev", _c_p), ("gate_prev", _c_p), ("in_dtype", _c_int),
                ("gamma", _c_p), ("B", _c_int), ("T", _c_int), ("in_bstride", _c_i64), ("D", _c_int),
                ("ratio", _c_int), ("overlap", _c_int), ("rope_dim", _c_int), ("rope_base", _c_f), ("eps", _c_f),
                ("tok0", _c_int), ("e0", _c_int), ("n_entries", _c_int), ("pos", _c_p), ("out", _c_p),
                ("out_dtype", _c_int), ("out_bstride", _c_i64), ("out_cap", _c_int), ("ws", _c_p),
                ("ws_bytes", _c_sz)]


CSA_MAX_COMPRESS_JOBS = 16


class PageTableC(ctypes.Structure):
    """csa_page_table of include/csa.h."""
    _fields_ = [("pages", _c_p), ("max_pages", _c_int), ("page_rows", _c_int), ("pool_pages", _c_int)]


# name -> (restype, argtypes); mirrors include/csa.h
SIGNATURES = {
    "csa_status_string": (ctypes.c_char_p, [_c_int]),
    "csa_version": (_c_int, []),
    "csa_kv4_row_bytes": (_c_sz, [_c_int, _c_int]),
    "csa_kv4_quantize": (_c_int, [_c_p, _c_int, _c_i64, _c_int, _c_int, _c_p, _c_p]),
    "csa_compress_workspace_size": (_c_sz, [_c_i64, _c_int, _c_int, _c_int]),
    "csa_compress": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_int, _c_p, _c_int, _c_int, _c_i64, _c_int, _c_int, _c_int,
                              _c_int, _c_f, _c_f, _c_int, _c_int, _c_int, _c_p, _c_p, _c_int, _c_i64, _c_int, _c_p,
                              _c_sz, _c_p]),
    "csa_compress_jobs": (_c_int, [ctypes.POINTER(CompressJob), _c_int, _c_p]),
    "csa_compress_paged": (_c_int, [ctypes.POINTER(CompressJob), ctypes.POINTER(PageTableC), _c_int, _c_p]),
    "csa_index_score_paged": (_c_int, [_c_p, _c_p, _c_p, _c_int, _c_p, _c_int, _c_int, _c_int, _c_int,
                                       ctypes.POINTER(PageTableC), _c_int, _c_p, _c_p]),
    "csa_sparse_attn_paged": (_c_int, [_c_p, _c_p, ctypes.POINTER(PageTableC), _c_p, _c_int, _c_p, _c_int, _c_int,
                                       _c_p, _c_p, _c_int, _c_f, _c_int, _c_f, _c_int, _c_int, _c_int, _c_int, _c_p,
                                       _c_int, _c_p, _c_sz, _c_p]),
    "hca_attn_paged": (_c_int, [_c_p, _c_p, ctypes.POINTER(PageTableC), _c_int, _c_p, _c_int, _c_int, _c_p, _c_p,
                                _c_int, _c_f, _c_int, _c_f, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p, _c_sz,
                                _c_p]),
    "csa_page_pool_create": (_c_p, [_c_int]),
    "csa_page_pool_destroy": (None, [_c_p]),
    "csa_page_pool_available": (_c_int, [_c_p]),
    "csa_page_pool_alloc": (_c_int, [_c_p, _c_int, _c_p]),
    "csa_page_pool_release": (_c_int, [_c_p, _c_int, _c_p]),
    "csa_page_table_reserve": (_c_int, [_c_p, _c_p, _c_int, _c_int, _c_i64]),
    "csa_page_table_release": (_c_int, [_c_p, _c_p, _c_int]),
    "csa_index_score": (_c_int, [_c_p, _c_p, _c_p, _c_int, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_p, _c_p]),
    "csa_topk_workspace_size": (_c_sz, [_c_int, _c_int, _c_int]),
    "csa_topk": (_c_int, [_c_p, _c_p, _c_int, _c_int, _c_int, _c_p, _c_p, _c_sz, _c_p]),
    "csa_topk_noalloc": (_c_int, [_c_p, _c_p, _c_int, _c_int, _c_int, _c_p, _c_p]),
    "csa_sparse_attn_workspace_size": (_c_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "csa_sparse_attn": (_c_int, [_c_p, _c_p, _c_int, _c_p, _c_int, _c_p, _c_int, _c_int, _c_p, _c_p, _c_int, _c_f,
                                 _c_int, _c_f, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p, _c_sz, _c_p]),
    "csa_q_proj_workspace_size": (_c_sz, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "csa_q_proj": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_f, _c_f,
                            _c_p, _c_p, _c_sz, _c_p]),
    "csa_out_proj_workspace_size": (_c_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "csa_out_proj": (_c_int, [_c_p, _c_int, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int,
                              _c_p, _c_sz, _c_p]),
    "hca_attn_workspace_size": (_c_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "hca_attn": (_c_int, [_c_p, _c_p, _c_int, _c_int, _c_p, _c_int, _c_int, _c_p, _c_p, _c_int, _c_f, _c_int, _c_f,
                          _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p, _c_sz, _c_p]),
}

_lib = None


class CsaError(RuntimeError):
    pass


def lib():
    """The loaded libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CsaError(f"{LIB_PATH} is missing: build it with `python -m compressed_sparse_attention_06_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def _check(status, what):
    if status != 0:
        raise CsaError(f"{what}: {STATUS.get(status, status)} ({status})")


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.uint8:      # a quantised cache: rows of csa_kv4_row_bytes bytes
        return CSA_KV4
    raise CsaError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ws(size, ws, device):
    if size == 0:
        return ws
    if ws is None or ws.numel() * ws.element_size() < size:
        ws = torch.empty(size, dtype=torch.uint8, device=device)
    return ws


def _bytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _dense(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise CsaError("tensors passed to the C ABI must be contiguous")


def _rows(t):
    """Batch stride (elements) of a [B, rows, D] tensor whose rows are packed."""
    if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        raise CsaError("rows of a [B, rows, D] tensor must be contiguous and packed")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1] * t.shape[2]


# ---------------------------------------------------------------------------
def csa_kv4_row_bytes(D, rope_dim):
    return int(lib().csa_kv4_row_bytes(D, rope_dim))


def csa_kv4_quantize(x, out, *, rope_dim, stream=None):
    """x [..., D] (f32 or bf16) -> out [..., csa_kv4_row_bytes(D, rope_dim)] uint8 (quantised cache rows)."""
    D = x.shape[-1]
    rows = x.numel() // D
    _dense(x, out)
    if out.dtype != torch.uint8 or out.numel() != rows * csa_kv4_row_bytes(D, rope_dim):
        raise CsaError("out must be a uint8 tensor of rows x csa_kv4_row_bytes(D, rope_dim) bytes")
    st = lib().csa_kv4_quantize(_ptr(x), _dtype(x), rows, D, rope_dim, _ptr(out), _stream(stream))
    _check(st, "csa_kv4_quantize")
    return out


def csa_compress_workspace_size(entries, D, ratio, overlap):
    return int(lib().csa_compress_workspace_size(entries, D, ratio, overlap))


def _compress_job(kv, gate, gamma, out, *, ratio, overlap, rope_dim, rope_base=10000.0, eps=1e-6,
                  kv_prev=None, gate_prev=None, tok0=0, e0=0, n_entries=None, pos=None, ws=None):
    """(CompressJob, tensors it points to) for one compressor call."""
    B, T, D = kv.shape
    n = (out.shape[1] - e0) if n_entries is None else n_entries
    bstride = _rows(kv)
    for t in (gate, kv_prev, gate_prev):
        if t is not None and (t.shape != kv.shape or _rows(t) != bstride):
            raise CsaError("kv, gate, kv_prev and gate_prev must share one layout")
    _dense(gamma, pos)
    need = csa_compress_workspace_size(B if pos is not None else B * n, D, ratio, overlap)
    if need and (ws is None or _bytes(ws) < need):
        ws = torch.zeros(need, dtype=torch.uint8, device=kv.device)
    # (a uint8 out is a quantised cache: its batch stride is in bytes)
    job = CompressJob(_ptr(kv), _ptr(gate), _ptr(kv_prev), _ptr(gate_prev), _dtype(kv), _ptr(gamma), B, T, bstride,
                      D, ratio, overlap, rope_dim, rope_base, eps, tok0, e0, n, _ptr(pos), _ptr(out), _dtype(out),
                      _rows(out), out.shape[1], _ptr(ws), _bytes(ws))
    return job, (kv, gate, gamma, out, kv_prev, gate_prev, pos, ws)


def csa_compress(kv, gate, gamma, out, *, ratio, overlap, rope_dim, rope_base=10000.0, eps=1e-6,
                 kv_prev=None, gate_prev=None, tok0=0, e0=0, n_entries=None, pos=None, ws=None, stream=None):
    """kv, gate: [B, T, D] (rows contiguous); out: [B, out_cap, D]; pos: [B] int32 (ring mode) or None.

    ws: a zero-filled uint8 device tensor of at least csa_compress_workspace_size bytes (kept by the
    caller across calls, each of which leaves it ready for the next), or None to allocate one."""
    j, keep = _compress_job(kv, gate, gamma, out, ratio=ratio, overlap=overlap, rope_dim=rope_dim,
                            rope_base=rope_base, eps=eps, kv_prev=kv_prev, gate_prev=gate_prev, tok0=tok0, e0=e0,
                            n_entries=n_entries, pos=pos, ws=ws)
    st = lib().csa_compress(j.kv, j.gate, j.kv_prev, j.gate_prev, j.in_dtype, j.gamma, j.B, j.T, j.in_bstride, j.D,
                            j.ratio, j.overlap, j.rope_dim, j.rope_base, j.eps, j.tok0, j.e0, j.n_entries, j.pos,
                            j.out, j.out_dtype, j.out_bstride, j.out_cap, j.ws, j.ws_bytes, _stream(stream))
    _check(st, "csa_compress")
    return out


def csa_compress_jobs(jobs, stream=None):
    """Independent compressor calls in one launch: `jobs` is a list of dicts holding the keyword
    arguments of csa_compress (kv, gate, gamma, out, ratio, overlap, rope_dim, ...)."""
    built = [_compress_job(**j) for j in jobs]
    arr = (CompressJob * max(1, len(built)))(*[b[0] for b in built])
    st = lib().csa_compress_jobs(arr, len(built), _stream(stream))
    _check(st, "csa_compress_jobs")
    return [j["out"] for j in jobs]


def csa_index_score(q_idx, w, idx_cache, pos, scores, *, ratio, stream=None):
    """q_idx [B,S,H_I,D_I], w [B,S,H_I] f32, idx_cache [B,Ncap,D_I], pos [B,S] i32 -> scores [B,S,Ncap] f32."""
    B, S, H, D = q_idx.shape
    Ncap = idx_cache.shape[1]
    _dense(q_idx, w, idx_cache, pos, scores)
    st = lib().csa_index_score(_ptr(q_idx), _ptr(w), _ptr(idx_cache), _dtype(q_idx), _ptr(pos), B, S, H, D, Ncap,
                               ratio, _ptr(scores), _stream(stream))
    _check(st, "csa_index_score")
    return scores


def csa_topk_workspace_size(R, N, k):
    return int(lib().csa_topk_workspace_size(R, N, k))


def csa_topk(scores, n_valid, k, idx, *, ws=None, stream=None):
    """scores [R,N] f32, n_valid [R] i32 or None -> idx [R,k] i32 (ascending, -1 padded)."""
    R, N = scores.shape
    _dense(scores, n_valid, idx)
    ws = _ws(csa_topk_workspace_size(R, N, k), ws, scores.device)
    st = lib().csa_topk(_ptr(scores), _ptr(n_valid), R, N, k, _ptr(idx), _ptr(ws), _bytes(ws), _stream(stream))
    _check(st, "csa_topk")
    return idx


CSA_TOPK_NOALLOC_SCRATCH_BYTES = 16 << 20


def csa_topk_noalloc(scores, n_valid, k, idx, *, stream=None):
    """csa_topk with the library's static scratch instead of a workspace (allocates nothing)."""
    R, N = scores.shape
    _dense(scores, n_valid, idx)
    st = lib().csa_topk_noalloc(_ptr(scores), _ptr(n_valid), R, N, k, _ptr(idx), _stream(stream))
    _check(st, "csa_topk_noalloc")
    return idx


def _attn_dtype(q, cmp):
    """The attention's dtype code: CSA_KV4 when cmp holds quantised rows (uint8; q then bf16)."""
    if cmp.dtype == torch.uint8:
        if q.dtype != torch.bfloat16:
            raise CsaError("a quantised cache needs bf16 queries and window rows")
        return CSA_KV4
    return _dtype(q)


def csa_sparse_attn_workspace_size(B, S, H, D, k, window):
    return int(lib().csa_sparse_attn_workspace_size(B, S, H, D, k, window))


def csa_sparse_attn(q, cmp, idx, win, pos, sink, out, *, window, scale, rope_dim, rope_base=10000.0,
                    ws=None, stream=None):
    """q [B,S,H,D], cmp [B,Ncap,D], idx [B,S,k] i32, win [B,Wcap,D], pos [B,S] i32, sink [H] f32 -> out."""
    B, S, H, D = q.shape
    k = idx.shape[-1]
    _dense(q, cmp, idx, win, pos, sink, out)
    ws = _ws(csa_sparse_attn_workspace_size(B, S, H, D, k, window), ws, q.device)
    st = lib().csa_sparse_attn(_ptr(q), _ptr(cmp), cmp.shape[1], _ptr(idx), k, _ptr(win), win.shape[1], window,
                               _ptr(pos), _ptr(sink), _attn_dtype(q, cmp), scale, rope_dim, rope_base, B, S, H, D, _ptr(out),
                               _dtype(out), _ptr(ws), _bytes(ws), _stream(stream))
    _check(st, "csa_sparse_attn")
    return out


def hca_attn_workspace_size(B, S, H, D, Ncap, window):
    return int(lib().hca_attn_workspace_size(B, S, H, D, Ncap, window))


def hca_attn(q, cmp, win, pos, sink, out, *, ratio, window, scale, rope_dim, rope_base=10000.0,
             ws=None, stream=None):
    """q [B,S,H,D], cmp [B,Ncap,D], win [B,Wcap,D], pos [B,S] i32, sink [H] f32 -> out [B,S,H,D]."""
    B, S, H, D = q.shape
    Ncap = cmp.shape[1]
    _dense(q, cmp, win, pos, sink, out)
    ws = _ws(hca_attn_workspace_size(B, S, H, D, Ncap, window), ws, q.device)
    st = lib().hca_attn(_ptr(q), _ptr(cmp), Ncap, ratio, _ptr(win), win.shape[1], window, _ptr(pos), _ptr(sink),
                        _attn_dtype(q, cmp), scale, rope_dim, rope_base, B, S, H, D, _ptr(out), _dtype(out), _ptr(ws),
                        _bytes(ws), _stream(stream))
    _check(st, "hca_attn")
    return out


def csa_q_proj_workspace_size(M, d_model, q_rank, H, head_dim):
    return int(lib().csa_q_proj_workspace_size(M, d_model, q_rank, H, head_dim))


def csa_q_proj(x, wq_a, gamma_q, wq_b, pos, q, *, rope_dim, rope_base=10000.0, eps=1e-6, ws=None, stream=None):
    """x [M, d_model] bf16, wq_a [q_rank, d_model], gamma_q [q_rank] f32, wq_b [H*head_dim, q_rank], pos [M] i32
    -> q [M, H, head_dim] bf16 (token rows may carry leading batch axes: x [..., d], q [..., H, head_dim])."""
    d = x.shape[-1]
    M = x.numel() // d
    H, hd = q.shape[-2], q.shape[-1]
    r = wq_a.shape[0]
    _dense(x, wq_a, gamma_q, wq_b, pos, q)
    ws = _ws(csa_q_proj_workspace_size(M, d, r, H, hd), ws, x.device)
    st = lib().csa_q_proj(_ptr(x), _ptr(wq_a), _ptr(gamma_q), _ptr(wq_b), _ptr(pos), M, d, r, H, hd, rope_dim,
                          rope_base, eps, _ptr(q), _ptr(ws), _bytes(ws), _stream(stream))
    _check(st, "csa_q_proj")
    return q


def csa_out_proj_workspace_size(M, H, head_dim, groups, o_rank, d_model, o_dtype=CSA_BF16):
    return int(lib().csa_out_proj_workspace_size(M, H, head_dim, groups, o_rank, d_model, o_dtype))


def csa_out_proj(o, wo_a, wo_b, y, *, ws=None, stream=None):
    """o [..., H, head_dim] (bf16 or f32), wo_a [groups, o_rank, H*head_dim/groups], wo_b [d_model, groups*o_rank]
    -> y [..., d_model]."""
    H, hd = o.shape[-2], o.shape[-1]
    M = o.numel() // (H * hd)
    groups, o_rank = wo_a.shape[0], wo_a.shape[1]
    d = wo_b.shape[0]
    _dense(o, wo_a, wo_b, y)
    ws = _ws(csa_out_proj_workspace_size(M, H, hd, groups, o_rank, d, _dtype(o)), ws, o.device)
    st = lib().csa_out_proj(_ptr(o), _dtype(o), _ptr(wo_a), _ptr(wo_b), M, H, hd, groups, o_rank, d, _ptr(y),
                            _dtype(y), _ptr(ws), _bytes(ws), _stream(stream))
    _check(st, "csa_out_proj")
    return y


# ---------------------------------------------------------------------------
# Paged caches and the page allocator
# ---------------------------------------------------------------------------
def _page_table(pages, page_rows, pool):
    """csa_page_table for a device int32 [B, max_pages] table over `pool` (rows of the cache)."""
    _dense(pages)
    if pages.dtype != torch.int32 or pages.dim() != 2:
        raise CsaError("pages must be an int32 [B, max_pages] device tensor")
    return PageTableC(_ptr(pages), pages.shape[1], page_rows, pool.shape[0] // page_rows)


def _paged_job(kv, gate, gamma, pool, pages, *, page_rows, ratio, overlap, rope_dim, rope_base=10000.0, eps=1e-6,
               kv_prev=None, gate_prev=None, tok0=0, e0=0, n_entries=None, pos=None, ws=None):
    """(CompressJob, csa_page_table, tensors they point to) for one paged compressor call."""
    B, T, D = kv.shape
    bstride = _rows(kv)
    for t in (gate, kv_prev, gate_prev):
        if t is not None and (t.shape != kv.shape or _rows(t) != bstride):
            raise CsaError("kv, gate, kv_prev and gate_prev must share one layout")
    _dense(gamma, pos, pool)
    if pos is None and n_entries is None:
        raise CsaError("span mode needs n_entries")
    n = 0 if n_entries is None else n_entries
    need = csa_compress_workspace_size(B if pos is not None else B * n, D, ratio, overlap)
    if need and (ws is None or _bytes(ws) < need):
        ws = torch.zeros(need, dtype=torch.uint8, device=kv.device)
    job = CompressJob(_ptr(kv), _ptr(gate), _ptr(kv_prev), _ptr(gate_prev), _dtype(kv), _ptr(gamma), B, T, bstride,
                      D, ratio, overlap, rope_dim, rope_base, eps, tok0, e0, n, _ptr(pos), _ptr(pool), _dtype(pool),
                      0, 0, _ptr(ws), _bytes(ws))
    return job, _page_table(pages, page_rows, pool), (kv, gate, gamma, pool, pages, kv_prev, gate_prev, pos, ws)


def csa_compress_paged(kv, gate, gamma, pool, pages, *, page_rows, ratio, overlap, rope_dim, rope_base=10000.0,
                       eps=1e-6, kv_prev=None, gate_prev=None, tok0=0, e0=0, n_entries=None, pos=None, ws=None,
                       stream=None):
    """csa_compress into a paged cache: pool [pool_rows, D] (or uint8 [pool_rows, row_bytes] quantised),
    pages [B, max_pages] int32.  Span mode needs n_entries."""
    csa_compress_paged_jobs([dict(kv=kv, gate=gate, gamma=gamma, pool=pool, pages=pages, page_rows=page_rows,
                                  ratio=ratio, overlap=overlap, rope_dim=rope_dim, rope_base=rope_base, eps=eps,
                                  kv_prev=kv_prev, gate_prev=gate_prev, tok0=tok0, e0=e0, n_entries=n_entries,
                                  pos=pos, ws=ws)], stream=stream)
    return pool


def csa_compress_paged_jobs(jobs, stream=None):
    """Paged compressor calls in one launch: `jobs` is a list of dicts holding the keyword arguments of
    csa_compress_paged (kv, gate, gamma, pool, pages, page_rows, ratio, ...)."""
    built = [_paged_job(**j) for j in jobs]
    n = max(1, len(built))
    arr = (CompressJob * n)(*[b[0] for b in built])
    tabs = (PageTableC * n)(*[b[1] for b in built])
    st = lib().csa_compress_paged(arr, tabs, len(built), _stream(stream))
    _check(st, "csa_compress_paged")
    return [j["pool"] for j in jobs]


def csa_index_score_paged(q_idx, w, idx_pool, pos, scores, pages, *, page_rows, ratio, stream=None):
    """scores [B,S,max_pages*page_rows] f32 from a paged index cache idx_pool [pool_rows, D_I]."""
    B, S, H, D = q_idx.shape
    _dense(q_idx, w, idx_pool, pos, scores)
    pt = _page_table(pages, page_rows, idx_pool)
    st = lib().csa_index_score_paged(_ptr(q_idx), _ptr(w), _ptr(idx_pool), _dtype(q_idx), _ptr(pos), B, S, H, D,
                                     ctypes.byref(pt), ratio, _ptr(scores), _stream(stream))
    _check(st, "csa_index_score_paged")
    return scores


def csa_sparse_attn_paged(q, cmp_pool, pages, idx, win, pos, sink, out, *, page_rows, window, scale, rope_dim,
                          rope_base=10000.0, ws=None, stream=None):
    B, S, H, D = q.shape
    k = idx.shape[-1]
    _dense(q, cmp_pool, idx, win, pos, sink, out)
    pt = _page_table(pages, page_rows, cmp_pool)
    ws = _ws(csa_sparse_attn_workspace_size(B, S, H, D, k, window), ws, q.device)
    st = lib().csa_sparse_attn_paged(_ptr(q), _ptr(cmp_pool), ctypes.byref(pt), _ptr(idx), k, _ptr(win),
                                     win.shape[1], window, _ptr(pos), _ptr(sink), _attn_dtype(q, cmp_pool), scale,
                                     rope_dim, rope_base, B, S, H, D, _ptr(out), _dtype(out), _ptr(ws), _bytes(ws),
                                     _stream(stream))
    _check(st, "csa_sparse_attn_paged")
    return out


def hca_attn_paged(q, cmp_pool, pages, win, pos, sink, out, *, page_rows, ratio, window, scale, rope_dim,
                   rope_base=10000.0, ws=None, stream=None):
    B, S, H, D = q.shape
    _dense(q, cmp_pool, win, pos, sink, out)
    pt = _page_table(pages, page_rows, cmp_pool)
    ws = _ws(hca_attn_workspace_size(B, S, H, D, pages.shape[1] * page_rows, window), ws, q.device)
    st = lib().hca_attn_paged(_ptr(q), _ptr(cmp_pool), ctypes.byref(pt), ratio, _ptr(win), win.shape[1], window,
                              _ptr(pos), _ptr(sink), _attn_dtype(q, cmp_pool), scale, rope_dim, rope_base, B, S, H, D,
                              _ptr(out), _dtype(out), _ptr(ws), _bytes(ws), _stream(stream))
    _check(st, "hca_attn_paged")
    return out


class PagePool:
    """The library's page allocator (csa_page_pool): which pages of a device pool are free.

    Tables are host int32 numpy rows (-1 = no page); upload them to the device for the kernels."""

    def __init__(self, n_pages):
        self._h = lib().csa_page_pool_create(n_pages)
        if not self._h:
            raise CsaError("csa_page_pool_create failed")
        self.n_pages = n_pages

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.csa_page_pool_destroy(h)

    def available(self):
        return int(lib().csa_page_pool_available(self._h))

    def alloc(self, n):
        import numpy as np
        out = np.empty(max(n, 1), dtype=np.int32)
        _check(lib().csa_page_pool_alloc(self._h, n, out.ctypes.data), "csa_page_pool_alloc")
        return out[:n]

    def release(self, pages):
        import numpy as np
        arr = np.ascontiguousarray(pages, dtype=np.int32)
        _check(lib().csa_page_pool_release(self._h, arr.size, arr.ctypes.data), "csa_page_pool_release")

    def reserve(self, row, page_rows, n_entries):
        """Make the host table row (int32 numpy, modified in place) cover n_entries entries."""
        _check(lib().csa_page_table_reserve(self._h, row.ctypes.data, row.size, page_rows, n_entries),
               "csa_page_table_reserve")
        return row

    def release_row(self, row):
        _check(lib().csa_page_table_release(self._h, row.ctypes.data, row.size), "csa_page_table_release")
        return row
