"""MI355X-native CSA / HCA compressed-KV attention path.

The hot path is hand-written HIP for gfx950 behind the C ABI in
``include/csa.h`` (``libcsa.so``); this package holds its sources, the build
step and a thin ctypes binding with the same function names.
"""
from ._lib import (CSA_BF16, CSA_F32, CSA_KV4, CsaError, csa_compress, csa_compress_jobs,  # noqa: F401
                   csa_kv4_row_bytes, csa_kv4_quantize, csa_compress_paged, csa_compress_paged_jobs, csa_index_score_paged,
                   csa_sparse_attn_paged, hca_attn_paged, PagePool,
                   csa_compress_workspace_size,
                   csa_index_score,
                   csa_sparse_attn, csa_sparse_attn_workspace_size, csa_topk, csa_topk_noalloc, csa_topk_workspace_size,
                   CSA_TOPK_NOALLOC_SCRATCH_BYTES,
                   csa_q_proj, csa_q_proj_workspace_size, csa_out_proj, csa_out_proj_workspace_size,
                   hca_attn, hca_attn_workspace_size, lib, LIB_PATH)

__all__ = ["csa_compress_paged", "csa_compress_paged_jobs", "csa_index_score_paged", "csa_sparse_attn_paged", "hca_attn_paged", "PagePool",
           "csa_kv4_row_bytes", "csa_kv4_quantize", "CSA_KV4", "csa_compress", "csa_compress_jobs", "csa_compress_workspace_size", "csa_index_score", "csa_topk", "csa_topk_noalloc", "csa_topk_workspace_size", "csa_sparse_attn",
           "csa_sparse_attn_workspace_size", "hca_attn", "hca_attn_workspace_size", "csa_q_proj",
           "csa_q_proj_workspace_size", "csa_out_proj", "csa_out_proj_workspace_size", "CsaError", "lib",
           "CSA_F32", "CSA_BF16", "CSA_TOPK_NOALLOC_SCRATCH_BYTES", "LIB_PATH"]
