"""MI355X-native CSA / HCA compressed-KV attention path.

The hot path is hand-written HIP for gfx950 behind the C ABI in
``include/csa.h`` (``libcsa.so``); this package holds its sources, the build
step and a thin ctypes binding with the same function names.
"""
from ._lib import (CSA_BF16, CSA_F32, CsaError, csa_compress, csa_compress_jobs,  # noqa: F401
                   csa_compress_workspace_size,
                   csa_index_score,
                   csa_sparse_attn, csa_sparse_attn_workspace_size, csa_topk, csa_topk_workspace_size,
                   hca_attn, hca_attn_workspace_size, lib, LIB_PATH)

__all__ = ["csa_compress", "csa_compress_jobs", "csa_compress_workspace_size", "csa_index_score", "csa_topk", "csa_topk_workspace_size", "csa_sparse_attn",
           "csa_sparse_attn_workspace_size", "hca_attn", "hca_attn_workspace_size", "CsaError", "lib",
           "CSA_F32", "CSA_BF16", "LIB_PATH"]
