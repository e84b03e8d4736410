"""Float64 CPU oracle of the CSA / HCA compressed-KV attention path.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library and imports nothing from it.
"""
from . import csa, pipeline, projection, quant  # noqa: F401
from .csa import (NEG_INF, attend, compress, compress_entry, entry_candidates, entry_from_rows, hca_attn,  # noqa: F401
                  index_score, pool, rms_norm, rope, round_bf16, sparse_attn, topk, visible,
                  window_positions, StreamingCompressor)
