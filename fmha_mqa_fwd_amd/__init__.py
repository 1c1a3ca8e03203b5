"""MI355X-native multi-query attention forward.

``fwd`` and ``lse_merge`` call the C ABI of ``libfmha_mqa.so`` (hand-written
HIP kernels for gfx950; declarations in include/fmha_mqa.h).  Importing the
package raises ImportError when the library is not built.
"""
from ._binding import (FMHA_BF16, FMHA_ERR_SCRATCH_LIMIT, FMHA_F32, LIB_PATH, SCRATCH_BYTES,
                       SIGNATURES, FmhaError, FwdPlan, KvSource, SourcesPlan, apply_sink,
                       default_scale, fwd, fwd_noalloc, fwd_partials, fwd_sources,
                       fwd_sources_partials, gather_floor, index_scores,
                       indexer_topk, lse_merge, mfma_ceiling, raw_fwd, raw_merge, read_floor,
                       status_string, topk_select, workspace_bytes)

__all__ = ["fwd", "FwdPlan", "fwd_noalloc", "fwd_partials", "fwd_sources",
           "fwd_sources_partials", "SourcesPlan", "KvSource", "apply_sink",
           "index_scores", "topk_select", "indexer_topk", "lse_merge", "workspace_bytes",
           "default_scale", "status_string", "gather_floor", "read_floor", "mfma_ceiling",
           "FmhaError", "FMHA_F32", "FMHA_BF16",
           "FMHA_ERR_SCRATCH_LIMIT", "SCRATCH_BYTES", "LIB_PATH", "SIGNATURES", "raw_fwd",
           "raw_merge"]
