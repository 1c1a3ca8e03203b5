"""MI355X-native multi-query attention forward.

``fwd`` and ``lse_merge`` call the C ABI of ``libfmha_mqa.so`` (hand-written
HIP kernels for gfx950; declarations in include/fmha_mqa.h).  Importing the
package raises ImportError when the library is not built.
"""
from ._binding import (FMHA_BF16, FMHA_F32, LIB_PATH, SIGNATURES, FmhaError, FwdPlan,
                       apply_sink, default_scale, fwd, fwd_partials, fwd_sources, gather_floor, index_scores,
                       indexer_topk, lse_merge, topk_select, raw_fwd, raw_merge,
                       status_string, workspace_bytes)

__all__ = ["fwd", "FwdPlan", "fwd_partials", "fwd_sources", "apply_sink", "index_scores", "topk_select",
           "indexer_topk", "lse_merge", "workspace_bytes", "default_scale", "status_string",
           "gather_floor", "FmhaError", "FMHA_F32", "FMHA_BF16", "LIB_PATH", "SIGNATURES",
           "raw_fwd", "raw_merge"]
