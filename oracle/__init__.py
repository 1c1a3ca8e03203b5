"""CPU oracle for the MQA attention forward — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and shares no
code with it; the two meet only through the seeded tensors of ``workloads``.

Contents
  * ``oracle.fp64``      — plain softmax attention, numpy float64, rows chunked
    only to bound memory (no tiling, no online rescale, no fusion).
  * ``oracle.brute``     — the same definition as scalar pure-Python loops with
    ``math.fsum``; used on tiny shapes to pin ``oracle.fp64``.
  * ``oracle.indexer``   — top-k indexer scores (float64) and the exact top-k
    selection that produce gather lists.

Every function here is pinned by CPU tests (brute force, closed forms, library
routines, invariants); none is "parity unpinned".
"""
from .fp64 import (attention, attention_rows, attention_probs, attention_sources,
                   lse_merge, row_metrics, split_partials, to_f64)
from .indexer import index_scores, topk_select

__all__ = ["attention", "attention_rows", "attention_probs", "attention_sources", "lse_merge",
           "index_scores", "topk_select",
           "row_metrics", "split_partials", "to_f64"]
