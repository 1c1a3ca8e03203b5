"""Top-k indexer that produces the gather lists (``kv_idx``) — plain float64
scores and an exact top-k selection.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` only, never by the product
path.

What the pages fix (the dsv4/kernels/cuda commit log, indexer_score_topk):
index scores are formed per index head with per-head weights (a 64-entry
weight array), the 1024 best pool entries are kept for each token (a 1024-entry
heap of scores and entry ids), and the selection is checked by exact match
against ``torch.topk``.  The score formula itself is not printed; the reading
taken is the DeepSeek sparse-attention indexer form, with one index key per
pool entry shared by the index heads:

    score[b, t, s] = sum_h w[b, t, h] * max(0, q[b, t, h, :] . k[s, :])

(q: bf16 index queries [B, T, H, c]; k: bf16 index keys [P, c]; w: fp32 head
weights [B, T, H]).  The pages' FP4 key format is not part of this reading.

Selection (reading where the pages are silent): the ``top_k`` entries with
the largest scores, ties broken towards the smaller entry id, returned in
ascending entry-id order; when the pool has fewer than ``top_k`` entries every
entry is kept and the list is padded with -1 (a key the attention masks).
"""
from __future__ import annotations

import numpy as np

from .fp64 import to_f64

__all__ = ["index_scores", "topk_select"]


def index_scores(q, k, w) -> np.ndarray:
    """score [B, T, P] in float64 (``matmul`` is the only library primitive)."""
    q = to_f64(q)
    k = to_f64(k)
    w = to_f64(w)
    B, T, H, c = q.shape
    out = np.empty((B, T, k.shape[0]), np.float64)
    for b in range(B):
        for t in range(T):
            d = q[b, t] @ k.T                     # [H, P]: one dot product per head and entry
            out[b, t] = w[b, t] @ np.maximum(d, 0.0)
    return out


def topk_select(scores, top_k: int) -> np.ndarray:
    """Exact top-k of each row of ``scores`` [..., P]: int64 [..., top_k] entry
    ids in ascending order (ties towards the smaller id, -1 padding)."""
    s = np.asarray(scores, np.float64)
    lead, P = s.shape[:-1], s.shape[-1]
    flat = s.reshape(-1, P)
    res = np.full((flat.shape[0], top_k), -1, np.int64)
    n = min(top_k, P)
    for r in range(flat.shape[0]):
        # order by (score descending, id ascending); keep the first n ids
        order = np.lexsort((np.arange(P), -flat[r]))
        res[r, :n] = np.sort(order[:n])
    return res.reshape(*lead, top_k)
