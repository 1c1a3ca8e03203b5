"""Plain float64 softmax attention (multi-query), its split partials and the
log-sum-exp merge — the oracle the HIP path is checked against.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.

What is computed, and where the pages fix it (dev-log pages of the DeepSeek-V4
NVFP4 kernel project):

* Attention itself — QK^T, softmax, PV, output: page "CURRENT ISSUE: UMMA FMHA —
  Full Pipeline + Production", section "What's working" (the QK -> softmax ->
  PV -> output pipeline).  The same page's "Key lessons from this session" says
  the QK product is the *unscaled* dot product and the 1/sqrt(HD) factor is
  applied inside the softmax; so logits are ``x_j = scale * (q . k_j)``.
* Multi-query layout — every query head reads the same K/V head: page "May 24,
  2026 — Session Start Plan", section "Start D2: Multi-Query Grid" (Q indexed
  per head, K/V shared).
* LSE output — the kernel returns O together with the log-sum-exp of the row:
  same page, "D1 Status Summary" (D5a).  Base: the natural log, because the
  merge formula weights parts by exp(lse_i) (next item).
* Merge of parts — ``O = sum_i exp(lse_i) O_i / sum_i exp(lse_i)``: page
  "CURRENT ISSUE: UMMA FMHA — Full Pipeline + Production", "Next steps" item 4
  (Multi-KV-tile).  It is exact only when every O_i is normalised over the keys
  of its own part, which is the reading taken here; the merged LSE is then
  ``ln sum_i exp(lse_i)``, the LSE over all keys.
* Attention sink — page "May 24, 2026 — Session Start Plan" lists a "sink
  merge" (File Map: the decode op holds the "Sink merge formula"; D1 Status
  Summary: "D5b (Python sink merge)") without printing it.  Reading taken: a
  sink is one extra logit per query head, in the units of the scaled logits,
  whose value vector is zero.  It joins the softmax's denominator and nothing
  else: ``lse = ln(sum_j exp(x_j) + exp(sink_h))``, ``O = sum_j exp(x_j - lse)
  V_j``; ``sink_h = -inf`` is no sink.
* Selected keys — a row attends to s_k = top_k keys picked from a KV store: page
  "May 24, 2026 — Session Start Plan", "Key Numbers" (top_k 1024 -> s_k 1024),
  and the ``dsv4/kernels/cuda`` commit log (KV row gather, 32768-row pool).

Readings where the pages are silent: inputs are bf16, converted exactly to
float64; there is no causal or other mask; an empty part (no keys) has O = 0 and
lse = -inf; the split of s_k keys into n parts uses contiguous chunks of
ceil(s_k / n) keys (the result does not depend on the chunking).

All arithmetic is float64 numpy; ``matmul`` is the only library primitive used
for the two contractions.  Rows are processed in chunks purely to bound memory.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["to_f64", "attention_rows", "attention_probs", "attention",
           "attention_sources", "split_partials", "lse_merge"]

_CHUNK_ROWS = 2048


def to_f64(t) -> np.ndarray:
    """Exact conversion of a (CPU) torch tensor of bf16/f32/int to numpy.

    bf16 -> f32 -> f64 is exact, so the oracle sees the very bits the GPU reads.
    Integer tensors keep an integer dtype.
    """
    import torch  # local: the oracle's arithmetic below is numpy only

    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t
    t = t.detach().cpu()
    if t.dtype in (torch.int32, torch.int64, torch.int16, torch.int8, torch.uint8):
        return t.numpy().astype(np.int64)
    return t.to(torch.float32).numpy().astype(np.float64)


def _logits(q_rows: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    # x[r, j] = scale * sum_d q[r, d] * K[j, d]   (scale applied after the product)
    return float(scale) * (q_rows @ K.T)


def attention_probs(q_rows: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Softmax probabilities p[r, j] = exp(x_rj - m_r) / sum_j' exp(x_rj' - m_r)."""
    x = _logits(q_rows, K, scale)
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=1, keepdims=True)


def attention_rows(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
                   scale: float, sink_rows=None):
    """Attention of independent query rows against one shared K/V set.

    q_rows [R, hd], K [S, hd], V [S, hd]  ->  (O [R, hd], lse [R]).
    O[r] = sum_j p_rj V[j];  lse[r] = m_r + ln sum_j exp(x_rj - m_r).
    S = 0 gives O = 0 and lse = -inf (empty part).
    sink_rows [R] (optional): each row's sink logit, one more term of the
    softmax's denominator with a zero value vector (-inf: none).
    """
    R, hd = q_rows.shape
    sink = None if sink_rows is None else np.asarray(sink_rows, np.float64).reshape(R, 1)
    if K.shape[0] == 0:
        lse = np.full(R, -np.inf) if sink is None else sink[:, 0].copy()
        return np.zeros((R, V.shape[1]), np.float64), lse
    x = _logits(q_rows, K, scale)
    m = x.max(axis=1, keepdims=True)
    if sink is not None:
        m = np.maximum(m, sink)
    e = np.exp(x - m)
    l = e.sum(axis=1, keepdims=True)
    if sink is not None:
        l = l + np.exp(sink - m)
    o = (e / l) @ V
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def _kv_for_group(k, v, kv_idx, b, t):
    if kv_idx is None:
        return k[b], v[b]
    sel = kv_idx[b, t]
    return k[sel], v[sel]


def attention(q, k, v, scale: float, kv_idx=None, rows=None,
              key_range=None, sink=None):
    """Multi-query attention forward in float64.

    q [B, T, n_h, hd]; dense: k, v [B, s_k, hd]; gather: k, v [P, hd] pools and
    kv_idx [B, T, s_k] (row j of token (b, t) is pool row kv_idx[b, t, j]).

    rows: None for every row, else flat row ids r = (b*T + t)*n_h + h; the
    result is then [len(rows), hd] / [len(rows)] in the given order.
    key_range: optional (lo, hi) restricting attention to keys lo..hi-1 of each
    row's key list (used to form split partials).
    sink: optional [n_h] sink logits (natural-log units, -inf = none), one per
    query head.

    Returns (O, lse) as float64; full shape [B, T, n_h, hd] and [B, T, n_h].
    """
    q = to_f64(q)
    k = to_f64(k)
    v = to_f64(v)
    kv_idx = to_f64(kv_idx)
    sink = None if sink is None else to_f64(sink).reshape(-1)
    B, T, n_h, hd = q.shape
    dv = v.shape[-1]
    if rows is None:
        flat = np.arange(B * T * n_h)
    else:
        flat = np.asarray(rows, dtype=np.int64).reshape(-1)
    O = np.empty((flat.size, dv), np.float64)
    L = np.empty(flat.size, np.float64)
    qf = q.reshape(B * T * n_h, hd)
    b_of = flat // (T * n_h)
    t_of = (flat // n_h) % T
    # group rows that share one K/V set: per batch (dense) or per token (gather)
    gkey = b_of if kv_idx is None else b_of * T + t_of
    order = np.argsort(gkey, kind="stable")
    bounds = np.flatnonzero(np.diff(gkey[order])) + 1
    for grp in np.split(order, bounds):
        if grp.size == 0:
            continue
        b, t = int(b_of[grp[0]]), int(t_of[grp[0]])
        K, V = _kv_for_group(k, v, kv_idx, b, t)
        if key_range is not None:
            K, V = K[key_range[0]:key_range[1]], V[key_range[0]:key_range[1]]
        for c0 in range(0, grp.size, _CHUNK_ROWS):
            sel = grp[c0:c0 + _CHUNK_ROWS]
            o, lse = attention_rows(qf[flat[sel]], K, V, scale,
                                    None if sink is None else sink[flat[sel] % n_h])
            O[sel] = o
            L[sel] = lse
    if rows is None:
        return O.reshape(B, T, n_h, dv), L.reshape(B, T, n_h)
    return O, L


def attention_sources(q, sources, scale: float, rows=None, sink=None):
    """Attention of every query row over the union of several key sources.

    Reading of the multi-source decode (the dsv4/kernels/cuda commit log keeps
    a compressed KV store read through top-k row gathers and a sliding-window
    KV store, KVCache.append_swa and gather_kv / gather_swa; their window
    semantics are not printed): each source is ``(k, v, kv_idx)`` — dense
    ``k, v [B, S, hd]`` with ``kv_idx None``, or pools ``[P, hd]`` with
    ``kv_idx [B, T, S]`` — and token (b, t) attends to the concatenation of all
    sources' keys for it, in one softmax.  Same outputs as ``attention``.
    """
    q = to_f64(q)
    B, T, n_h, hd = q.shape
    srcs = [(to_f64(k), to_f64(v), to_f64(i)) for k, v, i in sources]
    dv = srcs[0][1].shape[-1]
    sink = None if sink is None else to_f64(sink).reshape(-1)
    flat = (np.arange(B * T * n_h) if rows is None
            else np.asarray(rows, dtype=np.int64).reshape(-1))
    O = np.empty((flat.size, dv), np.float64)
    L = np.empty(flat.size, np.float64)
    qf = q.reshape(B * T * n_h, hd)
    tok = flat // n_h
    order = np.argsort(tok, kind="stable")
    bounds = np.flatnonzero(np.diff(tok[order])) + 1
    for grp in np.split(order, bounds):
        if grp.size == 0:
            continue
        b, t = divmod(int(tok[grp[0]]), T)
        kv = [_kv_for_group(k, v, i, b, t) for k, v, i in srcs]
        K = np.concatenate([x[0] for x in kv], axis=0)
        V = np.concatenate([x[1] for x in kv], axis=0)
        o, lse = attention_rows(qf[flat[grp]], K, V, scale,
                                None if sink is None else sink[flat[grp] % n_h])
        O[grp] = o
        L[grp] = lse
    if rows is None:
        return O.reshape(B, T, n_h, dv), L.reshape(B, T, n_h)
    return O, L


def split_partials(q, k, v, scale: float, num_splits: int, kv_idx=None,
                   rows=None):
    """Per-part (O_i, lse_i) for keys cut into ``num_splits`` contiguous chunks
    of ceil(s_k / num_splits) keys.  Each O_i is normalised over its own keys.

    Returns o_parts [num_splits, R, hd], lse_parts [num_splits, R] (R = all rows
    flattened, or len(rows)).
    """
    s_k = (to_f64(kv_idx).shape[-1] if kv_idx is not None
           else to_f64(k).shape[1])
    chunk = -(-s_k // num_splits)
    outs, lses = [], []
    for i in range(num_splits):
        lo, hi = min(i * chunk, s_k), min((i + 1) * chunk, s_k)
        o, lse = attention(q, k, v, scale, kv_idx=kv_idx, rows=rows,
                           key_range=(lo, hi))
        outs.append(o.reshape(-1, o.shape[-1]))
        lses.append(lse.reshape(-1))
    return np.stack(outs), np.stack(lses)


def lse_merge(o_parts, lse_parts):
    """Merge normalised partial outputs by their log-sum-exps.

    o_parts [P, R, hd], lse_parts [P, R] (natural log; -inf = empty part)
      M   = max_i lse_i
      w_i = exp(lse_i - M)
      O   = sum_i w_i O_i / sum_i w_i ,   lse = M + ln sum_i w_i
    A row whose parts are all empty gets O = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    M = lse_parts.max(axis=0)
    live = np.isfinite(M)
    Ms = np.where(live, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Ms[None, :]), 0.0)
    den = w.sum(axis=0)
    num = (w[:, :, None] * o_parts).sum(axis=0)
    O = np.where(live[:, None], num / np.where(live, den, 1.0)[:, None], 0.0)
    lse = np.where(live, Ms + np.log(np.where(live, den, 1.0)), -np.inf)
    return O, lse


def row_metrics(o_test, o_ref, lse_test=None, lse_ref=None):
    """Comparison metrics: max |diff|, minimum per-row cosine (1 for two zero
    rows), global cosine, max |lse diff| (None when no lse given)."""
    a = np.asarray(o_test, np.float64).reshape(-1, np.shape(o_ref)[-1])
    b = np.asarray(o_ref, np.float64).reshape(a.shape)
    max_abs = float(np.max(np.abs(a - b))) if a.size else 0.0
    na = np.linalg.norm(a, axis=1)
    nb = np.linalg.norm(b, axis=1)
    dot = (a * b).sum(axis=1)
    both_zero = (na == 0) & (nb == 0)
    cos = np.where(both_zero, 1.0, dot / np.maximum(na * nb, 1e-300))
    gcos = float((a * b).sum() / max(math.sqrt((a * a).sum() * (b * b).sum()), 1e-300))
    lse_err = None
    if lse_test is not None:
        lt = np.asarray(lse_test, np.float64).reshape(-1)
        lr = np.asarray(lse_ref, np.float64).reshape(-1)
        same_inf = np.isinf(lt) & np.isinf(lr) & (np.sign(lt) == np.sign(lr))
        with np.errstate(invalid="ignore"):
            d = np.where(same_inf, 0.0, np.abs(lt - lr))
        lse_err = float(np.max(d)) if d.size else 0.0
    return {"max_abs": max_abs, "min_row_cos": float(cos.min()) if cos.size else 1.0,
            "global_cos": gcos, "lse_err": lse_err}
