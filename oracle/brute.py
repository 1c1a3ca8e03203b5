"""Scalar pure-Python attention, one row and one key at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It restates the same
definition as ``oracle.attention`` without numpy: logits ``x_j = scale * q.k_j``
(the scale applied in the softmax, page "CURRENT ISSUE: UMMA FMHA — Full
Pipeline + Production", "Key lessons from this session"), the max-shifted
exponentials, ``math.fsum`` for every sum, ``O = sum_j p_j V_j`` and
``lse = m + ln sum_j exp(x_j - m)``.  It is only run on tiny shapes, where its
exactly rounded sums make it the tie-breaker for ``oracle.fp64``.

With a sink (one logit per query head, zero value vector; the reading of the
sink merge named on page "May 24, 2026 — Session Start Plan") the sink logit is
one more term of the softmax's denominator.
"""
from __future__ import annotations

import math

__all__ = ["brute_attention", "brute_merge"]


def _row(qr, keys, vals, scale, sink=-math.inf):
    xs = [scale * math.fsum(a * b for a, b in zip(qr, kj)) for kj in keys]
    if not xs:
        return [0.0] * len(vals[0]) if vals else [], sink
    m = max(xs + [sink])
    es = [math.exp(x - m) for x in xs]
    l = math.fsum(es + [math.exp(sink - m)])
    hd = len(vals[0])
    o = [math.fsum(es[j] * vals[j][d] for j in range(len(es))) / l for d in range(hd)]
    return o, m + math.log(l)


def brute_attention(q, k, v, scale, kv_idx=None, sink=None):
    """q nested lists [B][T][n_h][hd]; dense k, v [B][s_k][hd]; gather k, v
    [P][hd] with kv_idx [B][T][s_k]; optional sink [n_h].  Returns
    (O [B][T][n_h][hd], lse [B][T][n_h]) as nested Python lists of floats."""
    O, L = [], []
    for b in range(len(q)):
        Ob, Lb = [], []
        for t in range(len(q[b])):
            if kv_idx is None:
                keys, vals = k[b], v[b]
            else:
                keys = [k[i] for i in kv_idx[b][t]]
                vals = [v[i] for i in kv_idx[b][t]]
            Ot, Lt = [], []
            for h in range(len(q[b][t])):
                o, lse = _row(q[b][t][h], keys, vals, scale,
                              -math.inf if sink is None else sink[h])
                Ot.append(o)
                Lt.append(lse)
            Ob.append(Ot)
            Lb.append(Lt)
        O.append(Ob)
        L.append(Lb)
    return O, L


def brute_merge(o_parts, lse_parts):
    """Merge of per-part rows: o_parts [P][R][hd], lse_parts [P][R]."""
    P = len(lse_parts)
    R = len(lse_parts[0])
    hd = len(o_parts[0][0])
    O, L = [], []
    for r in range(R):
        ls = [lse_parts[i][r] for i in range(P)]
        M = max(ls)
        if M == -math.inf:
            O.append([0.0] * hd)
            L.append(-math.inf)
            continue
        w = [math.exp(x - M) if x != -math.inf else 0.0 for x in ls]
        den = math.fsum(w)
        O.append([math.fsum(w[i] * o_parts[i][r][d] for i in range(P)) / den
                  for d in range(hd)])
        L.append(M + math.log(den))
    return O, L
