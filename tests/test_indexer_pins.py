"""Pins of the indexer oracle (oracle.indexer) against what fixes it
independently: brute-force scalar scores, closed forms, torch.topk and a
sort-based brute-force selection; plus planted mistakes that must fail."""
import math

import numpy as np
import pytest
import torch

from oracle import indexer as I


def _inputs(B, T, H, c, P, seed, nonneg=False):
    g = np.random.default_rng(seed)
    q = torch.from_numpy(g.standard_normal((B, T, H, c))).to(torch.bfloat16)
    k = torch.from_numpy(g.standard_normal((P, c))).to(torch.bfloat16)
    if nonneg:
        q, k = q.abs(), k.abs()
    w = torch.from_numpy(g.uniform(-1, 1, (B, T, H)).astype(np.float32))
    return q, k, w


def _brute_scores(q, k, w):
    qf, kf, wf = (x.double().tolist() for x in (q, k, w))
    B, T, H = len(qf), len(qf[0]), len(qf[0][0])
    out = []
    for b in range(B):
        rows = []
        for t in range(T):
            row = []
            for kr in kf:
                terms = [wf[b][t][h] * max(0.0, math.fsum(a * x for a, x in zip(qf[b][t][h], kr)))
                         for h in range(H)]
                row.append(math.fsum(terms))
            rows.append(row)
        out.append(rows)
    return np.array(out)


@pytest.mark.parametrize("B,T,H,c,P", [(1, 1, 1, 1, 3), (2, 3, 4, 8, 7), (1, 2, 32, 16, 5)])
def test_scores_match_brute_force(B, T, H, c, P):
    q, k, w = _inputs(B, T, H, c, P, seed=B + T + H + c + P)
    np.testing.assert_allclose(I.index_scores(q, k, w), _brute_scores(q, k, w), rtol=1e-12,
                               atol=1e-12)


def test_one_hot_weight_picks_one_head_relu():
    q, k, w = _inputs(1, 2, 5, 16, 9, seed=3)
    w = torch.zeros_like(w)
    w[..., 2] = 1.0
    d = q[0, :, 2].double() @ k.double().T
    np.testing.assert_allclose(I.index_scores(q, k, w)[0], np.maximum(d.numpy(), 0), rtol=1e-13)


def test_nonnegative_inputs_make_the_score_linear():
    """q, k >= 0: every dot product is >= 0, so the ReLU is inactive and the
    score is the single dot product (sum_h w_h q_h) . k."""
    q, k, w = _inputs(2, 2, 6, 12, 8, seed=4, nonneg=True)
    lin = torch.einsum("bth,bthc->btc", w.double(), q.double()) @ k.double().T
    np.testing.assert_allclose(I.index_scores(q, k, w), lin.numpy(), rtol=1e-12, atol=1e-12)


def test_selection_matches_torch_topk_on_distinct_scores():
    g = np.random.default_rng(5)
    s = g.permutation(5000).reshape(2, 2500).astype(np.float64) * 0.37
    sel = I.topk_select(s, 100)
    ref = torch.topk(torch.from_numpy(s), 100, dim=-1).indices.numpy()
    assert np.array_equal(sel, np.sort(ref, axis=-1))
    assert np.all(np.diff(sel, axis=-1) > 0)


def test_selection_ties_go_to_the_smaller_id():
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 3.0, 0.0]])
    assert I.topk_select(s, 3).tolist() == [[1, 2, 4]]
    brute = sorted(range(7), key=lambda i: (-s[0, i], i))[:3]
    assert sorted(brute) == [1, 2, 4]


def test_selection_pads_short_pools():
    s = np.array([[0.5, -1.0, 2.0]])
    assert I.topk_select(s, 5).tolist() == [[0, 1, 2, -1, -1]]


def test_planted_mistakes_fail_a_pin():
    """Four plausible misreadings, each swapped into the oracle in turn, must
    each fail at least one pin: the ReLU dropped, the ReLU applied after the
    head weighting, the selection listed in descending id order, and ties
    broken towards the larger id."""
    good_scores, good_sel = I.index_scores, I.topk_select

    def no_relu(q, k, w):
        q, k, w = (x.double().numpy() for x in (q, k, w))
        return np.einsum("bth,bthp->btp", w, q @ k.T)

    def relu_after_weighting(q, k, w):
        q, k, w = (x.double().numpy() for x in (q, k, w))
        return np.maximum(w[..., None] * (q @ k.T), 0.0).sum(axis=2)

    def descending_ids(scores, top_k):
        sel = good_sel(scores, top_k)
        n = min(top_k, np.shape(scores)[-1])
        out = sel.copy()
        out[..., :n] = sel[..., :n][..., ::-1]
        return out

    def ties_to_larger(scores, top_k):
        s = np.asarray(scores, np.float64)
        P = s.shape[-1]
        out = []
        for row in s.reshape(-1, P):
            order = sorted(range(P), key=lambda i: (-row[i], -i))[:top_k]
            out.append(sorted(order) + [-1] * (top_k - len(order)))
        return np.array(out).reshape(*s.shape[:-1], top_k)

    pins = (lambda: test_scores_match_brute_force(2, 3, 4, 8, 7),
            test_one_hot_weight_picks_one_head_relu,
            test_nonnegative_inputs_make_the_score_linear,
            test_selection_matches_torch_topk_on_distinct_scores,
            test_selection_ties_go_to_the_smaller_id,
            test_selection_pads_short_pools)
    for name, patch in (("index_scores", no_relu), ("index_scores", relu_after_weighting),
                        ("topk_select", descending_ids), ("topk_select", ties_to_larger)):
        setattr(I, name, patch)
        try:
            caught = 0
            for chk in pins:
                try:
                    chk()
                except AssertionError:
                    caught += 1
            assert caught >= 1, f"planted mistake {patch.__name__} passed every pin"
        finally:
            I.index_scores, I.topk_select = good_scores, good_sel
