"""GPU parity of the top-k indexer (fmha_index_scores, fmha_topk_select)
against oracle.indexer.

Scores: fp32 on the GPU vs float64, within fp32 accumulation error.  The
selection is an integer decision taken from floating point, so it is checked
in the kernel's precision: the GPU's top-k of its own fp32 scores must equal
the oracle's exact top-k of those same values (bit-exact).  End to end, the
GPU's lists may differ from the float64 top-k only at near-ties."""
import numpy as np
import pytest
import torch

import oracle
from oracle import indexer as OI

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def F():
    import fmha_mqa_fwd_amd
    return fmha_mqa_fwd_amd


def _inputs(B, T, H, c, P, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, T, H, c, generator=g).to(torch.bfloat16)
    k = torch.randn(P, c, generator=g).to(torch.bfloat16)
    w = torch.rand(B, T, H, generator=g) * 2 - 1
    return q, k, w


def _score_bar(ref):
    # fp32 accumulation of ~H*c products: relative error ~1e-6 of the row's scale
    return 1e-5 * (np.abs(ref).max(axis=-1, keepdims=True) + 1.0)


@pytest.mark.parametrize("H,c", [(64, 128), (32, 128), (64, 64), (32, 64)])
@pytest.mark.parametrize("P", [1, 63, 65, 1000, 4097])
def test_scores_match_oracle(F, H, c, P):
    q, k, w = _inputs(2, 3, H, c, P, seed=H + c + P)
    s = F.index_scores(q.to(DEV), k.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    ref = OI.index_scores(q, k, w)
    assert np.all(np.abs(s.cpu().numpy() - ref) <= _score_bar(ref))


def _select_case(F, scores, top_k):
    sel = F.topk_select(scores.to(DEV), top_k)
    torch.cuda.synchronize()
    ref = OI.topk_select(scores.double().numpy(), top_k)
    assert np.array_equal(sel.cpu().numpy().astype(np.int64), ref)


@pytest.mark.parametrize("rows,P,top_k", [(3, 5000, 1024), (2, 32768, 1024), (4, 700, 64),
                                          (2, 1, 1), (3, 10, 16), (2, 1000, 1000),
                                          (1, 32768, 32768), (2, 32768, 1), (2, 31001, 1024),
                                          (3, 2047, 2048)])
def test_selection_is_exact_on_random_scores(F, rows, P, top_k):
    g = torch.Generator().manual_seed(rows * P + top_k)
    _select_case(F, torch.randn(rows, P, generator=g), top_k)


def test_selection_breaks_ties_towards_smaller_ids(F):
    g = torch.Generator().manual_seed(11)
    # few distinct values: the top_k-th value is shared by many entries
    s = torch.randint(-3, 4, (4, 3000), generator=g).float()
    s[1] = 0.0                      # all equal
    s[2, ::2] = -0.0                # -0 and +0 are the same score
    _select_case(F, s, 500)


def test_selection_orders_negative_and_large_values(F):
    s = torch.tensor([[-1e30, 3.5, -0.25, 1e30, 7.0, -7.0, 0.0, 1e-30, -1e-30]])
    _select_case(F, s, 4)
    _select_case(F, s, 9)


def test_indexer_end_to_end_matches_float64_up_to_near_ties(F):
    B, T, H, c, P, top_k = 2, 4, 64, 128, 32768, 1024
    q, k, w = _inputs(B, T, H, c, P, seed=5)
    idx = F.indexer_topk(q.to(DEV), k.to(DEV), w.to(DEV), top_k).cpu().numpy()
    ref_s = OI.index_scores(q, k, w)
    ref = OI.topk_select(ref_s, top_k)
    bar = _score_bar(ref_s)[..., 0]
    for b in range(B):
        for t in range(T):
            got, want = set(idx[b, t].tolist()), set(ref[b, t].tolist())
            kth = np.sort(ref_s[b, t])[::-1][top_k - 1]
            for e in got ^ want:   # only entries within the error bar of the cut may differ
                assert abs(ref_s[b, t, e] - kth) <= 2 * bar[b, t], (b, t, e)
            assert len(got) == top_k and np.all(np.diff(idx[b, t]) > 0)


def test_selected_lists_feed_the_sparse_attention(F):
    """indexer -> kv_idx -> gathered attention, checked against the float64
    attention on the same lists."""
    B, T, H, c, P, n_h, hd, top_k = 1, 4, 32, 64, 4096, 16, 128, 256
    q_i, k_i, w = _inputs(B, T, H, c, P, seed=9)
    g = torch.Generator().manual_seed(10)
    q = torch.randn(B, T, n_h, hd, generator=g).to(torch.bfloat16)
    kp = torch.randn(P, hd, generator=g).to(torch.bfloat16)
    vp = torch.randn(P, hd, generator=g).to(torch.bfloat16)
    idx = F.indexer_topk(q_i.to(DEV), k_i.to(DEV), w.to(DEV), top_k)
    out, lse = F.fwd(q.to(DEV), kp.to(DEV), vp.to(DEV), idx, scale=hd ** -0.5,
                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = oracle.attention(q, kp, vp, hd ** -0.5, kv_idx=idx.cpu())
    m = oracle.row_metrics(out.cpu().numpy().reshape(-1, hd), O.reshape(-1, hd),
                           lse.cpu().numpy().reshape(-1), L.reshape(-1))
    assert m["max_abs"] <= 1e-2 and m["min_row_cos"] >= 0.9999 and m["lse_err"] <= 1e-3, m


def test_indexer_at_the_benchmarked_size_all_tokens(F):
    """The shape bench.py times (B=4, T=512, 64 index heads x 128, a
    32768-entry pool, top-k 1024): every token's scores against float64, and
    every selection bit-exact against the exact top-k of the GPU's own fp32
    scores (the selection is decided in the kernel's precision)."""
    B, T, H, c, P, top_k = 4, 512, 64, 128, 32768, 1024
    q, k, w = _inputs(B, T, H, c, P, seed=4001)
    qd, kd, wd = q.to(DEV), k.to(DEV), w.to(DEV)
    s = F.index_scores(qd, kd, wd)
    idx = F.topk_select(s, top_k)
    torch.cuda.synchronize()
    got_all = s.cpu().numpy()
    idx_all = idx.cpu().numpy().astype(np.int64)
    for b in range(B):
        ref = OI.index_scores(q[b:b + 1], k, w[b:b + 1])[0]          # [T, P] float64
        got = got_all[b]
        tol = 1e-5 * (np.abs(ref).max(axis=1, keepdims=True) + 1.0)
        assert np.all(np.abs(got - ref) <= tol), b
        want = OI.topk_select(got.astype(np.float64), top_k)
        assert np.array_equal(idx_all[b], want), b
