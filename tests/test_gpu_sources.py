"""GPU parity of attention over several key sources (top-k rows gathered from
a compressed pool + a dense sliding window), composed from fmha_mqa_fwd per
source, fmha_lse_merge and the sink, against oracle.attention_sources (one
softmax over the concatenated keys).  Same bar as the plain forward."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

MAX_ABS, MIN_COS, LSE_ERR = 1e-2, 0.9999, 1e-3
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def F():
    import fmha_mqa_fwd_amd
    return fmha_mqa_fwd_amd


def _inputs(B, T, n_h, hd, pool, top_k, window, seed):
    top = W.make_custom(B=B, T=T, n_h=n_h, hd=hd, s_k=top_k, pool=pool, out_dtype="bf16",
                        seed=seed)
    q, kp, vp, idx = W.make_inputs(top)
    win = W.make_custom(B=B, T=1, n_h=1, hd=hd, s_k=window, out_dtype="bf16", seed=seed + 1)
    _, kw, vw, _ = W.make_inputs(win)
    return q, (kp, vp, idx), (kw, vw, None), top.scale


def _check(out, lse, q, srcs, scale, sink=None):
    O_ref, L_ref = oracle.attention_sources(q, srcs, scale, sink=sink)
    hd = q.shape[-1]
    m = oracle.row_metrics(out.float().reshape(-1, hd).cpu().numpy(), O_ref.reshape(-1, hd),
                           lse.reshape(-1).cpu().numpy(), L_ref.reshape(-1))
    assert m["max_abs"] <= MAX_ABS, m
    assert m["min_row_cos"] >= MIN_COS, m
    assert m["lse_err"] <= LSE_ERR, m


def _d(src, splits=1):
    k, v, i = src
    return (k.to(DEV), v.to(DEV), None if i is None else i.to(DEV), splits)


@pytest.mark.parametrize("hd,top_k,window,splits,with_sink", [
    (128, 512, 128, 1, False),
    (128, 512, 128, 2, True),
    (64, 300, 45, 3, True),
    (256, 128, 64, 1, False),
])
def test_topk_plus_window_matches_one_softmax(F, hd, top_k, window, splits, with_sink):
    q, top, win, scale = _inputs(B=2, T=3, n_h=16, hd=hd, pool=4096, top_k=top_k,
                                 window=window, seed=90 + hd)
    sink = None
    if with_sink:
        sink = torch.from_numpy(np.random.default_rng(1).normal(0, 2, 16).astype(np.float32))
    out, lse = F.fwd_sources(q.to(DEV), [_d(top, splits), _d(win)], scale=scale,
                             out_dtype=torch.bfloat16,
                             sink=None if sink is None else sink.to(DEV))
    torch.cuda.synchronize()
    _check(out, lse, q, [top, win], scale, None if sink is None else sink.double().numpy())


def test_empty_window_leaves_the_topk_result(F):
    q, top, _, scale = _inputs(B=1, T=4, n_h=8, hd=128, pool=2048, top_k=256, window=1, seed=95)
    empty = (torch.zeros(1, 0, 128, dtype=torch.bfloat16),) * 2 + (None,)
    out, lse = F.fwd_sources(q.to(DEV), [_d(top), _d(empty)], scale=scale,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(out, lse, q, [top], scale)


def test_decode_shape_two_sources(F):
    """A decode step at a DeepSeek-V4 Flash-like shape: 64 heads, top-k 512 of
    a 32768-row pool plus a 128-key window, one token per sequence."""
    q, top, win, scale = _inputs(B=16, T=1, n_h=64, hd=128, pool=32768, top_k=512,
                                 window=128, seed=97)
    out, lse = F.fwd_sources(q.to(DEV), [_d(top), _d(win)], scale=scale,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check(out, lse, q, [top, win], scale)


def test_two_sources_benchmarked_size_sampled(F):
    """The multi-source row as bench.py times it: B=32, 64 heads, hd 512,
    top-k 512 of a 32768-row pool (8 splits) plus a 128-key window (4 splits),
    bf16 out; rows sampled against the one-softmax oracle."""
    q, top, win, scale = _inputs(B=32, T=1, n_h=64, hd=512, pool=32768, top_k=512, window=128,
                                 seed=98)
    out, lse = F.fwd_sources(q.to(DEV), [_d(top, 8), _d(win, 4)], scale=scale,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.concatenate([[0, 32 * 64 - 1], np.random.default_rng(9).choice(32 * 64, 200,
                                                                            replace=False)])
    O_ref, L_ref = oracle.attention_sources(q, [top, win], scale, rows=rows)
    ri = torch.as_tensor(rows, device=out.device)
    m = oracle.row_metrics(out.float().reshape(-1, 512)[ri].cpu().numpy(), O_ref,
                           lse.reshape(-1)[ri].cpu().numpy(), L_ref)
    assert m["max_abs"] <= MAX_ABS and m["min_row_cos"] >= MIN_COS and m["lse_err"] <= LSE_ERR, m
