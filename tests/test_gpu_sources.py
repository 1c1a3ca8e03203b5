"""GPU parity of attention over several key sources (top-k rows gathered from
a compressed pool + a dense sliding window), composed from
fmha_mqa_fwd_sources_partials (every source's split partials in one call),
fmha_lse_merge and the sink, against oracle.attention_sources (one softmax
over the concatenated keys).  Same bar as the plain forward; the one-call
partials also equal fmha_mqa_fwd_partials per source bit for bit."""
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


@pytest.mark.parametrize("splits", [(4, 1), (8, 4)])
def test_two_sources_benchmarked_size_all_rows(F, splits):
    """The multi-source row at full size: B=32, 64 heads, hd 512, top-k 512
    of a 32768-row pool plus a 128-key window, bf16 out, every row against
    the one-softmax oracle; bench.py times it with (4, 1) splits (every
    workgroup of the one launch takes 128 keys)."""
    q, top, win, scale = _inputs(B=32, T=1, n_h=64, hd=512, pool=32768, top_k=512, window=128,
                                 seed=98 + splits[0])
    out, lse = F.fwd_sources(q.to(DEV), [_d(top, splits[0]), _d(win, splits[1])], scale=scale,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check(out, lse, q, [top, win], scale)


def _top_and_window(B, T, n_h, hd, pool, top_k, window, seed, mask=True):
    """Inputs as _inputs; with mask, some top-k entries are invalid (outside
    [0, pool): masked keys)."""
    q, top, win, scale = _inputs(B=B, T=T, n_h=n_h, hd=hd, pool=pool, top_k=max(top_k, 1),
                                 window=window, seed=seed)
    kp, vp, idx = top
    if top_k == 0:
        idx = torch.zeros((B, T, 0), dtype=torch.int32)
    elif mask:
        idx = idx.clone()
        idx[0, 0, ::7] = -1           # masked entries: outside [0, pool)
        idx[-1, -1, 1::5] = pool + 3
    return q, (kp, vp, idx), win, scale


@pytest.mark.parametrize("hd,B,T,n_h,pool,top_k,window,splits", [
    (512, 2, 1, 64, 4096, 512, 128, (4, 2)),   # one launch, the decode shape
    (512, 2, 2, 32, 4096, 600, 128, (1, 1)),   # one launch; a 19-tile list in region order
    (512, 2, 3, 24, 2048, 300, 70, (3, 2)),    # one launch; token groups beside batch groups
    (512, 1, 2, 8, 512, 0, 40, (1, 1)),        # an empty top-k source
    (512, 3, 1, 16, 1024, 100, 33, (1, 3)),
    (128, 2, 3, 16, 2048, 200, 64, (2, 1)),    # one launch per source
])
def test_sources_partials_equal_per_source_partials(F, hd, B, T, n_h, pool, top_k, window,
                                                    splits):
    """fmha_mqa_fwd_sources_partials writes, plane for plane and bit for bit,
    what fmha_mqa_fwd_partials writes for each source on its own."""
    q, top, win, scale = _top_and_window(B, T, n_h, hd, pool, top_k, window, seed=300 + hd + T)
    qd = q.to(DEV)
    srcs = [_d(top, splits[0]), _d(win, splits[1])]
    o, lse = F.fwd_sources_partials(qd, srcs, scale)
    first = 0
    for src in srcs:
        o1, l1 = F.fwd_partials(qd, src[0], src[1], src[2], scale, src[3])
        torch.cuda.synchronize()
        s = src[3]
        assert torch.equal(o[first:first + s], o1), first
        assert torch.equal(lse[first:first + s], l1), first
        first += s
    assert first == o.shape[0]


@pytest.mark.parametrize("n_src", [3, 5])
def test_several_sources_at_hd512(F, n_src):
    """Three sources run in one launch, five (over the one-launch limit of
    four) in one launch each; both match the one-softmax oracle over all keys
    and the per-source partials bit for bit."""
    q, top, win, scale = _top_and_window(2, 2, 16, 512, 1024, 96, 40, seed=400, mask=False)
    srcs_h = [top, win]
    for i in range(n_src - 2):
        _, t2, _, _ = _top_and_window(2, 2, 16, 512, 700, 50 + 9 * i, 1, seed=410 + i,
                                      mask=False)
        srcs_h.append(t2)
    qd = q.to(DEV)
    srcs = [_d(s, 1 + (i % 3)) for i, s in enumerate(srcs_h)]
    o, lse = F.fwd_sources_partials(qd, srcs, scale)
    first = 0
    for src in srcs:
        o1, l1 = F.fwd_partials(qd, src[0], src[1], src[2], scale, src[3])
        torch.cuda.synchronize()
        s = src[3]
        assert torch.equal(o[first:first + s], o1) and torch.equal(lse[first:first + s], l1)
        first += s
    out, L = F.fwd_sources(qd, srcs, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(out, L, q, srcs_h, scale)
