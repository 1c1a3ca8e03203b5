"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar (every case): max |O - O_ref| <= 1e-2, minimum per-row cosine >= 0.9999,
max |lse - lse_ref| <= 1e-3, with O_ref, lse_ref from oracle.fp64 on the very
bf16 inputs the GPU read.  Every case compares every row, the full-size
prefill, decode and sparse top-k workloads and the head-dim-512 rows at their
benchmarked sizes included.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from conftest import say

pytestmark = pytest.mark.gpu

MAX_ABS, MIN_COS, LSE_ERR = 1e-2, 0.9999, 1e-3


@pytest.fixture(scope="module")
def F():
    import fmha_mqa_fwd_amd
    return fmha_mqa_fwd_amd


def _dt(name):
    return torch.float32 if name == "f32" else torch.bfloat16


def _run(F, q, k, v, idx, scale, out_dtype, num_splits):
    dev = torch.device("cuda:0")
    out, lse = F.fwd(q.to(dev), k.to(dev), v.to(dev), None if idx is None else idx.to(dev),
                     scale=scale, out_dtype=out_dtype, num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse


def _check(out, lse, q, k, v, idx, scale, rows=None, bar=(MAX_ABS, MIN_COS, LSE_ERR)):
    hd = q.shape[-1]
    O_ref, L_ref = oracle.attention(q, k, v, scale, kv_idx=idx, rows=rows)
    o = out.float().reshape(-1, hd)
    l_ = lse.reshape(-1)
    if rows is not None:
        ri = torch.as_tensor(rows, device=o.device)
        o, l_ = o[ri], l_[ri]
    m = oracle.row_metrics(o.cpu().numpy(), O_ref, l_.cpu().numpy(), L_ref)
    assert m["max_abs"] <= bar[0], m
    assert m["min_row_cos"] >= bar[1], m
    assert m["lse_err"] <= bar[2], m
    return m


def _case(F, w, rows=None):
    q, k, v, idx = W.make_inputs(w)
    out, lse = _run(F, q, k, v, idx, w.scale, _dt(w.out_dtype), w.num_splits)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    m = _check(out, lse, q, k, v, idx, w.scale, rows=rows)
    # the measured margins, on the real stderr (pytest captures stdout)
    say(f"[parity] {w.describe()}{'' if rows is None else f' ({len(rows)} sampled rows)'}: "
        f"max_abs {m['max_abs']:.3e} min_row_cos {m['min_row_cos']:.7f} "
        f"lse_err {m['lse_err']:.3e}")
    return m


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("cid", [1, 2])
def test_small_workloads_all_rows(F, cid):
    _case(F, W.get(cid))


def test_mqa_decode_split8_all_rows(F):
    _case(F, W.get(3))


def test_mqa_prefill_full_size_all_rows(F):
    """The prefill workload at its full size (B=2, T=4096, 64 heads, s_k=1024:
    524288 rows), every row against the oracle."""
    _case(F, W.get(4))


def test_sparse_topk_full_size_all_rows(F):
    """The sparse top-k workload at its full size (B=4, T=512, 128 heads,
    1024 of 32768 pool rows per token: 262144 rows), every row."""
    _case(F, W.get(5))


# ------------------------------------------------------------------ sweeps
@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("s_k", [1, 7, 64, 129, 256, 1000])
def test_head_dim_and_key_count_sweep(F, hd, s_k):
    w = W.make_custom(B=2, T=3, n_h=37, hd=hd, s_k=s_k, out_dtype="f32", seed=hd * 7 + s_k)
    _case(F, w)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("rows", [(1, 1, 1), (1, 129, 2), (3, 5, 64), (1, 2, 200), (2, 1, 300)])
def test_ragged_row_counts(F, hd, rows):
    B, T, n_h = rows
    w = W.make_custom(B=B, T=T, n_h=n_h, hd=hd, s_k=300, out_dtype="bf16", seed=B * T * n_h + hd)
    _case(F, w)


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 13])
@pytest.mark.parametrize("hd", [64, 128, 256, 512])
def test_split_kv(F, splits, hd):
    w = W.make_custom(B=3, T=1, n_h=128, hd=hd, s_k=1000, out_dtype="bf16",
                      num_splits=splits, seed=splits * 31 + hd)
    _case(F, w)


@pytest.mark.parametrize("hd,pool,s_k,splits", [(128, 0, 300, 3), (512, 0, 300, 3),
                                                (128, 2048, 333, 4), (512, 2048, 333, 4),
                                                (64, 0, 9, 8), (256, 700, 9, 8)])
def test_partials_entry_point_planes_are_the_splits(F, hd, pool, s_k, splits):
    """fmha_mqa_fwd_partials: plane i is attention over split i's keys alone
    (contiguous chunks of ceil(s_k / splits); a split without keys gives O = 0,
    lse = -inf), and the planes merged equal attention over all keys."""
    w = W.make_custom(B=2, T=2, n_h=48, hd=hd, s_k=s_k, pool=pool, out_dtype="f32",
                      num_splits=splits, seed=hd + s_k + splits)
    q, k, v, idx = W.make_inputs(w)
    dev = torch.device("cuda:0")
    o_parts, l_parts = F.fwd_partials(q.to(dev), k.to(dev), v.to(dev),
                                      None if idx is None else idx.to(dev), scale=w.scale,
                                      num_splits=splits)
    torch.cuda.synchronize()
    c = -(-s_k // splits)
    for i in range(splits):
        lo, hi = min(i * c, s_k), min((i + 1) * c, s_k)
        if hi <= lo:
            assert torch.all(o_parts[i] == 0) and torch.all(torch.isneginf(l_parts[i]))
            continue
        if idx is None:
            ks, vs, ids = k[:, lo:hi].contiguous(), v[:, lo:hi].contiguous(), None
        else:
            ks, vs, ids = k, v, idx[:, :, lo:hi].contiguous()
        _check(o_parts[i], l_parts[i], q, ks, vs, ids, w.scale)
    rows = w.B * w.T * w.n_h
    out, lse = F.lse_merge(o_parts.view(splits, rows, hd), l_parts.view(splits, rows),
                           torch.float32)
    torch.cuda.synchronize()
    _check(out.view(w.B, w.T, w.n_h, hd), lse.view(w.B, w.T, w.n_h), q, k, v, idx, w.scale)


def test_partials_through_the_two_workgroup_hd512_gather(F):
    """fmha_mqa_fwd_partials with gathered splits of 300 keys over 600
    workgroups (the single-stage kernel, two per CU): each plane is attention
    over its split's keys."""
    w = W.make_custom(B=1, T=300, n_h=16, hd=512, s_k=600, pool=4096, out_dtype="f32",
                      num_splits=2, seed=92)
    q, k, v, idx = W.make_inputs(w)
    dev = torch.device("cuda:0")
    o_parts, l_parts = F.fwd_partials(q.to(dev), k.to(dev), v.to(dev), idx.to(dev),
                                      scale=w.scale, num_splits=2)
    torch.cuda.synchronize()
    for i in range(2):
        _check(o_parts[i], l_parts[i], q, k, v, idx[:, :, 300 * i:300 * (i + 1)].contiguous(),
               w.scale)


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
def test_split_workspace_contents_do_not_matter(F, hd, fill):
    """Whatever the split-KV workspace held before (zero bytes, all-one bytes,
    random bytes, or what a previous call left), the result is the same."""
    w = W.make_custom(B=4, T=1, n_h=128, hd=hd, s_k=700, out_dtype="bf16", num_splits=6,
                      seed=hd + len(fill))
    q, k, v, idx = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ws = torch.empty(F.workspace_bytes(w.B, w.T, w.n_h, w.hd, w.num_splits), dtype=torch.uint8,
                     device=dev)
    if fill == "zeros":
        ws.zero_()
    elif fill == "ones":
        ws.fill_(0xFF)
    else:
        g = torch.Generator().manual_seed(hd)
        ws.copy_(torch.randint(0, 256, ws.shape, generator=g, dtype=torch.uint8))
    o1, l1 = F.fwd(qd, kd, vd, scale=w.scale, out_dtype=torch.bfloat16, num_splits=6, workspace=ws)
    o2, l2 = F.fwd(qd, kd, vd, scale=w.scale, out_dtype=torch.bfloat16, num_splits=6, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _check(o1, l1, q, k, v, None, w.scale)


@pytest.mark.parametrize("n_h,T", [(1, 1), (37, 1), (100, 1), (65, 3)])
@pytest.mark.parametrize("splits", [2, 5])
def test_split_row_tiles_ragged(F, n_h, T, splits):
    """Split-KV groups whose row count is not a multiple of a workgroup's row
    tile (one row, part of one tile, one and a half tiles; dense groups of
    T*n_h rows)."""
    w = W.make_custom(B=3, T=T, n_h=n_h, hd=256, s_k=333, out_dtype="f32", num_splits=splits,
                      seed=n_h * 10 + T + splits)
    _case(F, w)


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_split_gather_masks_invalid_entries(F, hd):
    """Gathered split-KV: invalid entries (-1, pool_rows, INT32_MAX) inside
    splits, a split whose entries are all invalid and a token with one valid
    entry give attention over the valid entries alone."""
    P, s_k = 2000, 300
    w = W.make_custom(B=1, T=3, n_h=64, hd=hd, s_k=s_k, pool=P, out_dtype="f32", num_splits=4,
                      seed=91 + hd)
    q, k, v, idx = W.make_inputs(w)
    bad = idx.clone()
    bad[0, 0, 3] = -1
    bad[0, 0, 80:95] = P
    bad[0, 0, 150:225] = 2 ** 31 - 1      # the whole third split (75 keys each)
    bad[0, 1, ::7] = -5
    bad[0, 2, :] = -1
    bad[0, 2, 260] = idx[0, 2, 260]
    out, lse = _run(F, q, k, v, bad, w.scale, torch.float32, 4)
    for t in range(3):
        ok = [int(bad[0, t, j]) for j in range(s_k) if 0 <= int(bad[0, t, j]) < P]
        sub = torch.tensor([[ok]], dtype=torch.int32)
        _check(out[:, t:t + 1], lse[:, t:t + 1], q[:, t:t + 1], k, v, sub, w.scale)


def test_split_kv_replays_in_a_hip_graph(F):
    """The split-KV forward (split kernel + merge kernel) captured in a HIP
    graph: every replay, with the program's own eager work and
    synchronisations between replays, gives the eager result bit for bit."""
    w = W.make_custom(B=8, T=1, n_h=128, hd=256, s_k=1024, out_dtype="bf16", num_splits=8,
                      seed=77)
    q, k, v, _ = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    plan = F.FwdPlan(qd, kd, vd, scale=w.scale, out_dtype=torch.bfloat16, num_splits=8,
                     stream=side)
    with torch.cuda.stream(side):
        ref_out, ref_lse = (t.clone() for t in plan())
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        plan()
    for i in range(4):
        plan.out.fill_(float("nan"))
        plan.lse.fill_(float("nan"))
        x = torch.randn(1 << 20, device=dev) * (i + 1)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.out, ref_out) and torch.equal(plan.lse, ref_lse), i
        del x
    _check(ref_out, ref_lse, q, k, v, None, w.scale)


@pytest.mark.parametrize("hd,pool", [(128, 0), (512, 0), (128, 300), (512, 300)])
def test_split_with_empty_trailing_chunks(F, hd, pool):
    # 9 keys in 8 chunks of 2: chunks 5..7 are empty (lse -inf) and must vanish
    w = W.make_custom(B=2, T=1, n_h=16, hd=hd, s_k=9, pool=pool, out_dtype="f32", num_splits=8,
                      seed=9 + hd + pool)
    _case(F, w)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("n_h", [1, 16, 128, 200])
def test_gather(F, hd, n_h):
    w = W.make_custom(B=2, T=5, n_h=n_h, hd=hd, s_k=333, pool=4096, out_dtype="bf16",
                      seed=hd + n_h)
    _case(F, w)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("s_k,splits", [(1024, 1), (1025, 1), (1500, 1), (1500, 2)])
def test_gather_list_lengths_around_the_staged_limit(F, hd, s_k, splits):
    """A split of up to 1024 gathered keys runs a kernel that stages its
    index list in LDS; longer splits run the streaming kernel's gather form."""
    w = W.make_custom(B=1, T=3, n_h=128, hd=hd, s_k=s_k, pool=4096, out_dtype="bf16",
                      num_splits=splits, seed=s_k + splits + hd)
    _case(F, w)


def test_gather_split(F):
    w = W.make_custom(B=2, T=3, n_h=128, hd=128, s_k=1024, pool=8192, out_dtype="bf16",
                      num_splits=4, seed=5)
    _case(F, w)


def test_gather_sorted_and_shuffled_indices_agree(F):
    w = W.make_custom(B=1, T=4, n_h=64, hd=128, s_k=500, pool=2048, out_dtype="f32", seed=3)
    q, k, v, idx = W.make_inputs(w)
    o1, l1 = _run(F, q, k, v, idx, w.scale, torch.float32, 1)
    srt = torch.sort(idx, dim=-1).values.contiguous()
    o2, l2 = _run(F, q, k, v, srt, w.scale, torch.float32, 1)
    _check(o2, l2, q, k, v, srt, w.scale)
    assert (o1 - o2).abs().max().item() < 1e-3


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
def test_gather_out_of_range_indices_are_masked(F, hd):
    """Entries outside [0, pool_rows) are never read and contribute nothing: the
    result equals attention over the valid entries only."""
    w = W.make_custom(B=1, T=3, n_h=32, hd=hd, s_k=200, pool=1000, out_dtype="f32", seed=17)
    q, k, v, idx = W.make_inputs(w)
    bad = idx.clone()
    bad[0, 0, 5] = -1
    bad[0, 1, 100:150] = 1000
    bad[0, 2, :] = 2 ** 31 - 1   # every entry of token 2 invalid: empty rows
    out, lse = _run(F, q, k, v, bad, w.scale, torch.float32, 1)
    # token 0 and 1: oracle on the valid subset
    for t, keep in [(0, [j for j in range(200) if j != 5]),
                    (1, [j for j in range(200) if not 100 <= j < 150])]:
        sub = bad[:, t:t + 1, keep].contiguous()
        _check(out[:, t:t + 1], lse[:, t:t + 1], q[:, t:t + 1], k, v, sub, w.scale)
    assert torch.all(out[0, 2] == 0) and torch.all(torch.isneginf(lse[0, 2]))


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
def test_long_split_gather_masks_invalid_entries(F, hd):
    """A split of more than 1024 gathered keys runs the streaming kernel's
    gather form, which fetches its index entries tile by tile: entries -1,
    pool_rows, 2^31-1 and INT32_MIN in middle tiles, a whole invalid tile
    (keys 640..703, a full 32- and 64-key tile) and a token whose entries are
    all invalid but one must give attention over the valid entries alone."""
    P, s_k = 4096, 1500
    w = W.make_custom(B=1, T=3, n_h=64, hd=hd, s_k=s_k, pool=P, out_dtype="f32", seed=71 + hd)
    q, k, v, idx = W.make_inputs(w)
    bad = idx.clone()
    bad[0, 0, 100] = -1
    bad[0, 0, 101] = P
    bad[0, 0, 333:340] = 2 ** 31 - 1
    bad[0, 0, 640:704] = -2 ** 31          # one whole tile of either key width
    bad[0, 0, 1499] = P + 17               # the last key of the split
    bad[0, 1, 500:1200:3] = -7             # scattered through many tiles
    bad[0, 2, :] = -1
    bad[0, 2, 777] = idx[0, 2, 777]        # a single valid key
    out, lse = _run(F, q, k, v, bad, w.scale, torch.float32, 1)
    for t in range(3):
        ok = [(j, int(bad[0, t, j])) for j in range(s_k) if 0 <= int(bad[0, t, j]) < P]
        sub = torch.tensor([[[e for _, e in ok]]], dtype=torch.int32)
        _check(out[:, t:t + 1], lse[:, t:t + 1], q[:, t:t + 1], k, v, sub, w.scale)
    row = v[int(idx[0, 2, 777])].float()
    assert torch.allclose(out[0, 2].cpu(), row.expand(64, -1), atol=1e-5)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
def test_region_ordered_gather_masks_invalid_entries(F, hd):
    """Lists of 8 tiles or more are walked in pool-region order (the result
    does not depend on the key order): invalid entries spread over every
    region of the list, a whole invalid tile's worth (keys 320..383), repeated
    rows, and a token with a single valid entry must still give attention over
    the valid entries alone, each counted as often as it is listed."""
    P, s_k = 30000, 1000
    w = W.make_custom(B=1, T=3, n_h=48, hd=hd, s_k=s_k, pool=P, out_dtype="f32", seed=91 + hd)
    q, k, v, idx = W.make_inputs(w)
    bad = idx.clone()
    bad[0, 0, 3:1000:37] = -1
    bad[0, 0, 320:384] = P
    bad[0, 0, 500:520] = bad[0, 0, 600:620]    # repeated rows
    bad[0, 0, 999] = 2 ** 31 - 1
    bad[0, 1, ::2] = -2 ** 31                  # half the list, every other key
    bad[0, 2, :] = P + 5
    bad[0, 2, 431] = idx[0, 2, 431]            # a single valid key
    out, lse = _run(F, q, k, v, bad, w.scale, torch.float32, 1)
    for t in range(3):
        ok = [int(bad[0, t, j]) for j in range(s_k) if 0 <= int(bad[0, t, j]) < P]
        sub = torch.tensor([[ok]], dtype=torch.int32)
        _check(out[:, t:t + 1], lse[:, t:t + 1], q[:, t:t + 1], k, v, sub, w.scale)
    row = v[int(idx[0, 2, 431])].float()
    assert torch.allclose(out[0, 2].cpu(), row.expand(48, -1), atol=1e-5)


@pytest.mark.parametrize("hd,P", [(64, 1 << 20), (128, 1), (512, 3)])
def test_region_ordered_gather_pool_extremes(F, hd, P):
    """Region classes come from the pool's size (row >> shift, 32 regions):
    a 2^20-row pool (shift 15) with its first and last rows listed, and pools
    of 1 and 3 rows (shift 0, every key a repeat), all through lists long
    enough to be ordered."""
    s_k = 700
    w = W.make_custom(B=1, T=2, n_h=16, hd=hd, s_k=s_k, pool=4096, out_dtype="f32",
                      seed=77 + hd)
    q, k, v, _ = W.make_inputs(w)
    g = torch.Generator().manual_seed(78 + hd)
    if P > 4096:
        k = torch.randn(P, hd, generator=g).to(torch.bfloat16)
        v = torch.randn(P, hd, generator=g).to(torch.bfloat16)
    else:
        k, v = k[:P].contiguous(), v[:P].contiguous()
    idx = torch.randint(0, P, (1, 2, s_k), generator=g, dtype=torch.int32)
    idx[0, 0, 3] = 0
    idx[0, 0, 500] = P - 1
    idx[0, 1, 17] = -1
    out, lse = _run(F, q, k, v, idx, w.scale, torch.float32, 1)
    for t in range(2):
        ok = [int(e) for e in idx[0, t].tolist() if 0 <= int(e) < P]
        sub = torch.tensor([[ok]], dtype=torch.int32)
        _check(out[:, t:t + 1], lse[:, t:t + 1], q[:, t:t + 1], k, v, sub, w.scale)


@pytest.mark.parametrize("hd,s_k", [(128, 1024), (256, 160), (512, 512), (512, 1024)])
def test_region_ordered_gather_runs_are_bitwise_identical(F, hd, s_k):
    """The region order is a stable counting sort (no atomics): repeated calls
    give the same bits."""
    w = W.make_custom(B=2, T=4, n_h=64, hd=hd, s_k=s_k, pool=32768, out_dtype="bf16",
                      seed=5 + hd)
    q, k, v, idx = W.make_inputs(w)
    o1, l1 = _run(F, q, k, v, idx, w.scale, torch.bfloat16, 1)
    for _ in range(2):
        o2, l2 = _run(F, q, k, v, idx, w.scale, torch.bfloat16, 1)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _check(o1, l1, q, k, v, idx, w.scale)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("splits", [1, 3])
def test_gather_repeated_indices_count_each_time(F, splits, hd):
    """A pool row listed several times is several keys (each takes its own
    softmax weight), as in the oracle's definition; a list of one repeated
    row gives that row's V exactly."""
    w = W.make_custom(B=1, T=3, n_h=64, hd=hd, s_k=256, pool=512, out_dtype="f32", seed=23)
    q, k, v, idx = W.make_inputs(w)
    rep = idx.clone()
    rep[0, 0, 128:] = rep[0, 0, :128]        # every row twice
    rep[0, 1, ::2] = 7                       # row 7 on half the keys
    rep[0, 2, :] = 11                        # one row only
    out, lse = _run(F, q, k, v, rep, w.scale, torch.float32, splits)
    _check(out, lse, q, k, v, rep, w.scale)
    row = v[11].float()
    assert torch.allclose(out[0, 2].cpu(), row.expand(64, -1), atol=1e-5)


@pytest.mark.parametrize("hd,gather", [(64, False), (128, False), (256, False), (512, False),
                                       (128, True), (256, True), (512, True)])
def test_bf16_output_is_the_fp32_output_rounded_to_nearest_even(F, hd, gather):
    """The bf16 epilogue rounds the same fp32 values the fp32 epilogue stores,
    to nearest-even (torch's fp32 -> bf16 conversion is round-to-nearest-even)."""
    w = W.make_custom(B=2, T=3, n_h=64, hd=hd, s_k=300, pool=2048 if gather else 0,
                      out_dtype="f32", seed=31 + hd)
    q, k, v, idx = W.make_inputs(w)
    o32, l32 = _run(F, q, k, v, idx, w.scale, torch.float32, 1)
    o16, l16 = _run(F, q, k, v, idx, w.scale, torch.bfloat16, 1)
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32)


def test_merge_bf16_output_is_its_fp32_output_rounded_to_nearest_even(F):
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(41)
    parts = torch.randn(5, 300, 128, generator=g).to(dev)
    lses = (torch.randn(5, 300, generator=g) * 3).to(dev)
    o32, l32 = F.lse_merge(parts, lses, torch.float32)
    o16, l16 = F.lse_merge(parts, lses, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32)


# ---------------------------------------------------- structure / adversarial
def test_structured_inputs_catch_layout_swaps(F):
    """Distinct, smooth values per (key, d) and per head: any swapped axis or
    wrong key<->value pairing shows up far above the tolerance."""
    B, T, n_h, hd, s_k = 1, 2, 64, 128, 384
    j = torch.arange(s_k, dtype=torch.float32)[:, None]
    d = torch.arange(hd, dtype=torch.float32)[None, :]
    v = torch.sin(0.37 * j + 0.11 * d * d / hd + 0.5 * d).to(torch.bfloat16)[None]
    k = (torch.cos(0.05 * j * (1 + d / hd)) * (1 + d / hd)).to(torch.bfloat16)[None]
    h = torch.arange(n_h, dtype=torch.float32)[:, None]
    q = torch.stack([torch.sin(0.3 * h + 0.07 * d * (t + 1)) * 3 for t in range(T)])
    q = q.to(torch.bfloat16)[None]
    scale = 1 / math.sqrt(hd)
    out, lse = _run(F, q, k, v, None, scale, torch.float32, 1)
    _check(out, lse, q, k, v, None, scale)


@pytest.mark.parametrize("splits", [1, 4])
def test_logits_growing_tile_after_tile(F, splits):
    """Row maxima rise in every KV tile (the O rescale runs at each tile), and
    the last key dominates."""
    B, T, n_h, hd, s_k = 1, 1, 128, 128, 1024
    g = torch.Generator().manual_seed(1)
    u = torch.randn(hd, generator=g)
    a = torch.linspace(0.0, 3.0, s_k)
    noise = 0.1 * torch.randn(s_k, hd, generator=g)
    k = (a[:, None] * u[None, :] + noise)
    k[-1] = 6.0 * u
    q = (u[None, :] + 0.2 * torch.randn(n_h, hd, generator=g)).reshape(1, 1, n_h, hd)
    v = torch.randn(1, s_k, hd, generator=g)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k[None], v))
    scale = 1 / math.sqrt(hd)
    out, lse = _run(F, q, k, v, None, scale, torch.float32, splits)
    _check(out, lse, q, k, v, None, scale)


def test_large_magnitude_logits_stay_finite(F):
    """q, k ~ N(0, 8^2): logits of a few hundred, softmax nearly one-hot; the
    max-shifted exponentials must neither overflow nor lose the row."""
    w = W.make_custom(B=1, T=4, n_h=64, hd=128, s_k=512, out_dtype="f32", seed=8)
    q, k, v, _ = W.make_inputs(w)
    q = (q.float() * 8).to(torch.bfloat16)
    k = (k.float() * 8).to(torch.bfloat16)
    out, lse = _run(F, q, k, v, None, w.scale, torch.float32, 1)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    assert lse.abs().max().item() > 100
    _check(out, lse, q, k, v, None, w.scale)


@pytest.mark.parametrize("splits,gather", [(1, False), (4, False), (1, True)])
def test_large_values_error_bounded_by_the_p_rounding(F, splits, gather):
    """V ~ N(0, 1000^2), fp32 out: the absolute bar has no meaning at this
    scale, so the bound is the one the bf16 P operand implies.  Each weight
    is rounded once, p~ = p (1 + e) with |e| <= 2^-8, so |O - O_ref| <=
    2^-8 * sum p |v| / sum p per element (plus fp32 accumulation); the oracle
    gives that weighted mean of |v| as attention over |v|.  The merge of split
    parts keeps the bound (its weights sum to one).  Per-row cosine and lse
    keep the usual bar."""
    w = W.make_custom(B=2, T=3, n_h=40, hd=128, s_k=700, out_dtype="f32", num_splits=splits,
                      pool=2048 if gather else 0, seed=31 + splits + 10 * gather)
    q, k, v, idx = W.make_inputs(w)
    v = (v.float() * 1000).to(torch.bfloat16)
    out, lse = _run(F, q, k, v, idx, w.scale, torch.float32, splits)
    O_ref, L_ref = oracle.attention(q, k, v, w.scale, kv_idx=idx)
    A_ref, _ = oracle.attention(q, k, v.float().abs().to(torch.bfloat16), w.scale, kv_idx=idx)
    o = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(o - O_ref)
    bound = (2.0 ** -8 + 1e-4) * A_ref + 1e-6   # 1e-4: fp32 sums over 700 keys
    assert np.all(err <= bound), float((err / bound).max())
    m = oracle.row_metrics(o.reshape(-1, 128), O_ref.reshape(-1, 128), lse.cpu().numpy().ravel(),
                           L_ref.ravel())
    assert m["min_row_cos"] >= MIN_COS and m["lse_err"] <= LSE_ERR, m
    say(f"[parity] |V|~1000 splits={splits} gather={gather}: max err/bound "
        f"{float((err / bound).max()):.3f}, max_abs {m['max_abs']:.3e}")


def test_single_key_returns_that_value_row(F):
    """s_k = 1: O = V_0.  The kernel folds scale*log2(e) into an FMA, so the
    lone weight is 1 within fp32 rounding, not bit-exactly."""
    w = W.make_custom(B=2, T=3, n_h=50, hd=128, s_k=1, out_dtype="f32", seed=1)
    q, k, v, _ = W.make_inputs(w)
    out, lse = _run(F, q, k, v, None, w.scale, torch.float32, 1)
    ref = v.float()[:, None, None, 0, :].expand(out.shape)
    torch.testing.assert_close(out.cpu(), ref, rtol=1e-6, atol=0)
    _check(out, lse, q, k, v, None, w.scale)


def test_zero_keys_gives_empty_rows(F):
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 4, 64).to(torch.bfloat16).to(dev)
    k = torch.empty(1, 0, 64, dtype=torch.bfloat16, device=dev)
    out, lse = F.fwd(q, k, k.clone(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_repeat_runs_are_bitwise_identical(F):
    w = W.make_custom(B=2, T=16, n_h=64, hd=128, s_k=1024, out_dtype="bf16", num_splits=2, seed=2)
    q, k, v, idx = W.make_inputs(w)
    o1, l1 = _run(F, q, k, v, idx, w.scale, torch.bfloat16, 2)
    o2, l2 = _run(F, q, k, v, idx, w.scale, torch.bfloat16, 2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_runs_on_a_side_stream(F):
    w = W.make_custom(B=1, T=8, n_h=64, hd=128, s_k=256, out_dtype="f32", seed=6)
    q, k, v, _ = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out, lse = F.fwd(qd, kd, vd, out_dtype=torch.float32)
    s.synchronize()
    _check(out, lse, q, k, v, None, w.scale)


def test_plan_relaunches_on_the_same_tensors(F):
    """FwdPlan (arguments marshalled once) matches fwd on every relaunch,
    also after its inputs change in place."""
    w = W.make_custom(B=2, T=4, n_h=64, hd=128, s_k=300, out_dtype="bf16", num_splits=3, seed=8)
    q, k, v, idx = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    plan = F.FwdPlan(qd, kd, vd, scale=w.scale, out_dtype=torch.bfloat16, num_splits=3)
    for _ in range(2):
        out, lse = plan()
        torch.cuda.synchronize()
        _check(out, lse, q, k, v, None, w.scale)
    v2 = (v.float() * -0.5).to(torch.bfloat16)
    vd.copy_(v2)
    out, lse = plan()
    torch.cuda.synchronize()
    _check(out, lse, q, k, v2, None, w.scale)


# ------------------------------------------------------------ head dim 512
# DeepSeek-V4's head dim (page "May 24, 2026 — Session Start Plan", File Map:
# config hd=512; Key Numbers: Flash n_h 64 / top_k 512, Pro n_h 128 / top_k 1024).
def test_hd512_pro_decode_split(F):
    w = W.make_custom(B=4, T=1, n_h=128, hd=512, s_k=1024, out_dtype="bf16", num_splits=8,
                      seed=512)
    _case(F, w)


def test_hd512_flash_sparse_topk(F):
    w = W.make_custom(B=2, T=16, n_h=64, hd=512, s_k=512, pool=8192, out_dtype="bf16", seed=513)
    _case(F, w)


@pytest.mark.parametrize("splits", [4, 8])
def test_hd512_decode_benchmarked_size_all_rows(F, splits):
    """The hd 512 decode row at full size: B=32, 128 heads, s_k=1024, bf16
    out, every row; bench.py times it with 4 splits (one 256-workgroup launch
    whose two 64-row tiles of a split share an XCD), 8 is the split count of
    the hd 256 decode config."""
    w = W.make_custom(B=32, T=1, n_h=128, hd=512, s_k=1024, out_dtype="bf16",
                      num_splits=splits, seed=515 + splits)
    _case(F, w)


def test_hd512_flash_topk_benchmarked_size_all_rows(F):
    """The hd 512 Flash top-k row as bench.py times it: B=4, T=512, 64 heads,
    top-k 512 of a 32768-row pool, bf16 out, every row."""
    w = W.make_custom(B=4, T=512, n_h=64, hd=512, s_k=512, pool=32768, out_dtype="bf16",
                      seed=516)
    _case(F, w)


@pytest.mark.parametrize("T,n_h,s_k,pool,out_dtype,plant", [
    (600, 64, 512, 4096, "bf16", False),   # 600 workgroups: more than one round on the chip
    (200, 100, 512, 2048, "bf16", False),  # two row tiles per token, the second of 36 rows
    (400, 64, 100, 1000, "f32", True),     # four tiles, the last partly past s_k; bad entries
    (300, 64, 1024, 8192, "bf16", False),  # 32 tiles per token
    (600, 64, 600, 4096, "f32", True),     # two workgroups per CU (long splits, 600 of them):
                                           # bad entries; its first tokens bit-equal to the
                                           # double-buffered kernel's small launch
])
def test_hd512_gather_many_tokens(F, T, n_h, s_k, pool, out_dtype, plant):
    """The head-dim-512 gather over more tokens than the chip runs at once:
    ragged heads, invalid and repeated entries, a last tile partly past s_k, 32
    tiles per token.  Every row against the oracle, and the first 200 row tiles
    bit-equal to a call over those tokens alone (a row's result does not depend
    on the size of the launch)."""
    w = W.make_custom(B=1, T=T, n_h=n_h, hd=512, s_k=s_k, pool=pool, out_dtype=out_dtype,
                      seed=900 + T + s_k)
    q, k, v, idx = W.make_inputs(w)
    if plant:
        idx = idx.clone()
        idx[0, ::7, 3] = -1            # invalid entries: masked keys
        idx[0, ::5, 17] = pool         # one past the pool
        idx[0, ::9, 40] = pool + 1000
        idx[0, ::3, 50] = idx[0, ::3, 51]  # a row gathered twice
    dt = _dt(out_dtype)
    out, lse = _run(F, q, k, v, idx, w.scale, dt, 1)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    # tokens with invalid entries: attention over their valid entries alone
    bad_t = [t for t in range(T) if ((idx[0, t] < 0) | (idx[0, t] >= pool)).any()]
    for t in bad_t:
        ok = [int(j) for j in idx[0, t] if 0 <= int(j) < pool]
        sub = torch.tensor([[ok]], dtype=torch.int32)
        _check(out[:, t:t + 1], lse[:, t:t + 1], q[:, t:t + 1], k, v, sub, w.scale)
    good = sorted(set(range(T)) - set(bad_t))
    m = _check(out, lse, q, k, v, idx, w.scale,
               rows=None if not bad_t else [t * n_h + h for t in good for h in range(n_h)])
    t_small = 200 // ((n_h + 63) // 64)
    out2, lse2 = _run(F, q[:, :t_small].contiguous(), k, v, idx[:, :t_small].contiguous(),
                      w.scale, dt, 1)
    assert torch.equal(out[:, :t_small], out2)
    assert torch.equal(lse[:, :t_small], lse2)
    say(f"[parity] hd 512 gather {w.describe()}: max_abs {m['max_abs']:.3e} "
        f"min_row_cos {m['min_row_cos']:.7f} lse_err {m['lse_err']:.3e}; first {t_small} "
        f"tokens bit-equal to a call over them alone")


@pytest.mark.parametrize("s_k,splits", [(1024, 1), (1025, 1), (2000, 1), (2000, 2)])
def test_hd512_dense_key_counts_around_the_staged_limit(F, s_k, splits):
    """At head dim 512 a split of up to 1024 keys runs the kernel that stages
    its row offsets in LDS; longer splits run the streaming kernel."""
    w = W.make_custom(B=2, T=3, n_h=24, hd=512, s_k=s_k, out_dtype="bf16", num_splits=splits,
                      seed=s_k + 7 * splits)
    _case(F, w)


@pytest.mark.parametrize("splits,out_dtype", [(1, "f32"), (3, "f32"), (2, "bf16")])
def test_hd512_dense_prefill(F, splits, out_dtype):
    w = W.make_custom(B=1, T=40, n_h=8, hd=512, s_k=700, out_dtype=out_dtype, num_splits=splits,
                      seed=514 + splits)
    _case(F, w)


# --------------------------------------------------------------- the merge
@pytest.mark.parametrize("B,T,n_h,hd,pool,splits", [
    (8, 1, 128, 64, 0, 8), (16, 1, 128, 128, 0, 5), (8, 1, 128, 256, 0, 8),
    (8, 1, 128, 512, 0, 4), (8, 1, 256, 256, 0, 3), (2, 4, 64, 128, 1000, 4),
    (3, 1, 128, 256, 0, 8), (8, 1, 100, 128, 0, 6)])
def test_split_path_merge_equals_the_merge_of_its_partials(F, B, T, n_h, hd, pool, splits):
    """fmha_mqa_fwd with splits (fp32 out: fp32 partials) is, bit for bit, the
    public merge of fmha_mqa_fwd_partials' planes for the same call.  A multiple
    of 8 groups with at most 512 rows each takes the merge's XCD-following
    block order, the other cases its plain order; the arithmetic of a row is
    the same either way."""
    w = W.make_custom(B=B, T=T, n_h=n_h, hd=hd, s_k=700, pool=pool, out_dtype="f32",
                      num_splits=splits, seed=B * 31 + n_h + hd + splits)
    q, k, v, idx = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    idd = None if idx is None else idx.to(dev)
    out, lse = F.fwd(qd, kd, vd, idd, scale=w.scale, out_dtype=torch.float32, num_splits=splits)
    o_parts, l_parts = F.fwd_partials(qd, kd, vd, idd, scale=w.scale, num_splits=splits)
    rows = B * T * n_h
    o2, l2 = F.lse_merge(o_parts.view(splits, rows, hd), l_parts.view(splits, rows),
                         torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out.view(rows, hd), o2) and torch.equal(lse.view(rows), l2)
    _check(out, lse, q, k, v, idx, w.scale)


@pytest.mark.parametrize("hd,out_dtype", [(64, "f32"), (128, "bf16"), (256, "f32"), (20, "f32")])
def test_lse_merge_entry_point(F, hd, out_dtype):
    g = np.random.default_rng(hd)
    P, R = 5, 333
    o = (0.25 * g.standard_normal((P, R, hd))).astype(np.float32)  # |o| < 2: bf16 half-ulp < 1e-2
    lse = (g.standard_normal((P, R)) * 5).astype(np.float32)
    lse[2, ::7] = -np.inf
    o[2, ::7] = np.nan          # an empty part's O is never read
    lse[:, 10] = -np.inf        # a row whose parts are all empty
    dev = torch.device("cuda:0")
    out, L = F.lse_merge(torch.from_numpy(o).to(dev), torch.from_numpy(lse).to(dev),
                         out_dtype=_dt(out_dtype))
    torch.cuda.synchronize()
    Oref, Lref = oracle.lse_merge(np.where(np.isneginf(lse)[:, :, None], 0.0, o), lse)
    m = oracle.row_metrics(out.float().cpu().numpy(), Oref, L.cpu().numpy(), Lref)
    assert m["max_abs"] <= (1e-2 if out_dtype == "bf16" else 1e-5), m
    assert m["lse_err"] <= 1e-5, m
    assert torch.all(out[10] == 0) and torch.isneginf(L[10])


# ------------------------------------------------- measurement helper
@pytest.mark.parametrize("hd,s_k", [(128, 100), (512, 512), (64, 1500)])
def test_gather_floor_reads_every_gathered_row(F, hd, s_k):
    """fmha_gather_floor (the sparse config's gather-only floor) reads each
    listed K and V row once, lists of up to 1024 keys in region order and
    longer ones in list order: its per-token XOR of the words read equals the
    XOR computed on the CPU; masked entries read nothing."""
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(61 + s_k)
    P, B, T = 500, 2, 3
    k = torch.randn(P, hd, generator=g).to(torch.bfloat16)
    v = torch.randn(P, hd, generator=g).to(torch.bfloat16)
    idx = torch.randint(0, P, (B, T, s_k), generator=g, dtype=torch.int32)
    idx[0, 1, 7] = -1
    idx[1, 2, :10] = P + 3
    got = F.gather_floor(k.to(dev), v.to(dev), idx.to(dev)).cpu().numpy().view(np.uint32)
    kw = k.view(torch.int32).numpy().view(np.uint32)   # [P, hd/2] words
    vw = v.view(torch.int32).numpy().view(np.uint32)
    for b in range(B):
        for t in range(T):
            rows = idx[b, t].numpy()
            rows = rows[(rows >= 0) & (rows < P)]
            want = np.bitwise_xor.reduce(np.concatenate([kw[rows].ravel(), vw[rows].ravel()]))
            assert got[b, t] == want, (b, t)
