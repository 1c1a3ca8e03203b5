"""GPU parity of the attention sink (fmha_mqa_fwd_sink, fmha_attention_sink)
against the float64 oracle's sink (one extra logit per query head with a zero
value vector; the reading of the sink merge named on page "May 24, 2026 —
Session Start Plan").  Same bar as the plain forward."""
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


def _sinks(n_h, seed, shift=0.0):
    g = np.random.default_rng(seed)
    s = g.normal(shift, 2.0, n_h).astype(np.float32)
    s[0] = -np.inf
    if n_h > 2:
        s[2] = shift + 12.0  # a sink far above the row's logits
    return torch.from_numpy(s)


def _check(out, lse, q, k, v, idx, scale, sink):
    O_ref, L_ref = oracle.attention(q, k, v, scale, kv_idx=idx, sink=sink)
    hd = q.shape[-1]
    m = oracle.row_metrics(out.float().reshape(-1, hd).cpu().numpy(), O_ref.reshape(-1, hd),
                           lse.reshape(-1).cpu().numpy(), L_ref.reshape(-1))
    assert m["max_abs"] <= MAX_ABS, m
    assert m["min_row_cos"] >= MIN_COS, m
    assert m["lse_err"] <= LSE_ERR, m
    return m


def _dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


@pytest.mark.parametrize("hd,s_k,splits,out_dtype,gather", [
    (64, 200, 1, "f32", False),
    (128, 513, 1, "bf16", False),
    (256, 96, 1, "f32", False),
    (128, 300, 3, "bf16", False),    # whole-chunk split kernel + merge
    (128, 1024, 2, "f32", False),    # streaming split kernel + merge
    (128, 256, 1, "bf16", True),
    (64, 130, 2, "f32", True),
])
def test_fwd_sink_matches_oracle(F, hd, s_k, splits, out_dtype, gather):
    w = W.make_custom(B=2, T=3, n_h=8, hd=hd, s_k=s_k, out_dtype=out_dtype, num_splits=splits,
                      pool=4096 if gather else 0, seed=70 + hd + s_k)
    q, k, v, idx = W.make_inputs(w)
    sink = _sinks(8, s_k)
    qd, kd, vd, idd, sd = _dev(q, k, v, idx, sink)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out, lse = F.fwd(qd, kd, vd, idd, scale=w.scale, out_dtype=od, num_splits=splits, sink=sd)
    torch.cuda.synchronize()
    _check(out, lse, q, k, v, idx, w.scale, sink.double().numpy())


def test_sink_through_the_two_workgroup_hd512_gather(F):
    """Long gathered splits at hd 512 over enough tokens for two workgroups
    per CU run the single-stage kernel; the sink joins in its epilogue."""
    w = W.make_custom(B=1, T=600, n_h=8, hd=512, s_k=512, out_dtype="f32", pool=4096, seed=91)
    q, k, v, idx = W.make_inputs(w)
    sink = _sinks(8, w.s_k)
    qd, kd, vd, idd, sd = _dev(q, k, v, idx, sink)
    out, lse = F.fwd(qd, kd, vd, idd, scale=w.scale, out_dtype=torch.float32, num_splits=1,
                     sink=sd)
    torch.cuda.synchronize()
    _check(out, lse, q, k, v, idx, w.scale, sink.double().numpy())


@pytest.mark.parametrize("splits", [1, 4])
def test_minus_inf_sinks_change_nothing(F, splits):
    w = W.make_custom(B=1, T=4, n_h=16, hd=128, s_k=384, out_dtype="bf16", num_splits=splits,
                      seed=77)
    q, k, v, _ = W.make_inputs(w)
    qd, kd, vd = _dev(q, k, v)
    o0, l0 = F.fwd(qd, kd, vd, scale=w.scale, out_dtype=torch.bfloat16, num_splits=splits)
    none = torch.full((16,), float("-inf"), device=DEV)
    o1, l1 = F.fwd(qd, kd, vd, scale=w.scale, out_dtype=torch.bfloat16, num_splits=splits,
                   sink=none)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_in_place_sink_on_finished_rows(F, out_dtype):
    w = W.make_custom(B=2, T=5, n_h=8, hd=128, s_k=640, out_dtype=out_dtype, seed=78)
    q, k, v, _ = W.make_inputs(w)
    sink = _sinks(8, 5, shift=1.0)
    qd, kd, vd, sd = _dev(q, k, v, sink)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out, lse = F.fwd(qd, kd, vd, scale=w.scale, out_dtype=od)
    F.apply_sink(out, lse, sd)
    torch.cuda.synchronize()
    _check(out, lse, q, k, v, None, w.scale, sink.double().numpy())


def test_sink_on_rows_without_keys(F):
    q = torch.randn(1, 2, 4, 64).to(torch.bfloat16)
    k = torch.zeros(1, 0, 64, dtype=torch.bfloat16)
    sink = torch.tensor([0.5, float("-inf"), -3.0, 7.0])
    qd, kd, sd = _dev(q, k, sink)
    out, lse = F.fwd(qd, kd, kd.clone(), out_dtype=torch.float32, sink=sd)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    assert torch.equal(lse.cpu(), sink.expand(1, 2, 4))
