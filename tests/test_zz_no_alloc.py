"""fmha_mqa_fwd_noalloc: the forward whose split-KV partials live in the
library's static per-GPU scratch buffer.  Called through the C ABI and checked
against fmha_mqa_fwd (same kernels, caller workspace) and the float64 oracle,
on consecutive calls that reuse the buffer with different sizes."""
import pytest
import torch

import oracle
import workloads as W
from conftest import say

pytestmark = pytest.mark.gpu

MAX_ABS, MIN_COS, LSE_ERR = 1e-2, 0.9999, 1e-3
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def F():
    import fmha_mqa_fwd_amd
    return fmha_mqa_fwd_amd


def _both(F, w):
    q, k, v, idx = W.make_inputs(w)
    dt = torch.float32 if w.out_dtype == "f32" else torch.bfloat16
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    idd = None if idx is None else idx.to(DEV)
    ref_out, ref_lse = F.fwd(qd, kd, vd, idd, scale=w.scale, out_dtype=dt,
                             num_splits=w.num_splits)
    out = torch.full((w.B, w.T, w.n_h, w.hd), float("nan"), dtype=dt, device=DEV)
    lse = torch.full((w.B, w.T, w.n_h), float("nan"), dtype=torch.float32, device=DEV)
    F.fwd_noalloc(qd, kd, vd, out, lse, kv_idx=idd, scale=w.scale, num_splits=w.num_splits)
    torch.cuda.synchronize()
    return (q, k, v, idx), (out, lse), (ref_out, ref_lse)


def _check_oracle(inp, out, lse, w):
    q, k, v, idx = inp
    O, L = oracle.attention(q, k, v, w.scale, kv_idx=idx)
    m = oracle.row_metrics(out.float().cpu().numpy(), O, lse.cpu().numpy(), L)
    say(f"[no-alloc] {w.describe()}: {m}")
    assert m["max_abs"] <= MAX_ABS and m["min_row_cos"] >= MIN_COS and m["lse_err"] <= LSE_ERR, m


def test_two_calls_in_a_row_the_second_smaller(F):
    """The decode workload (32.1 MiB of partials in the scratch buffer), then a
    smaller gather problem with a different split count and fp32 output: each
    equals fmha_mqa_fwd's result bit for bit and the oracle within the bar."""
    for w in (W.get(3),
              W.make_custom(B=2, T=3, n_h=40, hd=128, s_k=700, pool=3000, out_dtype="f32",
                            num_splits=3, seed=808)):
        inp, (out, lse), (ref_out, ref_lse) = _both(F, w)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), w.describe()
        _check_oracle(inp, out, lse, w)


def test_unsplit_call_needs_no_scratch(F):
    w = W.make_custom(B=1, T=5, n_h=64, hd=64, s_k=300, out_dtype="bf16", seed=809)
    inp, (out, lse), (ref_out, ref_lse) = _both(F, w)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    _check_oracle(inp, out, lse, w)


def test_partials_beyond_the_buffer_are_rejected_before_any_launch(F):
    """4096 rows at hd 256 with 16 splits need 64.25 MiB > 64 MiB: status
    FMHA_ERR_SCRATCH_LIMIT, and the outputs are left untouched."""
    B, n_h, hd, s_k = 32, 128, 256, 1024
    assert F.workspace_bytes(B, 1, n_h, hd, 16) > F.SCRATCH_BYTES >= F.workspace_bytes(
        B, 1, n_h, hd, 15)
    q = torch.zeros(B, 1, n_h, hd, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(B, s_k, hd, dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, 1, n_h, hd), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, 1, n_h), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(F.FmhaError) as e:
        F.fwd_noalloc(q, k, k, out, lse, num_splits=16)
    assert e.value.status == F.FMHA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
    # 15 splits fit, and run
    F.fwd_noalloc(q, k, k, out, lse, num_splits=15)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.allclose(lse, torch.full_like(lse, float(torch.log(
        torch.tensor(float(s_k))))))
