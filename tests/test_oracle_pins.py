"""Pins for the float64 oracle: each check ties it to something other than
itself — brute force, closed forms, library routines, invariants.

The pages print no worked numeric example for attention, so no pin here is a
value taken from them; the closed forms below follow from the definition of
softmax attention and of the merge formula (page "CURRENT ISSUE: UMMA FMHA —
Full Pipeline + Production", "Next steps" item 4).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import workloads as W

TOL = 1e-12


def _rand(shape, rng, scale=1.0):
    # bf16-representable values, like every real input
    x = torch.from_numpy(rng.standard_normal(shape) * scale).to(torch.bfloat16)
    return oracle.to_f64(x)


def _tolist(a):
    return np.asarray(a).tolist()


# ------------------------------------------------------- the input conversion
def _decode_bf16(bits: int) -> float:
    """bf16 value of a 16-bit pattern from its fields (IEEE-754 binary16-brain:
    1 sign, 8 exponent bits with bias 127, 7 fraction bits), with no library
    conversion involved."""
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -133)          # subnormal: f * 2^(1 - 127 - 7)
    return sign * math.ldexp(128 + f, e - 134)     # (1 + f/128) * 2^(e - 127)


def test_to_f64_is_the_exact_bf16_value():
    """The oracle reads bf16 inputs through to_f64; every pattern class —
    signed zeros, subnormals, the smallest normal, the largest finite value,
    infinities and ordinary values — must arrive as its exact value."""
    named = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x4049,
             0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x3C00, 0x4780]
    rng = np.random.default_rng(11)
    finite = [int(b) for b in rng.integers(0, 1 << 16, 4000) if ((int(b) >> 7) & 0xFF) != 0xFF]
    pats = named + finite
    t = torch.tensor([b - (1 << 16) if b >= 1 << 15 else b for b in pats],
                     dtype=torch.int16).view(torch.bfloat16)
    got = oracle.to_f64(t)
    assert got.dtype == np.float64
    want = [_decode_bf16(b) for b in pats]
    for b, g_, w in zip(pats, got.tolist(), want):
        assert g_ == w, hex(b)
        assert math.copysign(1.0, g_) == math.copysign(1.0, w), hex(b)  # -0 stays -0
    assert got[named.index(0x0001)] == 2.0 ** -133
    assert got[named.index(0x7F7F)] == (2 - 2 ** -7) * 2.0 ** 127
    # integer index lists keep their exact values, as an integer dtype
    idx = torch.tensor([0, 1, 32767, -1, 2 ** 31 - 1, -2 ** 31], dtype=torch.int32)
    gi = oracle.to_f64(idx)
    assert gi.dtype.kind == "i" and gi.tolist() == [0, 1, 32767, -1, 2 ** 31 - 1, -2 ** 31]
    # fp32 inputs (sinks) arrive exactly too
    f = torch.tensor([1.0 / 3.0, -2.5e-40, 3.0e38], dtype=torch.float32)
    assert oracle.to_f64(f).tolist() == [float(np.float32(x)) for x in (1.0 / 3.0, -2.5e-40,
                                                                        3.0e38)]


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("B,T,n_h,s_k,hd", [
    (1, 1, 1, 1, 1), (1, 2, 3, 2, 3), (2, 3, 2, 5, 8), (3, 1, 2, 9, 3),
    (2, 2, 1, 7, 4)])
def test_dense_matches_brute_force(B, T, n_h, s_k, hd):
    rng = np.random.default_rng(B * 100 + T * 10 + s_k)
    q = _rand((B, T, n_h, hd), rng)
    k = _rand((B, s_k, hd), rng)
    v = _rand((B, s_k, hd), rng)
    scale = 1.0 / math.sqrt(hd)
    O, L = oracle.attention(q, k, v, scale)
    Ob, Lb = brute.brute_attention(_tolist(q), _tolist(k), _tolist(v), scale)
    np.testing.assert_allclose(O, np.array(Ob), atol=TOL, rtol=0)
    np.testing.assert_allclose(L, np.array(Lb), atol=TOL, rtol=0)


@pytest.mark.parametrize("B,T,n_h,s_k,hd,P", [
    (1, 1, 1, 1, 2, 3), (2, 3, 2, 4, 3, 11), (2, 2, 3, 9, 8, 16)])
def test_gather_matches_brute_force(B, T, n_h, s_k, hd, P):
    rng = np.random.default_rng(7 + P)
    q = _rand((B, T, n_h, hd), rng)
    k = _rand((P, hd), rng)
    v = _rand((P, hd), rng)
    idx = np.stack([rng.permutation(P)[:s_k] for _ in range(B * T)]).reshape(B, T, s_k)
    scale = 0.37
    O, L = oracle.attention(q, k, v, scale, kv_idx=idx)
    Ob, Lb = brute.brute_attention(_tolist(q), _tolist(k), _tolist(v), scale,
                                   kv_idx=_tolist(idx))
    np.testing.assert_allclose(O, np.array(Ob), atol=TOL, rtol=0)
    np.testing.assert_allclose(L, np.array(Lb), atol=TOL, rtol=0)


def test_merge_matches_brute_force():
    rng = np.random.default_rng(3)
    P, R, hd = 5, 7, 3
    o = rng.standard_normal((P, R, hd))
    lse = rng.standard_normal((P, R)) * 4
    lse[1, 2] = -np.inf
    lse[:, 4] = -np.inf          # a row whose parts are all empty
    O, L = oracle.lse_merge(o, lse)
    Ob, Lb = brute.brute_merge(o.tolist(), lse.tolist())
    np.testing.assert_allclose(O, np.array(Ob), atol=TOL, rtol=0)
    assert L[4] == -np.inf and np.all(O[4] == 0)
    fin = np.isfinite(L)
    np.testing.assert_allclose(L[fin], np.array(Lb)[fin], atol=TOL, rtol=0)


# --------------------------------------------------------- library routines
@pytest.mark.parametrize("B,T,n_h,s_k,hd", [(2, 5, 3, 37, 16), (1, 17, 4, 130, 64)])
def test_dense_matches_torch_sdpa_fp64(B, T, n_h, s_k, hd):
    """torch's own scaled_dot_product_attention (math path, float64, CPU) and
    torch.logsumexp are an independent implementation of the same definition."""
    rng = np.random.default_rng(11)
    q = _rand((B, T, n_h, hd), rng)
    k = _rand((B, s_k, hd), rng)
    v = _rand((B, s_k, hd), rng)
    scale = 1.0 / math.sqrt(hd)
    O, L = oracle.attention(q, k, v, scale)
    qt = torch.from_numpy(q).reshape(B, 1, T * n_h, hd)
    kt = torch.from_numpy(k).reshape(B, 1, s_k, hd)
    vt = torch.from_numpy(v).reshape(B, 1, s_k, hd)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    np.testing.assert_allclose(O.reshape(B, 1, T * n_h, hd), ref.numpy(), atol=1e-12, rtol=0)
    logits = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    lse_ref = torch.logsumexp(logits, dim=-1).reshape(B, T, n_h)
    np.testing.assert_allclose(L, lse_ref.numpy(), atol=1e-12, rtol=0)


def test_probs_match_scipy_softmax():
    from scipy.special import softmax
    rng = np.random.default_rng(5)
    q = _rand((6, 8), rng)
    k = _rand((13, 8), rng)
    p = oracle.attention_probs(q, k, 0.25)
    np.testing.assert_allclose(p, softmax(0.25 * (q @ k.T), axis=1), atol=1e-14, rtol=0)


# --------------------------------------------------------------- closed forms
def test_single_key_gives_that_value_row():
    """s_k = 1: p = 1, so O = V_0 exactly and lse = scale * q.k_0."""
    rng = np.random.default_rng(1)
    q = _rand((2, 3, 4, 8), rng)
    k = _rand((2, 1, 8), rng)
    v = _rand((2, 1, 8), rng)
    O, L = oracle.attention(q, k, v, 0.3)
    for b in range(2):
        np.testing.assert_array_equal(O[b], np.broadcast_to(v[b, 0], O[b].shape))
        np.testing.assert_allclose(L[b], 0.3 * (q[b] @ k[b, 0]), atol=1e-14, rtol=0)


def test_uniform_v_gives_v():
    """All V rows equal v: O = v for any q, k (softmax weights sum to one)."""
    rng = np.random.default_rng(2)
    q = _rand((1, 4, 3, 16), rng, 3.0)
    k = _rand((1, 50, 16), rng, 3.0)
    vrow = _rand((16,), rng)
    v = np.broadcast_to(vrow, (1, 50, 16)).copy()
    O, _ = oracle.attention(q, k, v, 0.25)
    np.testing.assert_allclose(O, np.broadcast_to(vrow, O.shape), atol=1e-14, rtol=0)


def test_uniform_k_gives_mean_and_log_count():
    """All K rows equal k: p_j = 1/s_k, O = mean_j V_j, lse = s q.k + ln s_k."""
    rng = np.random.default_rng(4)
    s_k, hd, s = 23, 8, 0.7
    q = _rand((1, 2, 3, hd), rng)
    krow = _rand((hd,), rng)
    k = np.broadcast_to(krow, (1, s_k, hd)).copy()
    v = _rand((1, s_k, hd), rng)
    O, L = oracle.attention(q, k, v, s)
    np.testing.assert_allclose(O, np.broadcast_to(v[0].mean(axis=0), O.shape), atol=1e-14, rtol=0)
    np.testing.assert_allclose(L, s * (q @ krow) + math.log(s_k), atol=1e-13, rtol=0)


def test_two_key_worked_example():
    """q = (1, 0), k_0 = (1, 0), k_1 = (0, 1), v_0 = (1, 2), v_1 = (3, 4),
    scale 1: logits (1, 0), p_0 = e/(1+e), O = p_0 v_0 + (1-p_0) v_1,
    lse = ln(1 + e)."""
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    v = np.array([[[1.0, 2.0], [3.0, 4.0]]])
    O, L = oracle.attention(q, k, v, 1.0)
    p0 = math.e / (1.0 + math.e)
    np.testing.assert_allclose(O[0, 0, 0], [p0 * 1 + (1 - p0) * 3, p0 * 2 + (1 - p0) * 4],
                               atol=1e-15, rtol=0)
    assert abs(L[0, 0, 0] - math.log(1.0 + math.e)) < 1e-15
    # scale halves the logits: lse = ln(e^0.5 + 1)
    _, L2 = oracle.attention(q, k, v, 0.5)
    assert abs(L2[0, 0, 0] - math.log(math.exp(0.5) + 1.0)) < 1e-15


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(6)
    q = _rand((40, 32), rng, 2.0)
    k = _rand((300, 32), rng, 2.0)
    p = oracle.attention_probs(q, k, 1 / math.sqrt(32))
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12, rtol=0)


# ------------------------------------------------ merge / tile-split identity
@pytest.mark.parametrize("seed", range(4))
def test_merge_of_random_key_partitions_equals_full(seed):
    """Any partition of the keys (uneven, singletons, any order), attended part
    by part and merged by lse, gives attention over all keys — this is the
    multi-KV-tile rescale identity and the split-KV identity at once."""
    rng = np.random.default_rng(100 + seed)
    s_k, hd = 61, 12
    q = _rand((1, 3, 5, hd), rng)
    k = _rand((1, s_k, hd), rng)
    v = _rand((1, s_k, hd), rng)
    O, L = oracle.attention(q, k, v, 0.4)
    perm = rng.permutation(s_k)
    cuts = np.sort(rng.choice(np.arange(1, s_k), size=rng.integers(1, 9), replace=False))
    parts = np.split(perm, cuts) + [np.array([], dtype=np.int64)]  # plus an empty part
    os_, ls_ = [], []
    for part in parts:
        o, l = oracle.attention(q, k[:, part], v[:, part], 0.4)
        os_.append(o.reshape(-1, hd))
        ls_.append(l.reshape(-1))
    Om, Lm = oracle.lse_merge(np.stack(os_), np.stack(ls_))
    np.testing.assert_allclose(Om, O.reshape(-1, hd), atol=TOL, rtol=0)
    np.testing.assert_allclose(Lm, L.reshape(-1), atol=TOL, rtol=0)


@pytest.mark.parametrize("n_split", [1, 2, 3, 8])
def test_split_partials_merge_to_full(n_split):
    """Contiguous chunks of ceil(s_k/n) keys merge back to the full result; the
    2-chunk case is the 'two KV tiles of 128' regime."""
    rng = np.random.default_rng(n_split)
    q = _rand((2, 2, 3, 16), rng)
    k = _rand((2, 256, 16), rng)
    v = _rand((2, 256, 16), rng)
    O, L = oracle.attention(q, k, v, 0.25)
    op, lp = oracle.split_partials(q, k, v, 0.25, n_split)
    Om, Lm = oracle.lse_merge(op, lp)
    np.testing.assert_allclose(Om, O.reshape(-1, 16), atol=TOL, rtol=0)
    np.testing.assert_allclose(Lm, L.reshape(-1), atol=TOL, rtol=0)


def test_split_with_an_empty_chunk():
    """5 keys in 4 chunks of ceil(5/4) = 2: sizes 2, 2, 1, 0.  The empty chunk
    is O = 0, lse = -inf and drops out of the merge."""
    rng = np.random.default_rng(21)
    q = _rand((1, 2, 3, 16), rng)
    k = _rand((1, 5, 16), rng)
    v = _rand((1, 5, 16), rng)
    op, lp = oracle.split_partials(q, k, v, 0.25, 4)
    assert np.all(np.isneginf(lp[3])) and np.all(op[3] == 0)
    O, L = oracle.attention(q, k, v, 0.25)
    Om, Lm = oracle.lse_merge(op, lp)
    np.testing.assert_allclose(Om, O.reshape(-1, 16), atol=TOL, rtol=0)
    np.testing.assert_allclose(Lm, L.reshape(-1), atol=TOL, rtol=0)


# ------------------------------------------------------------ overflow safety
def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(8)
    hd, s_k = 8, 33
    k = _rand((1, s_k, hd), rng)
    v = _rand((1, s_k, hd), rng)
    qv = k[0, 5] * 50.0
    q = qv.reshape(1, 1, 1, hd)
    x = (k[0] @ qv)
    assert x[5] - np.max(np.delete(x, 5)) > 40
    O, L = oracle.attention(q, k, v, 1.0)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 5], atol=1e-15 + math.exp(-40) * 10, rtol=0)
    assert abs(L[0, 0, 0] - x[5]) < 1e-12


def test_large_logits_stay_finite():
    rng = np.random.default_rng(9)
    q = _rand((1, 2, 2, 16), rng, 300.0)
    k = _rand((1, 40, 16), rng, 300.0)
    v = _rand((1, 40, 16), rng)
    O, L = oracle.attention(q, k, v, 1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    assert np.max(np.abs(L)) > 1e4      # the logits really are huge


# ---------------------------------------------------- gather and MQA mapping
def test_gather_equals_dense_on_gathered_rows_and_is_order_invariant():
    rng = np.random.default_rng(10)
    B, T, n_h, hd, P, s_k = 2, 3, 4, 8, 50, 17
    q = _rand((B, T, n_h, hd), rng)
    kp = _rand((P, hd), rng)
    vp = _rand((P, hd), rng)
    idx = np.stack([rng.permutation(P)[:s_k] for _ in range(B * T)]).reshape(B, T, s_k)
    O, L = oracle.attention(q, kp, vp, 0.3, kv_idx=idx)
    for b in range(B):
        for t in range(T):
            Od, Ld = oracle.attention(q[b:b + 1, t:t + 1], kp[idx[b, t]][None],
                                      vp[idx[b, t]][None], 0.3)
            np.testing.assert_allclose(O[b, t], Od[0, 0], atol=TOL, rtol=0)
            np.testing.assert_allclose(L[b, t], Ld[0, 0], atol=TOL, rtol=0)
    idx2 = np.stack([rng.permutation(row) for row in idx.reshape(-1, s_k)]).reshape(idx.shape)
    O2, L2 = oracle.attention(q, kp, vp, 0.3, kv_idx=idx2)
    np.testing.assert_allclose(O2, O, atol=TOL, rtol=0)
    np.testing.assert_allclose(L2, L, atol=TOL, rtol=0)


def test_mqa_row_equals_single_head_attention():
    rng = np.random.default_rng(12)
    B, T, n_h, hd, s_k = 2, 3, 5, 8, 19
    q = _rand((B, T, n_h, hd), rng)
    k = _rand((B, s_k, hd), rng)
    v = _rand((B, s_k, hd), rng)
    O, L = oracle.attention(q, k, v, 0.5)
    for (b, t, h) in [(0, 0, 0), (1, 2, 4), (0, 1, 3)]:
        Os, Ls = oracle.attention(q[b:b + 1, t:t + 1, h:h + 1], k[b:b + 1], v[b:b + 1], 0.5)
        np.testing.assert_allclose(O[b, t, h], Os[0, 0, 0], atol=TOL, rtol=0)
        assert abs(L[b, t, h] - Ls[0, 0, 0]) < TOL


def test_sampled_rows_match_full():
    w = W.make_custom(B=2, T=9, n_h=3, hd=16, s_k=40, seed=77)
    q, k, v, _ = W.make_inputs(w)
    O, L = oracle.attention(q, k, v, w.scale)
    rows = np.array([53, 0, 17, 2 * 9 * 3 - 1, 30])
    Os, Ls = oracle.attention(q, k, v, w.scale, rows=rows)
    np.testing.assert_allclose(Os, O.reshape(-1, 16)[rows], atol=0, rtol=0)
    np.testing.assert_allclose(Ls, L.reshape(-1)[rows], atol=0, rtol=0)


def test_row_metrics():
    a = np.array([[1.0, 0.0], [0.0, 0.0], [1.0, 1.0]])
    b = np.array([[1.0, 0.0], [0.0, 0.0], [1.0, 0.0]])
    m = oracle.row_metrics(a, b, np.array([0.0, -np.inf, 1.0]), np.array([0.0, -np.inf, 1.5]))
    assert m["max_abs"] == 1.0
    assert abs(m["min_row_cos"] - 1 / math.sqrt(2)) < 1e-15
    assert m["lse_err"] == 0.5


# ------------------------------------------------- the pins catch mistakes
def _mutants():
    from oracle import fp64 as A

    good = A.attention_rows

    def no_scale(q, K, V, s, sink_rows=None):
        return good(q, K, V, 1.0, sink_rows)

    def lse_log2(q, K, V, s, sink_rows=None):
        o, l = good(q, K, V, s, sink_rows)
        return o, l / math.log(2.0)

    def unnormalised(q, K, V, s, sink_rows=None):
        x = s * (q @ K.T)
        m = x.max(axis=1, keepdims=True)
        e = np.exp(x - m)
        return e @ V, m[:, 0] + np.log(e.sum(axis=1))

    def transposed_v(q, K, V, s, sink_rows=None):
        o, l = good(q, K, V[::-1], s, sink_rows)
        return o, l

    def wrong_sign(q, K, V, s, sink_rows=None):
        return good(q, -K, V, s, sink_rows)

    def lse_without_max(q, K, V, s, sink_rows=None):
        o, l = good(q, K, V, s, sink_rows)
        x = s * (q @ K.T)
        return o, l - x.max(axis=1)

    def sink_ignored(q, K, V, s, sink_rows=None):
        return good(q, K, V, s)

    def sink_value_one(q, K, V, s, sink_rows=None):
        # the sink's value vector taken as ones instead of zeros
        o, l = good(q, K, V, s, sink_rows)
        if sink_rows is None:
            return o, l
        return o + np.exp(np.asarray(sink_rows, np.float64) - l)[:, None], l

    return {"no_scale": no_scale, "lse_log2": lse_log2, "unnormalised": unnormalised,
            "reversed_v": transposed_v, "wrong_sign": wrong_sign,
            "lse_without_max": lse_without_max, "sink_ignored": sink_ignored,
            "sink_value_one": sink_value_one}


# ------------------------------------------------------------ attention sink
# Reading (page "May 24, 2026 — Session Start Plan", File Map and D1 Status
# Summary name a "sink merge" without its formula): one extra logit per query
# head with a zero value vector.


def _sinks(n_h, seed):
    g = np.random.default_rng(seed)
    s = g.normal(0.0, 2.0, n_h)
    s[0] = -np.inf  # the first head has no sink
    return s


@pytest.mark.parametrize("B,T,n_h,s_k,hd", [(1, 2, 3, 4, 3), (2, 1, 2, 1, 5), (1, 1, 4, 7, 2)])
def test_sink_matches_brute_force(B, T, n_h, s_k, hd):
    w = W.make_custom(B=B, T=T, n_h=n_h, hd=hd, s_k=s_k, out_dtype="f32", seed=50 + s_k)
    q, k, v, _ = W.make_inputs(w)
    sink = _sinks(n_h, s_k)
    O, L = oracle.attention(q, k, v, 0.7, sink=sink)
    Ob, Lb = brute.brute_attention(_tolist(oracle.to_f64(q)), _tolist(oracle.to_f64(k)),
                                   _tolist(oracle.to_f64(v)), 0.7, sink=list(sink))
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb), rtol=1e-13, atol=1e-12)


def test_sink_is_an_extra_key_with_zero_value():
    """For one query row, a sink logit s equals appending the key
    k* = q * s / (scale |q|^2) (its logit is exactly s) with value 0."""
    g = np.random.default_rng(7)
    hd, s_k, scale = 6, 5, 0.4
    q = g.normal(size=(1, 1, 1, hd))
    k = g.normal(size=(1, s_k, hd))
    v = g.normal(size=(1, s_k, hd))
    for s in (-3.0, 0.5, 4.0, 30.0):
        kstar = q[0, 0, 0] * s / (scale * float(q[0, 0, 0] @ q[0, 0, 0]))
        k2 = np.concatenate([k, kstar[None, None, :]], axis=1)
        v2 = np.concatenate([v, np.zeros((1, 1, hd))], axis=1)
        O_ref, L_ref = oracle.attention(q, k2, v2, scale)
        O, L = oracle.attention(q, k, v, scale, sink=np.array([s]))
        np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, L_ref, rtol=1e-13, atol=1e-12)


def test_sink_minus_inf_changes_nothing():
    w = W.make_custom(B=2, T=3, n_h=2, hd=8, s_k=9, out_dtype="f32", seed=61)
    q, k, v, idx = W.make_inputs(w)
    O0, L0 = oracle.attention(q, k, v, w.scale)
    O1, L1 = oracle.attention(q, k, v, w.scale, sink=np.full(2, -np.inf))
    assert np.array_equal(O0, O1) and np.array_equal(L0, L1)


def test_dominant_sink_empties_the_row():
    """A sink 60 above every logit: O within e^-60 of zero, lse = sink."""
    w = W.make_custom(B=1, T=2, n_h=2, hd=8, s_k=9, out_dtype="f32", seed=62)
    q, k, v, _ = W.make_inputs(w)
    O0, L0 = oracle.attention(q, k, v, w.scale)
    sink = np.full(2, float(L0.max()) + 60.0)
    O, L = oracle.attention(q, k, v, w.scale, sink=sink)
    assert np.abs(O).max() <= math.exp(-60) * np.abs(oracle.to_f64(v)).max() * 2
    np.testing.assert_allclose(L, np.broadcast_to(sink, L.shape), rtol=1e-15, atol=1e-12)


def test_sink_without_keys_gives_the_sink_lse():
    q = np.ones((1, 1, 2, 4))
    k = np.zeros((1, 0, 4))
    O, L = oracle.attention(q, k, k.copy(), 0.5, sink=np.array([1.5, -np.inf]))
    assert np.all(O == 0) and L[0, 0, 0] == 1.5 and L[0, 0, 1] == -np.inf


# ------------------------------------------------------------ several key sources
def _two_sources(seed, B=2, T=3, n_h=2, hd=4, pool=11, s_top=5, win=3):
    g = np.random.default_rng(seed)
    kp = _rand((pool, hd), g)
    vp = _rand((pool, hd), g)
    idx = np.stack([np.stack([g.permutation(pool)[:s_top] for _ in range(T)]) for _ in range(B)])
    kw = _rand((B, win, hd), g)
    vw = _rand((B, win, hd), g)
    q = _rand((B, T, n_h, hd), g)
    return q, [(kp, vp, idx), (kw, vw, None)]


def test_sources_match_brute_force_over_the_concatenated_keys():
    q, src = _two_sources(3)
    (kp, vp, idx), (kw, vw, _) = src
    sink = np.array([0.3, -np.inf])
    O, L = oracle.attention_sources(q, src, 0.6, sink=sink)
    B, T = q.shape[:2]
    for b in range(B):
        for t in range(T):
            keys = [list(r) for r in kp[idx[b, t]]] + [list(r) for r in kw[b]]
            vals = [list(r) for r in vp[idx[b, t]]] + [list(r) for r in vw[b]]
            Ob, Lb = brute.brute_attention([[_tolist(q[b, t])]], [keys], [vals], 0.6,
                                           sink=list(sink))
            np.testing.assert_allclose(O[b, t], np.array(Ob[0][0]), rtol=0, atol=1e-12)
            np.testing.assert_allclose(L[b, t], np.array(Lb[0][0]), rtol=1e-13, atol=1e-12)


def test_sources_equal_the_merge_of_each_source():
    """Union of sources = LSE merge of per-source results (the partition
    identity); one source alone = plain attention."""
    q, src = _two_sources(4, hd=6)
    O, L = oracle.attention_sources(q, src, 0.5)
    parts = [oracle.attention(q, k, v, 0.5, kv_idx=i) for k, v, i in src]
    Om, Lm = oracle.lse_merge(np.stack([p[0].reshape(-1, 6) for p in parts]),
                              np.stack([p[1].reshape(-1) for p in parts]))
    np.testing.assert_allclose(O.reshape(-1, 6), Om, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L.reshape(-1), Lm, rtol=1e-13, atol=1e-12)
    O1, L1 = oracle.attention_sources(q, src[1:], 0.5)
    O2, L2 = oracle.attention(q, src[1][0], src[1][1], 0.5)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-13)


def _sink_pin():
    test_sink_matches_brute_force(1, 2, 3, 4, 3)
    test_sink_is_an_extra_key_with_zero_value()


_PIN_CHECKS = [test_two_key_worked_example, test_uniform_v_gives_v,
               test_uniform_k_gives_mean_and_log_count, test_single_key_gives_that_value_row,
               lambda: test_dense_matches_brute_force(2, 3, 2, 5, 8),
               lambda: test_dense_matches_torch_sdpa_fp64(2, 5, 3, 37, 16), _sink_pin]


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_oracle_mistakes_are_caught(name, monkeypatch):
    """Plant a plausible mistake in the oracle (on the CPU) and check that at
    least one pin above fails."""
    from oracle import fp64 as A

    monkeypatch.setattr(A, "attention_rows", _mutants()[name])
    caught = 0
    for chk in _PIN_CHECKS:
        try:
            chk()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"


# Plausible misreadings of the multi-source oracle: each must fail a sources pin.
def _source_mutants():
    good = oracle.fp64.attention_sources

    def first_source_only(q, sources, scale, rows=None, sink=None):
        return good(q, sources[:1], scale, rows=rows, sink=sink)

    def mean_of_sources(q, sources, scale, rows=None, sink=None):
        outs = [good(q, [s], scale, rows=rows, sink=sink) for s in sources]
        return (sum(o for o, _ in outs) / len(outs),
                np.log(sum(np.exp(l) for _, l in outs)))

    def window_of_batch_zero(q, sources, scale, rows=None, sink=None):
        fixed = []
        for k, v, i in sources:
            if i is None:  # a dense source read from batch 0 for every batch
                k = np.repeat(np.asarray(k, np.float64)[:1], k.shape[0], axis=0)
                v = np.repeat(np.asarray(v, np.float64)[:1], v.shape[0], axis=0)
            fixed.append((k, v, i))
        return good(q, fixed, scale, rows=rows, sink=sink)

    return {"first_source_only": first_source_only, "mean_of_sources": mean_of_sources,
            "window_of_batch_zero": window_of_batch_zero}


@pytest.mark.parametrize("name", sorted(_source_mutants()))
def test_planted_source_mistakes_are_caught(name, monkeypatch):
    import oracle.fp64 as A

    mutant = _source_mutants()[name]  # wraps the correct function, taken before patching
    monkeypatch.setattr(A, "attention_sources", mutant)
    monkeypatch.setattr(oracle, "attention_sources", mutant)
    caught = 0
    for pin in (test_sources_match_brute_force_over_the_concatenated_keys,
                test_sources_equal_the_merge_of_each_source):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutant {name} passed every sources pin"
