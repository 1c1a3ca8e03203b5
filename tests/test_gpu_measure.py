"""GPU checks of the measurement helpers the benchmark reports beside the
attention: the decode read floor reads exactly the bytes the split kernel
reads, and the matrix-core ceiling computes the products it times."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def F():
    import fmha_mqa_fwd_amd
    return fmha_mqa_fwd_amd


def _words(t: torch.Tensor) -> np.ndarray:
    """The 32-bit words of a contiguous bf16 tensor's bytes, last dim halved."""
    return t.contiguous().view(torch.int32).numpy().view(np.uint32)


@pytest.mark.parametrize("B,T,n_h,hd,s_k,splits", [(32, 1, 128, 256, 1024, 8),
                                                   (2, 3, 50, 128, 700, 3),
                                                   (1, 1, 200, 64, 9, 8)])
def test_read_floor_reads_the_split_kernels_bytes(F, B, T, n_h, hd, s_k, splits):
    """Workgroup (tile, b, split) reads q rows [128 tile, +128) of batch b and
    K/V rows of split `split` of batch b, every word once: its XOR word equals
    the CPU's XOR of those bytes (an empty trailing split reads only q)."""
    w = W.make_custom(B=B, T=T, n_h=n_h, hd=hd, s_k=s_k, out_dtype="bf16", seed=s_k + hd)
    q, k, v, _ = W.make_inputs(w)
    got = F.read_floor(q.to(DEV), k.to(DEV), v.to(DEV), splits).cpu().numpy().view(np.uint32)
    rows = T * n_h
    tiles = -(-rows // 128)
    chunk = -(-s_k // splits)
    qw = _words(q).reshape(B, rows, hd // 2)
    kw, vw = _words(k).reshape(B, s_k, hd // 2), _words(v).reshape(B, s_k, hd // 2)
    assert got.shape == (tiles * B * splits,)
    for sp in range(splits):
        lo, hi = min(sp * chunk, s_k), min((sp + 1) * chunk, s_k)
        for b in range(B):
            kv = np.bitwise_xor.reduce(np.concatenate([kw[b, lo:hi].ravel(), vw[b, lo:hi].ravel(),
                                                       np.zeros(1, np.uint32)]))
            for t in range(tiles):
                want = kv ^ np.bitwise_xor.reduce(qw[b, 128 * t:128 * (t + 1)].ravel())
                assert got[t + tiles * (b + B * sp)] == want, (t, b, sp)


def _ops(seed, const=None):
    g = torch.Generator().manual_seed(seed)
    if const is not None:
        return torch.full((8, 8, 64, 8), const, dtype=torch.bfloat16)
    return torch.randn(8, 8, 64, 8, generator=g).to(torch.bfloat16)


def _expected_sums(ops: torch.Tensor, iters: int) -> np.ndarray:
    """Sum of the elements of D_c = iters * A_c.B_c for every wave and chain:
    sum_ij sum_k A[i,k] B[k,j] = sum_k (sum_i A[i,k]) (sum_j B[k,j]), where lane l
    of a fragment holds row/column l % 32 and k = 8 (l // 32) + e."""
    o = ops.double().numpy().reshape(8, 4, 2, 2, 32, 8)   # wave, chain, A/B, lane half, l%32, e
    colA = o[:, :, 0].sum(axis=3)                          # [wave, chain, half, e]
    rowB = o[:, :, 1].sum(axis=3)
    return iters * (colA * rowB).sum(axis=(2, 3))          # [wave, chain]


@pytest.mark.parametrize("const", [None, 0.5])
def test_mfma_ceiling_computes_the_products_it_times(F, const):
    ops = _ops(5, const)
    iters = 7
    sums, clocks = F.mfma_ceiling(ops.to(DEV), n_wg=300, iters=iters)
    torch.cuda.synchronize()
    want = _expected_sums(ops, iters)
    got = sums.cpu().double().numpy()
    scale = np.abs(ops.double().numpy()).max() ** 2 * 32 * 1024 * iters
    for wg in (0, 123, 299):
        np.testing.assert_allclose(got[wg], want, rtol=0, atol=1e-5 * scale)
    if const is not None:
        # every element of D_c is iters * 16 * 0.25: exact
        assert np.all(got == iters * 16 * 0.25 * 1024)
    c = clocks.cpu().numpy()
    assert np.all(c[:, 0] > 0) and np.all(c[:, 1] > 0)
    # shader cycles per 100 MHz tick: an effective clock between 0.5 and 3 GHz
    ghz = c[:, 0] / c[:, 1] * 0.1
    assert np.all((ghz > 0.5) & (ghz < 3.0)), ghz.min()
