"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/fmha_mqa.h declares, and rejects bad arguments with the
documented status before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmha_mqa.h")


def _lib_path():
    path = os.path.join(ROOT, "fmha_mqa_fwd_amd", "libfmha_mqa.so")
    if not os.path.exists(path):  # build only when nothing is built
        import importlib.util  # by path: the package import needs the library
        spec = importlib.util.spec_from_file_location(
            "fmha_mqa_build", os.path.join(ROOT, "fmha_mqa_fwd_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    return path


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fmha_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared_functions() == ["fmha_attention_sink", "fmha_gather_floor",
                                     "fmha_index_scores", "fmha_lse_merge",
                                     "fmha_mfma_ceiling", "fmha_mqa_fwd",
                                     "fmha_mqa_fwd_noalloc", "fmha_mqa_fwd_partials",
                                     "fmha_mqa_fwd_sink", "fmha_mqa_fwd_sources_partials",
                                     "fmha_mqa_workspace_bytes",
                                     "fmha_read_floor", "fmha_status_string",
                                     "fmha_topk_select"]


def test_library_exports_every_declared_symbol():
    path = _lib_path()
    lib = ctypes.CDLL(path)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True)
    exported = {ln.split()[-1] for ln in nm.stdout.splitlines() if " T " in ln}
    for name in _declared_functions():
        assert name in exported, f"{name} is not a dynamic text symbol"


def test_binding_covers_every_symbol():
    _lib_path()
    import fmha_mqa_fwd_amd as F
    assert sorted(F.SIGNATURES) == _declared_functions()


@pytest.fixture(scope="module")
def F():
    _lib_path()
    import fmha_mqa_fwd_amd
    return fmha_mqa_fwd_amd


# fake, suitably aligned device addresses: validation must reject before any use
A = 1 << 20


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


# The cases that hand the C entry points fake device addresses run only where
# no GPU is visible: should validation ever regress, no kernel can then be
# launched on an unmapped address.
fake_pointers = pytest.mark.skipif(_gpu_visible(),
                                   reason="passes fake device addresses: host-only check")


def _fwd(F, **kw):
    args = dict(q=A, k=A, v=A, kv_idx=None, out=A, lse=A, B=1, T=1, n_h=1, s_k=8, hd=64,
                pool_rows=0, scale=0.125, out_dtype=0, num_splits=1, ws=None, ws_bytes=0,
                stream=None)
    args.update(kw)
    return F.raw_fwd(args["q"], args["k"], args["v"], args["kv_idx"], args["out"], args["lse"],
                     args["B"], args["T"], args["n_h"], args["s_k"], args["hd"],
                     args["pool_rows"], args["scale"], args["out_dtype"], args["num_splits"],
                     args["ws"], args["ws_bytes"], args["stream"])


def test_status_strings(F):
    assert F.status_string(0) == "ok"
    assert "align" in F.status_string(3)
    assert "scratch" in F.status_string(F.FMHA_ERR_SCRATCH_LIMIT)
    assert F.status_string(99) == "unknown status"


def _noalloc(F, **kw):
    args = dict(q=A, k=A, v=A, kv_idx=None, out=A, lse=A, B=1, T=1, n_h=1, s_k=8, hd=64,
                pool_rows=0, scale=0.125, out_dtype=0, num_splits=1, stream=None)
    args.update(kw)
    return F._binding._lib.fmha_mqa_fwd_noalloc(
        args["q"], args["k"], args["v"], args["kv_idx"], args["out"], args["lse"], args["B"],
        args["T"], args["n_h"], args["s_k"], args["hd"], args["pool_rows"], args["scale"],
        args["out_dtype"], args["num_splits"], args["stream"])


@fake_pointers
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 0),                                   # nothing to compute
    (dict(hd=96), 2), (dict(q=None), 1), (dict(num_splits=9), 1), (dict(q=A + 8), 3),
    # partials over the 64 MiB buffer: 4096 rows x hd 256 x 16 splits (64.25 MiB)
    (dict(B=32, n_h=128, hd=256, s_k=1024, num_splits=16), 6),
    (dict(B=32, n_h=128, hd=512, s_k=1024, num_splits=8), 6),
])
def test_noalloc_validates_before_touching_the_device(F, kw, status):
    """fmha_mqa_fwd_noalloc rejects bad arguments, and partials larger than its
    static buffer, before any device call (every pointer here is fake)."""
    assert _noalloc(F, **kw) == status


def test_noalloc_limit_matches_the_workspace_size(F):
    assert F.SCRATCH_BYTES == 64 << 20
    assert F.workspace_bytes(32, 1, 128, 256, 15) <= F.SCRATCH_BYTES
    assert F.workspace_bytes(32, 1, 128, 256, 16) > F.SCRATCH_BYTES


@fake_pointers
@pytest.mark.parametrize("kw,status", [
    (dict(hd=96), 2), (dict(hd=1024), 2), (dict(hd=0), 2),
    (dict(out_dtype=2), 1), (dict(B=-1), 1), (dict(s_k=-1), 1), (dict(num_splits=0), 1),
    (dict(num_splits=9), 1), (dict(scale=0.0), 1), (dict(scale=-1.0), 1),
    (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1),
    (dict(q=None), 1), (dict(out=None), 1), (dict(lse=None), 1), (dict(k=None), 1),
    (dict(v=None), 1), (dict(kv_idx=A, pool_rows=0), 1),
    (dict(q=A + 8), 3), (dict(k=A + 2), 3), (dict(out=A + 4), 3), (dict(lse=A + 2), 3),
    (dict(kv_idx=A + 2, pool_rows=5), 3),
    (dict(num_splits=2), 4), (dict(num_splits=2, ws=A, ws_bytes=16), 4),
    (dict(num_splits=2, ws=A + 8, ws_bytes=1 << 30), 4),
])
def test_fwd_rejects_bad_arguments(F, kw, status):
    assert _fwd(F, **kw) == status


@fake_pointers
@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0), dict(n_h=0, q=None, out=None)])
def test_fwd_empty_problem_is_a_no_op(F, kw):
    # zero rows: nothing to launch, OK even with dangling pointers
    assert _fwd(F, **kw) == 0


def test_workspace_bytes(F):
    assert F.workspace_bytes(32, 1, 128, 256, 1) == 0
    rows = 32 * 128
    o = 8 * rows * 256 * 4
    l_ = 8 * rows * 4
    r = lambda x: (x + 255) // 256 * 256
    assert F.workspace_bytes(32, 1, 128, 256, 8) == r(o) + r(l_)
    assert F.workspace_bytes(-1, 1, 1, 64, 2) == 0


@fake_pointers
@pytest.mark.parametrize("args,status", [
    ((A, A, 0, 4, 64, A, 0, A, None), 1),      # n_parts < 1
    ((A, A, 2, 4, 62, A, 0, A, None), 1),      # hd not a multiple of 4
    ((A, A, 2, -1, 64, A, 0, A, None), 1),
    ((A, A, 2, 4, 64, A, 3, A, None), 1),      # bad dtype
    ((None, A, 2, 4, 64, A, 0, A, None), 1),
    ((A + 4, A, 2, 4, 64, A, 0, A, None), 3),
    ((A, A, 2, 4, 64, A + 4, 0, A, None), 3),  # fp32 out needs 16 B
    ((A, A, 2, 0, 64, None, 0, None, None), 0),  # no rows: no-op
])
def test_merge_rejects_bad_arguments(F, args, status):
    assert F.raw_merge(*args) == status


# ------------------------------------------------------------ attention sink
@fake_pointers
def test_fwd_sink_requires_a_sink(F):
    lib = F._binding._lib
    args = (A, A, A, None, A, A, 1, 1, 1, 8, 64, 0, 0.125, 0, 1, None, 0, None)
    assert lib.fmha_mqa_fwd_sink(*args, None) == 1
    assert lib.fmha_mqa_fwd_sink(*args, A + 2) == 3          # misaligned sink
    bad = (A, A, A, None, A, A, 1, 1, 1, 8, 96, 0, 0.125, 0, 1, None, 0, None)
    assert lib.fmha_mqa_fwd_sink(*bad, A) == 2               # same checks as the plain forward


@fake_pointers
@pytest.mark.parametrize("args,status", [
    ((A, A, A, 4, 1, 64, 2, None), 1),       # bad dtype
    ((A, A, A, -1, 1, 64, 0, None), 1),
    ((A, A, A, 4, 0, 64, 0, None), 1),       # n_h < 1
    ((A, A, A, 4, 1, 62, 0, None), 1),       # hd not a multiple of 4
    ((None, A, A, 4, 1, 64, 0, None), 1),
    ((A, None, A, 4, 1, 64, 0, None), 1),
    ((A, A, None, 4, 1, 64, 0, None), 1),
    ((A + 8, A, A, 4, 1, 64, 0, None), 3),   # fp32 out needs 16 B
    ((A, A + 2, A, 4, 1, 64, 0, None), 3),
    ((A, A, A + 1, 4, 1, 64, 0, None), 3),
    ((None, None, None, 0, 1, 64, 0, None), 0),  # no rows: no-op
])
def test_attention_sink_validates(F, args, status):
    assert F._binding._lib.fmha_attention_sink(*args) == status


# ------------------------------------------------------------ top-k indexer
@pytest.mark.parametrize("args,status", [
    ((A, A, A, A, 1, 2, 48, 128, 100, None), 2),    # index heads not 32/64
    ((A, A, A, A, 1, 2, 64, 96, 100, None), 2),     # width not 64/128
    ((A, A, A, A, -1, 2, 64, 128, 100, None), 1),
    ((A, A, A, A, 1, 2, 64, 128, 0, None), 1),      # empty pool
    ((None, A, A, A, 1, 2, 64, 128, 100, None), 1),
    ((A, A, None, A, 1, 2, 64, 128, 100, None), 1),
    ((A + 8, A, A, A, 1, 2, 64, 128, 100, None), 3),
    ((A, A, A, A + 2, 1, 2, 64, 128, 100, None), 3),
    ((None, None, None, None, 0, 5, 64, 128, 100, None), 0),  # no tokens: no-op
])
@fake_pointers
def test_index_scores_validates(F, args, status):
    assert F._binding._lib.fmha_index_scores(*args) == status


@fake_pointers
@pytest.mark.parametrize("args,status", [
    ((A, A, 4, 0, 8, None), 1),
    ((A, A, 4, 100, 0, None), 1),
    ((A, A, -1, 100, 8, None), 1),
    ((A, A, 4, 40000, 8, None), 2),     # row longer than the 32768 keys one workgroup holds
    ((None, A, 4, 100, 8, None), 1),
    ((A, A + 2, 4, 100, 8, None), 3),
    ((None, None, 0, 100, 8, None), 0),
])
def test_topk_select_validates(F, args, status):
    assert F._binding._lib.fmha_topk_select(*args) == status


# ------------------------------------------------------- Python-side checks
# Host tensors and wrong caller buffers are rejected before any device call,
# so these run without a GPU.
def test_wrappers_reject_host_tensors(F):
    import torch
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        F.fwd(q, k, k.clone())
    with pytest.raises(ValueError, match="GPU"):
        F.FwdPlan(q, k, k.clone(), num_splits=2)
    with pytest.raises(ValueError, match="GPU"):
        F.lse_merge(torch.zeros(2, 3, 8), torch.zeros(2, 3))
    with pytest.raises(ValueError, match="GPU"):
        F.apply_sink(torch.zeros(3, 4, 8), torch.zeros(3, 4), torch.zeros(4))
    with pytest.raises(ValueError, match="GPU"):
        F.index_scores(torch.zeros(1, 1, 32, 64, dtype=torch.bfloat16),
                       torch.zeros(5, 64, dtype=torch.bfloat16), torch.zeros(1, 1, 32))
    with pytest.raises(ValueError, match="GPU"):
        F.topk_select(torch.zeros(2, 100), 8)
    with pytest.raises(ValueError, match="GPU"):
        F.fwd_sources(q, [(k, k.clone(), None)])


def test_device_and_buffer_checks(F):
    import torch
    B = F._binding
    gpu = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="is on cpu"):
        B._same_gpu(gpu, out=torch.zeros(3))
    B._same_gpu(gpu, out=None)  # absent tensors are fine
    good = torch.zeros(2, 3, 4, 8)
    B._check_buf("out", good, (2, 3, 4, 8), (torch.float32,))
    for bad in (torch.zeros(2, 3, 4, 9), torch.zeros(2, 3, 4, 8, dtype=torch.float64),
                torch.zeros(2, 3, 8, 4).transpose(2, 3)):
        with pytest.raises(ValueError, match="out must be"):
            B._check_buf("out", bad, (2, 3, 4, 8), (torch.float32,))


@fake_pointers
@pytest.mark.parametrize("args,status", [
    ((A, A, A, A, 1, 2, 64, 100, 0, None), 1),      # empty pool
    ((A, A, A, A, 1, 2, 64, 96, 10, None), 2),      # head dim
    ((A, A, A, A, -1, 2, 64, 128, 10, None), 1),
    ((None, A, A, A, 1, 2, 64, 128, 10, None), 1),
    ((A + 8, A, A, A, 1, 2, 64, 128, 10, None), 3),
    ((None, None, None, None, 0, 2, 64, 128, 10, None), 0),  # no tokens: no-op
])
def test_gather_floor_validates(F, args, status):
    assert F._binding._lib.fmha_gather_floor(*args) == status


def _partials(F, **kw):
    args = dict(q=A, k=A, v=A, kv_idx=None, o=A, l=A, B=1, T=1, n_h=1, s_k=8, hd=64,
                pool_rows=0, scale=0.125, num_splits=1, stream=None)
    args.update(kw)
    return F._binding._lib.fmha_mqa_fwd_partials(
        args["q"], args["k"], args["v"], args["kv_idx"], args["o"], args["l"], args["B"],
        args["T"], args["n_h"], args["s_k"], args["hd"], args["pool_rows"], args["scale"],
        args["num_splits"], args["stream"])


@fake_pointers
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 0),                     # nothing to compute
    (dict(hd=96), 2),                   # unsupported head dim
    (dict(o=None), 1),                  # partial planes missing
    (dict(l=None), 1),
    (dict(num_splits=0), 1),
    (dict(num_splits=9, s_k=8), 1),     # more splits than keys
    (dict(scale=0.0), 1),
    (dict(o=A + 4), 3),                 # o_parts not 16-byte aligned
    (dict(l=A + 2), 3),                 # lse_parts not 4-byte aligned
    (dict(kv_idx=A, pool_rows=0), 1),   # gather without a pool
])
def test_partials_validates_before_launch(F, kw, status):
    """fmha_mqa_fwd_partials rejects bad arguments with the documented status
    (no device is touched: every pointer here is a fake address)."""
    assert _partials(F, **kw) == status


def _sources(F, srcs, **kw):
    """fmha_mqa_fwd_sources_partials over (k, v, kv_idx, s_k, pool_rows,
    num_splits) tuples; srcs None passes a NULL source array."""
    args = dict(q=A, o=A, l=A, B=1, T=1, n_h=1, hd=512, scale=0.125, stream=None, n=None)
    args.update(kw)
    arr = None
    if srcs is not None:
        arr = (F.KvSource * max(len(srcs), 1))(*[F.KvSource(*x) for x in srcs])
    n = len(srcs or []) if args["n"] is None else args["n"]
    return F._binding._lib.fmha_mqa_fwd_sources_partials(
        args["q"], arr, n, args["o"], args["l"], args["B"], args["T"], args["n_h"], args["hd"],
        args["scale"], args["stream"])


TOP = (A, A, A, 8, 100, 2)    # gather source: 8 keys of a 100-row pool, 2 splits
WIN = (A, A, None, 4, 0, 1)   # dense source: 4 keys


@fake_pointers
@pytest.mark.parametrize("srcs,kw,status", [
    ([TOP, WIN], dict(B=0), 0),                           # nothing to compute
    ([], {}, 1),                                          # no sources
    (None, dict(n=2), 1),                                 # NULL source array
    ([TOP, WIN], dict(hd=96), 2),
    ([TOP, (A, A, None, 4, 0, 5)], {}, 1),                # second source: more splits than keys
    ([(A, A, A, 8, 0, 1), WIN], {}, 1),                   # gather without a pool
    ([TOP, (None, A, None, 4, 0, 1)], {}, 1),             # second source without k
    ([TOP, (A + 8, A, None, 4, 0, 1)], {}, 3),            # second source's k misaligned
    ([TOP, WIN], dict(o=A + 4), 3),
    ([TOP, WIN], dict(l=A + 2), 3),
    ([TOP, WIN], dict(scale=0.0), 1),
    ([TOP, WIN], dict(q=None), 1),
])
def test_sources_partials_validate_every_source_before_launch(F, srcs, kw, status):
    """fmha_mqa_fwd_sources_partials rejects a bad source (first or later)
    with fmha_mqa_fwd_partials' status before anything is launched (every
    pointer here is a fake address)."""
    assert _sources(F, srcs, **kw) == status


@fake_pointers
@pytest.mark.parametrize("args,status", [
    ((A, A, A, A, 1, 1, 8, 128, 256, 0, None), 1),       # no splits
    ((A, A, A, A, 1, 1, 8, 128, 256, 129, None), 1),     # more splits than keys
    ((A, A, A, A, 1, 1, 8, 0, 256, 1, None), 1),         # no keys
    ((A, A, A, A, 1, 1, 8, 1024, 512, 8, None), 2),      # head dim
    ((A, A, A, A, 1, 1, 8, 1024, 256, 4, None), 2),      # 256-key split: over 64 KiB per tensor
    ((None, A, A, A, 1, 1, 8, 128, 256, 1, None), 1),
    ((A + 8, A, A, A, 1, 1, 8, 128, 256, 1, None), 3),
    ((A, A, A, A + 2, 1, 1, 8, 128, 256, 1, None), 3),
    ((None, None, None, None, 0, 1, 8, 128, 256, 1, None), 0),  # no rows: no-op
])
def test_read_floor_validates(F, args, status):
    assert F._binding._lib.fmha_read_floor(*args) == status


@fake_pointers
@pytest.mark.parametrize("args,status", [
    ((A, A, A, 0, 10, None), 1), ((A, A, A, 4, 0, None), 1), ((None, A, A, 4, 10, None), 1),
    ((A + 8, A, A, 4, 10, None), 3), ((A, A, A + 4, 4, 10, None), 3),
])
def test_mfma_ceiling_validates(F, args, status):
    assert F._binding._lib.fmha_mfma_ceiling(*args) == status
