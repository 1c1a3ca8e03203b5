"""ctypes binding over libfmha_mqa.so (argument marshalling only).

PyTorch supplies device memory (``tensor.data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``); every step of the attention
runs in the library's HIP kernels.  Importing this module fails loudly when the
library has not been built: there is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfmha_mqa.so")

FMHA_F32 = 0
FMHA_BF16 = 1
FMHA_ERR_SCRATCH_LIMIT = 6
SCRATCH_BYTES = 64 << 20   # FMHA_SCRATCH_BYTES: the static split-KV buffer per GPU

# Every symbol include/fmha_mqa.h declares, with its ctypes signature.
_c_int, _c_size, _c_void_p, _c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
class KvSource(ctypes.Structure):
    """fmha_kv_source: one key source of fmha_mqa_fwd_sources_partials."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("kv_idx", ctypes.c_void_p),
                ("s_k", ctypes.c_int), ("pool_rows", ctypes.c_int),
                ("num_splits", ctypes.c_int)]


SIGNATURES = {
    "fmha_mqa_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "fmha_mqa_fwd": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                              _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                              _c_int, _c_int, _c_void_p, _c_size, _c_void_p]),
    "fmha_mqa_fwd_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                      _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                      _c_float, _c_int, _c_int, _c_void_p]),
    "fmha_mqa_fwd_sink": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _c_float, _c_int, _c_int, _c_void_p, _c_size, _c_void_p,
                                   _c_void_p]),
    "fmha_mqa_fwd_partials": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_float, _c_int, _c_void_p]),
    "fmha_mqa_fwd_sources_partials": (_c_int, [_c_void_p, ctypes.POINTER(KvSource), _c_int,
                                               _c_void_p, _c_void_p, _c_int, _c_int, _c_int,
                                               _c_int, _c_float, _c_void_p]),
    "fmha_attention_sink": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int,
                                     _c_int, _c_void_p]),
    "fmha_lse_merge": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p,
                                _c_int, _c_void_p, _c_void_p]),
    "fmha_index_scores": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _c_void_p]),
    "fmha_topk_select": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p]),
    "fmha_gather_floor": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _c_void_p]),
    "fmha_read_floor": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _c_void_p]),
    "fmha_mfma_ceiling": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_void_p]),
    "fmha_status_string": (ctypes.c_char_p, [_c_int]),
}


class FmhaError(RuntimeError):
    """A non-zero fmha_status from the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with `python -m fmha_mqa_fwd_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def status_string(status: int) -> str:
    return _lib.fmha_status_string(int(status)).decode()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return FMHA_F32
    if dt == torch.bfloat16:
        return FMHA_BF16
    raise ValueError(f"out dtype must be float32 or bfloat16, got {dt}")


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _same_gpu(dev: torch.device, **tensors) -> None:
    """Every given tensor lives on the GPU `dev` (a host pointer or another
    device's memory must never reach a kernel)."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {dev}")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _check_buf(name: str, t: torch.Tensor, shape, dtypes) -> None:
    """A caller-provided output: exactly `shape`, one of `dtypes`, contiguous."""
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {'/'.join(str(d) for d in dtypes)} "
                         f"tensor of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _source_dims(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 kv_idx: Optional[torch.Tensor]) -> Tuple[int, int]:
    """(s_k, pool_rows) of one key source for q [B, T, n_h, hd]: dense k, v
    [B, s_k, hd] (kv_idx None) or pools [P, hd] with kv_idx int32 [B, T, s_k];
    all bf16 and contiguous."""
    B, T, _, hd = q.shape
    if kv_idx is None:
        if k.dim() != 3 or k.shape[0] != B or k.shape[2] != hd or v.shape != k.shape:
            raise ValueError("dense k/v must be [B, s_k, hd] with q's B and hd")
        s_k, pool_rows = k.shape[1], 0
    else:
        if k.dim() != 2 or k.shape[1] != hd or v.shape != k.shape:
            raise ValueError("gather k/v pools must be [P, hd] with q's hd")
        if kv_idx.dtype != torch.int32 or tuple(kv_idx.shape[:2]) != (B, T) or kv_idx.dim() != 3:
            raise ValueError("kv_idx must be int32 [B, T, s_k]")
        s_k, pool_rows = kv_idx.shape[2], k.shape[0]
        if not kv_idx.is_contiguous():
            raise ValueError("kv_idx must be contiguous")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return int(s_k), int(pool_rows)


def default_scale(hd: int) -> float:
    """1/sqrt(hd) as the fp32 value the kernel receives."""
    return float(torch.tensor(1.0 / math.sqrt(hd), dtype=torch.float32))


def workspace_bytes(B: int, T: int, n_h: int, hd: int, num_splits: int) -> int:
    return int(_lib.fmha_mqa_workspace_bytes(B, T, n_h, hd, num_splits))


class FwdPlan:
    """fmha_mqa_fwd with its arguments checked and marshalled once.

    Calling the plan launches the forward again on the same tensors and
    stream (for loops and timing, where per-call Python work would otherwise
    sit between launches); it returns (out, lse).  Arguments as for `fwd`.
    With partials=True the plan calls fmha_mqa_fwd_partials instead: out and
    lse are then the fp32 split planes [num_splits, B, T, n_h, hd] and
    [num_splits, B, T, n_h] (allocated when None); out_dtype, workspace and
    sink do not apply.  With noalloc=True it calls fmha_mqa_fwd_noalloc: out
    and lse must be given, and there is no workspace or sink.
    """

    def __init__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 kv_idx: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                 out_dtype: torch.dtype = torch.bfloat16, num_splits: int = 1,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None,
                 sink: Optional[torch.Tensor] = None, partials: bool = False,
                 noalloc: bool = False):
        if q.dim() != 4:
            raise ValueError("q must be [B, T, n_h, hd]")
        B, T, n_h, hd = q.shape
        s_k, pool_rows = _source_dims(q, k, v, kv_idx)
        if sink is not None:
            if sink.dtype != torch.float32 or sink.shape != (n_h,) or not sink.is_contiguous():
                raise ValueError("sink must be a contiguous float32 [n_h] tensor")
        dev = q.device
        _same_gpu(dev, k=k, v=v, kv_idx=kv_idx, sink=sink, out=out, lse=lse, workspace=workspace)
        if partials:
            if sink is not None or workspace is not None:
                raise ValueError("partials take neither a sink nor a workspace")
            if scale is None:
                scale = default_scale(hd)
            S = int(num_splits)
            if out is None:
                out = torch.empty((S, B, T, n_h, hd), dtype=torch.float32, device=dev)
            if lse is None:
                lse = torch.empty((S, B, T, n_h), dtype=torch.float32, device=dev)
            _check_buf("o_parts", out, (S, B, T, n_h, hd), (torch.float32,))
            _check_buf("lse_parts", lse, (S, B, T, n_h), (torch.float32,))
            self._keep = (q, k, v, kv_idx)
            self.out, self.lse = out, lse
            self._fn = _lib.fmha_mqa_fwd_partials
            self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(out), _ptr(lse),
                          B, T, n_h, s_k, hd, pool_rows, float(scale), S,
                          _stream_handle(stream))
            return
        if out is not None:
            _check_buf("out", out, (B, T, n_h, hd), (torch.float32, torch.bfloat16))
        if lse is not None:
            _check_buf("lse", lse, (B, T, n_h), (torch.float32,))
        if noalloc:
            if sink is not None or workspace is not None:
                raise ValueError("the allocation-free forward takes neither a sink nor a "
                                 "workspace")
            if out is None or lse is None:
                raise ValueError("the allocation-free forward writes into the caller's out "
                                 "and lse")
            self._keep = (q, k, v, kv_idx)
            self.out, self.lse = out, lse
            self._fn = _lib.fmha_mqa_fwd_noalloc
            self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(out), _ptr(lse),
                          B, T, n_h, s_k, hd, pool_rows,
                          float(default_scale(hd) if scale is None else scale),
                          _dtype_code(out.dtype), int(num_splits), _stream_handle(stream))
            return
        if workspace is not None and not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if scale is None:
            scale = default_scale(hd)
        if out is None:
            out = torch.empty((B, T, n_h, hd), dtype=out_dtype, device=dev)
        if lse is None:
            lse = torch.empty((B, T, n_h), dtype=torch.float32, device=dev)
        ws_need = workspace_bytes(B, T, n_h, hd, num_splits)
        if workspace is None and ws_need > 0:
            workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        # keep every tensor the launch reads or writes alive with the plan
        self._keep = (q, k, v, kv_idx, workspace, sink)
        self.out, self.lse = out, lse
        self._fn = _lib.fmha_mqa_fwd if sink is None else _lib.fmha_mqa_fwd_sink
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(out), _ptr(lse),
                      B, T, n_h, s_k, hd, pool_rows, float(scale),
                      _dtype_code(out.dtype), int(num_splits), _ptr(workspace), ws_bytes,
                      _stream_handle(stream))
        if sink is not None:
            self._args = self._args + (_ptr(sink),)

    def __call__(self) -> Tuple[torch.Tensor, torch.Tensor]:
        st = self._fn(*self._args)
        if st != 0:
            raise FmhaError(self._fn.__name__, st)
        return self.out, self.lse


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
        kv_idx: Optional[torch.Tensor] = None, scale: Optional[float] = None,
        out_dtype: torch.dtype = torch.bfloat16, num_splits: int = 1,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, stream=None,
        sink: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Multi-query attention forward (see include/fmha_mqa.h).

    q [B, T, n_h, hd] bf16; dense k, v [B, s_k, hd] bf16, or pools [P, hd] with
    kv_idx [B, T, s_k] int32.  Returns (out [B, T, n_h, hd], lse [B, T, n_h] fp32).
    With sink (fp32 [n_h]) the attention sink joins every row
    (fmha_mqa_fwd_sink).
    """
    return FwdPlan(q, k, v, kv_idx, scale, out_dtype, num_splits, out, lse, workspace, stream,
                   sink)()


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                lse: torch.Tensor, kv_idx: Optional[torch.Tensor] = None,
                scale: Optional[float] = None, num_splits: int = 1, stream=None
                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fmha_mqa_fwd_noalloc: the forward into the caller's out [B, T, n_h, hd]
    (fp32 or bf16) and lse [B, T, n_h] fp32 with no workspace — split-KV
    partials live in the library's static per-GPU scratch buffer, and nothing
    is allocated here either.  Arguments otherwise as for `fwd`."""
    return FwdPlan(q, k, v, kv_idx, scale, out.dtype, num_splits, out, lse, stream=stream,
                   noalloc=True)()


def fwd_partials(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 kv_idx: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                 num_splits: int = 1, o_parts: Optional[torch.Tensor] = None,
                 lse_parts: Optional[torch.Tensor] = None, stream=None
                 ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fmha_mqa_fwd_partials: the split-KV forward without its merge.  Returns
    the fp32 planes (o_parts [num_splits, B, T, n_h, hd], lse_parts
    [num_splits, B, T, n_h]); arguments as for `fwd`."""
    return FwdPlan(q, k, v, kv_idx, scale, num_splits=num_splits, out=o_parts, lse=lse_parts,
                   stream=stream, partials=True)()


class SourcesPlan:
    """fmha_mqa_fwd_sources_partials with its arguments checked and marshalled
    once; calling the plan launches again and returns (o_parts, lse_parts):
    fp32 [sum of splits, B, T, n_h, hd] and [sum of splits, B, T, n_h], the
    planes of sources[0] first (allocated when None).

    sources: sequence of (k, v, kv_idx, num_splits) as for `fwd_sources`."""

    def __init__(self, q: torch.Tensor, sources, scale: Optional[float] = None,
                 o_parts: Optional[torch.Tensor] = None,
                 lse_parts: Optional[torch.Tensor] = None, stream=None):
        if q.dim() != 4:
            raise ValueError("q must be [B, T, n_h, hd]")
        B, T, n_h, hd = q.shape
        if len(sources) < 1:
            raise ValueError("at least one key source is needed")
        dev = q.device
        descs, keep = [], [q]
        for src in sources:
            k, v, kv_idx = src[0], src[1], src[2]
            splits = int(src[3]) if len(src) > 3 else 1
            _same_gpu(dev, k=k, v=v, kv_idx=kv_idx)
            s_k, pool_rows = _source_dims(q, k, v, kv_idx)
            descs.append(KvSource(_ptr(k), _ptr(v), _ptr(kv_idx), s_k, pool_rows, splits))
            keep += [k, v, kv_idx]
        total = sum(d.num_splits for d in descs)
        if o_parts is None:
            o_parts = torch.empty((total, B, T, n_h, hd), dtype=torch.float32, device=dev)
        if lse_parts is None:
            lse_parts = torch.empty((total, B, T, n_h), dtype=torch.float32, device=dev)
        _same_gpu(dev, o_parts=o_parts, lse_parts=lse_parts)
        _check_buf("o_parts", o_parts, (total, B, T, n_h, hd), (torch.float32,))
        _check_buf("lse_parts", lse_parts, (total, B, T, n_h), (torch.float32,))
        self._srcs = (KvSource * len(descs))(*descs)
        self._keep = tuple(keep)
        self.o_parts, self.lse_parts = o_parts, lse_parts
        self._args = (_ptr(q), self._srcs, len(descs), _ptr(o_parts), _ptr(lse_parts), B, T,
                      n_h, hd, float(default_scale(hd) if scale is None else scale),
                      _stream_handle(stream))

    def __call__(self) -> Tuple[torch.Tensor, torch.Tensor]:
        st = _lib.fmha_mqa_fwd_sources_partials(*self._args)
        if st != 0:
            raise FmhaError("fmha_mqa_fwd_sources_partials", st)
        return self.o_parts, self.lse_parts


def fwd_sources_partials(q: torch.Tensor, sources, scale: Optional[float] = None,
                         o_parts: Optional[torch.Tensor] = None,
                         lse_parts: Optional[torch.Tensor] = None, stream=None
                         ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fmha_mqa_fwd_sources_partials: every source's split partials in one
    call (see SourcesPlan)."""
    return SourcesPlan(q, sources, scale, o_parts, lse_parts, stream)()


def fwd_sources(q: torch.Tensor, sources, scale: Optional[float] = None,
                out_dtype: torch.dtype = torch.bfloat16, sink: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention over the union of several key sources, e.g. top-k rows
    gathered from a compressed pool plus a dense sliding window.

    sources: sequence of (k, v, kv_idx, num_splits) — dense k, v [B, S, hd]
    with kv_idx None, or pools [P, hd] with kv_idx [B, T, S]; num_splits as
    for fwd.  One fmha_mqa_fwd_sources_partials call writes every source's
    split partials into its own planes of one fp32 buffer, and one
    fmha_lse_merge combines all planes; the sink (fp32 [n_h]) joins once,
    after the merge (fmha_attention_sink).  Returns (out [B, T, n_h, hd], lse
    [B, T, n_h]).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, T, n_h, hd]")
    B, T, n_h, hd = q.shape
    n = len(sources)
    if n < 1:
        raise ValueError("at least one key source is needed")
    dev = q.device
    _same_gpu(dev, sink=sink, out=out, lse=lse)
    if out is not None:
        _check_buf("out", out, (B, T, n_h, hd), (torch.float32, torch.bfloat16))
    if lse is not None:
        _check_buf("lse", lse, (B, T, n_h), (torch.float32,))
    rows = B * T * n_h
    parts, lse_parts = fwd_sources_partials(q, sources, scale, stream=stream)
    total = parts.shape[0]
    if out is None:
        out = torch.empty((B, T, n_h, hd), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, T, n_h), dtype=torch.float32, device=dev)
    lse_merge(parts.view(total, rows, hd), lse_parts.view(total, rows), out.dtype,
              out=out.view(rows, hd), lse=lse.view(rows), stream=stream)
    if sink is not None:
        apply_sink(out, lse, sink, stream=stream)
    return out, lse


def apply_sink(out: torch.Tensor, lse: torch.Tensor, sink: torch.Tensor, stream=None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fmha_attention_sink in place: out [..., n_h, hd] (fp32 or bf16) and lse
    [..., n_h] of finished rows; sink fp32 [n_h].  Returns (out, lse)."""
    if out.dim() < 2 or lse.shape != out.shape[:-1]:
        raise ValueError("out must be [..., n_h, hd] and lse [..., n_h]")
    n_h, hd = out.shape[-2], out.shape[-1]
    if sink.dtype != torch.float32 or sink.shape != (n_h,) or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 [n_h] tensor")
    if lse.dtype != torch.float32 or not (out.is_contiguous() and lse.is_contiguous()):
        raise ValueError("out and lse must be contiguous; lse float32")
    _same_gpu(out.device, lse=lse, sink=sink)
    st = _lib.fmha_attention_sink(_ptr(out), _ptr(lse), _ptr(sink), lse.numel(), n_h, hd,
                                  _dtype_code(out.dtype), _stream_handle(stream))
    if st != 0:
        raise FmhaError("fmha_attention_sink", st)
    return out, lse


def lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor,
              out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, stream=None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge fp32 partials o_parts [P, R, hd] / lse_parts [P, R] (natural log)."""
    if o_parts.dim() != 3 or lse_parts.shape != o_parts.shape[:2]:
        raise ValueError("o_parts must be [P, R, hd] and lse_parts [P, R]")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("partials must be float32")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("partials must be contiguous")
    P, R, hd = o_parts.shape
    dev = o_parts.device
    _same_gpu(dev, lse_parts=lse_parts, out=out, lse=lse)
    if out is not None:
        _check_buf("out", out, (R, hd), (torch.float32, torch.bfloat16))
    if lse is not None:
        _check_buf("lse", lse, (R,), (torch.float32,))
    if out is None:
        out = torch.empty((R, hd), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((R,), dtype=torch.float32, device=dev)
    st = _lib.fmha_lse_merge(_ptr(o_parts), _ptr(lse_parts), P, R, hd, _ptr(out),
                             _dtype_code(out.dtype), _ptr(lse), _stream_handle(stream))
    if st != 0:
        raise FmhaError("fmha_lse_merge", st)
    return out, lse


def index_scores(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor,
                 scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fmha_index_scores: q bf16 [B, T, H, c], k bf16 [P, c], w fp32 [B, T, H]
    -> scores fp32 [B, T, P]."""
    if q.dim() != 4 or k.dim() != 2 or k.shape[1] != q.shape[3] or w.shape != q.shape[:3]:
        raise ValueError("q must be [B, T, H, c], k [P, c] and w [B, T, H]")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or w.dtype != torch.float32:
        raise ValueError("q and k must be bfloat16, w float32")
    if not (q.is_contiguous() and k.is_contiguous() and w.is_contiguous()):
        raise ValueError("q, k and w must be contiguous")
    B, T, H, c = q.shape
    P = k.shape[0]
    _same_gpu(q.device, k=k, w=w, scores=scores)
    if scores is not None:
        _check_buf("scores", scores, (B, T, P), (torch.float32,))
    if scores is None:
        scores = torch.empty((B, T, P), dtype=torch.float32, device=q.device)
    st = _lib.fmha_index_scores(_ptr(q), _ptr(k), _ptr(w), _ptr(scores), B, T, H, c, P,
                                _stream_handle(stream))
    if st != 0:
        raise FmhaError("fmha_index_scores", st)
    return scores


def topk_select(scores: torch.Tensor, top_k: int, idx: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """fmha_topk_select over the last dim of fp32 scores [..., P] -> int32
    [..., top_k] (ascending ids, -1 padding)."""
    if scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be contiguous float32")
    if scores.dim() < 1:
        raise ValueError("scores must be [..., P]")
    P = scores.shape[-1]
    rows = scores.numel() // P if P else 0
    _same_gpu(scores.device, idx=idx)
    if idx is not None:
        _check_buf("idx", idx, (*scores.shape[:-1], top_k), (torch.int32,))
    if idx is None:
        idx = torch.empty((*scores.shape[:-1], top_k), dtype=torch.int32, device=scores.device)
    st = _lib.fmha_topk_select(_ptr(scores), _ptr(idx), rows, P, int(top_k),
                               _stream_handle(stream))
    if st != 0:
        raise FmhaError("fmha_topk_select", st)
    return idx


def indexer_topk(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, top_k: int,
                 stream=None) -> torch.Tensor:
    """kv_idx int32 [B, T, top_k] for fwd: the index scores, then the top-k."""
    return topk_select(index_scores(q, k, w, stream=stream), top_k, stream=stream)


def gather_floor(k: torch.Tensor, v: torch.Tensor, kv_idx: torch.Tensor,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fmha_gather_floor (a measurement helper): reads every gathered K and V
    row of pools k, v [P, hd] for kv_idx [B, T, s_k]; returns the per-token XOR
    of the words read, int32 [B, T] (the uint32 bit patterns)."""
    if k.dim() != 2 or v.shape != k.shape or kv_idx.dim() != 3:
        raise ValueError("k, v must be [P, hd] pools and kv_idx [B, T, s_k]")
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 or kv_idx.dtype != torch.int32:
        raise ValueError("k, v must be bfloat16 and kv_idx int32")
    if not (k.is_contiguous() and v.is_contiguous() and kv_idx.is_contiguous()):
        raise ValueError("k, v and kv_idx must be contiguous")
    B, T, s_k = kv_idx.shape
    _same_gpu(k.device, v=v, kv_idx=kv_idx, out=out)
    if out is not None:
        _check_buf("out", out, (B, T), (torch.int32,))
    if out is None:
        out = torch.empty((B, T), dtype=torch.int32, device=k.device)
    st = _lib.fmha_gather_floor(_ptr(k), _ptr(v), _ptr(kv_idx), _ptr(out), B, T, s_k, k.shape[1],
                                k.shape[0], _stream_handle(stream))
    if st != 0:
        raise FmhaError("fmha_gather_floor", st)
    return out


def read_floor(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, num_splits: int,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fmha_read_floor (a measurement helper): the split-KV whole-chunk
    kernel's reads of q [B, T, n_h, hd] and dense k, v [B, s_k, hd] with no
    arithmetic; returns one XOR word per workgroup (int32 bit patterns, in
    launch order tile + tiles * (b + B * split))."""
    if q.dim() != 4 or k.dim() != 3 or v.shape != k.shape or k.shape[0] != q.shape[0] \
            or k.shape[2] != q.shape[3]:
        raise ValueError("q must be [B, T, n_h, hd] and k, v [B, s_k, hd]")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous bfloat16")
    B, T, n_h, hd = q.shape
    s_k = k.shape[1]
    n_wg = -(-(T * n_h) // 128) * B * int(num_splits)
    _same_gpu(q.device, k=k, v=v, out=out)
    if out is not None:
        _check_buf("out", out, (n_wg,), (torch.int32,))
    else:
        out = torch.empty((n_wg,), dtype=torch.int32, device=q.device)
    st = _lib.fmha_read_floor(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, n_h, s_k, hd,
                              int(num_splits), _stream_handle(stream))
    if st != 0:
        raise FmhaError("fmha_read_floor", st)
    return out


def mfma_ceiling(ops: torch.Tensor, n_wg: int, iters: int,
                 sums: Optional[torch.Tensor] = None, clocks: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fmha_mfma_ceiling (a measurement helper): ops bf16 [8, 8, 64, 8] operand
    fragments; returns (sums fp32 [n_wg, 8, 4], clocks int64 [n_wg, 2]: shader
    cycles and 100 MHz ticks of each workgroup's loop)."""
    if ops.dtype != torch.bfloat16 or tuple(ops.shape) != (8, 8, 64, 8) or not ops.is_contiguous():
        raise ValueError("ops must be a contiguous bfloat16 [8, 8, 64, 8] tensor")
    dev = ops.device
    _same_gpu(dev, sums=sums, clocks=clocks)
    if sums is None:
        sums = torch.empty((n_wg, 8, 4), dtype=torch.float32, device=dev)
    if clocks is None:
        clocks = torch.empty((n_wg, 2), dtype=torch.int64, device=dev)
    _check_buf("sums", sums, (n_wg, 8, 4), (torch.float32,))
    _check_buf("clocks", clocks, (n_wg, 2), (torch.int64,))
    st = _lib.fmha_mfma_ceiling(_ptr(ops), _ptr(sums), _ptr(clocks), int(n_wg), int(iters),
                                _stream_handle(stream))
    if st != 0:
        raise FmhaError("fmha_mfma_ceiling", st)
    return sums, clocks


def raw_fwd(*args) -> int:
    """The C entry point itself, for tests of argument validation."""
    return int(_lib.fmha_mqa_fwd(*args))


def raw_merge(*args) -> int:
    return int(_lib.fmha_lse_merge(*args))
