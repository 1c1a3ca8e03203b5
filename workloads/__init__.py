"""Seeded synthetic inputs for the MQA attention forward.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path's tests/benchmark and the CPU oracle
receive the tensors it returns, so the two sides always see identical bf16 bits.

Workload shapes follow the dev-log pages of the DeepSeek-V4 NVFP4 kernel
project: page "May 24, 2026 — Session Start Plan", sections "Key Numbers"
(Pro decode: 128 query heads, top_k = s_k = 1024, 8 KV tiles of 128; one-head
test: s_k = 128, one tile) and "D1 Status Summary" (head dims 64/128/256); the
commit log of ``dsv4/kernels/cuda`` (pre-allocated compressed-KV pool of 32768
rows) for the sparse top-k pool size.

Recipe (fixed here, used everywhere):
  * ``torch.Generator`` on the CPU seeded with ``1000 + config_id``;
  * fp32 ``randn`` drawn in the order q, k, v (then the index lists);
  * multiplied by the config's ``scale_in`` (0.5 for the MQA prefill shape);
  * rounded to bf16 with round-to-nearest-even (torch's ``.to(bfloat16)``);
  * top-k index lists: for every (b, t) ``randperm(pool)[:s_k]`` as int32,
    i.e. s_k distinct rows drawn uniformly from one pool, unsorted.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "make_custom"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-forward problem.

    Rows of the output are (b, t, h); all query heads of a batch (dense) or of a
    token (gather) share one K/V head.
    """

    cid: int                  # config id (also selects the seed)
    name: str
    B: int
    T: int
    n_h: int
    hd: int
    s_k: int                  # keys each row attends to (top_k when gathering)
    out_dtype: str            # "f32" or "bf16"
    num_splits: int = 1       # split-KV chunks (1 = single pass)
    scale_in: float = 1.0     # multiplier applied to the N(0,1) draws
    pool: int = 0             # > 0: K/V are pools of this many rows + kv_idx
    seed_override: Optional[int] = None

    @property
    def seed(self) -> int:
        return 1000 + self.cid if self.seed_override is None else self.seed_override

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(hd), as the fp32 value the kernel receives."""
        return float(torch.tensor(1.0 / math.sqrt(self.hd), dtype=torch.float32))

    @property
    def gather(self) -> bool:
        return self.pool > 0

    @property
    def rows(self) -> int:
        return self.B * self.T * self.n_h

    @property
    def flops(self) -> int:
        """QK^T plus P.V multiply-adds, 2 flops each (exp not counted)."""
        return 4 * self.rows * self.s_k * self.hd

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move once: Q, K, V (+ index) in; O, LSE out.

        Dense: K/V counted once per batch.  Gather: every selected row counted
        once per token (the gathered volume), plus the int32 index list.
        """
        out_b = 4 if self.out_dtype == "f32" else 2
        q = self.rows * self.hd * 2
        if self.gather:
            kv = 2 * self.B * self.T * self.s_k * self.hd * 2
            idx = self.B * self.T * self.s_k * 4
        else:
            kv = 2 * self.B * self.s_k * self.hd * 2
            idx = 0
        return q + kv + idx + self.rows * self.hd * out_b + self.rows * 4

    def describe(self) -> str:
        s = (f"{self.name} B={self.B} T={self.T} n_h={self.n_h} hd={self.hd} "
             f"s_k={self.s_k}")
        if self.gather:
            s += f" pool={self.pool}"
        if self.num_splits > 1:
            s += f" splits={self.num_splits}"
        return s + f" out={self.out_dtype}"


WORKLOADS = {
    1: Workload(1, "single_head_decode", B=1, T=1, n_h=1, hd=64, s_k=128,
                out_dtype="f32"),
    2: Workload(2, "single_head_prefill", B=1, T=128, n_h=1, hd=128, s_k=256,
                out_dtype="f32"),
    3: Workload(3, "mqa_decode", B=32, T=1, n_h=128, hd=256, s_k=1024,
                out_dtype="bf16", num_splits=8),
    4: Workload(4, "mqa_prefill", B=2, T=4096, n_h=64, hd=128, s_k=1024,
                out_dtype="bf16", scale_in=0.5),
    5: Workload(5, "sparse_topk", B=4, T=512, n_h=128, hd=128, s_k=1024,
                out_dtype="bf16", pool=32768),
}


def get(cid: int) -> Workload:
    return WORKLOADS[cid]


def make_custom(B, T, n_h, hd, s_k, out_dtype="f32", num_splits=1, pool=0,
                scale_in=1.0, seed=0, name="custom") -> Workload:
    """A workload with arbitrary sizes (tests sweep these)."""
    return Workload(cid=0, name=name, B=B, T=T, n_h=n_h, hd=hd,
                    s_k=s_k, out_dtype=out_dtype, num_splits=num_splits,
                    scale_in=scale_in, pool=pool, seed_override=seed)


def _randn_bf16(g: torch.Generator, shape, scale_in: float) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if scale_in != 1.0:
        x = x * scale_in
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, seed: Optional[int] = None):
    """Return CPU tensors ``(q, k, v, kv_idx)`` for workload ``w``.

    q: bf16 [B, T, n_h, hd]; k, v: bf16 [B, s_k, hd] (dense) or [pool, hd]
    (gather); kv_idx: int32 [B, T, s_k] or None.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    q = _randn_bf16(g, (w.B, w.T, w.n_h, w.hd), w.scale_in)
    if w.gather:
        k = _randn_bf16(g, (w.pool, w.hd), w.scale_in)
        v = _randn_bf16(g, (w.pool, w.hd), w.scale_in)
        if w.s_k > w.pool:
            raise ValueError("top-k larger than the pool")
        idx = torch.empty((w.B, w.T, w.s_k), dtype=torch.int32)
        flat = idx.view(-1, w.s_k)
        for r in range(flat.shape[0]):
            flat[r] = torch.randperm(w.pool, generator=g)[: w.s_k].to(torch.int32)
        return q, k, v, idx
    k = _randn_bf16(g, (w.B, w.s_k, w.hd), w.scale_in)
    v = _randn_bf16(g, (w.B, w.s_k, w.hd), w.scale_in)
    return q, k, v, None
