"""Benchmark of the MQA attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path, each part on its own batch of
seeded synthetic input already resident in HBM:
  * mqa_prefill  B=2 T=4096 n_h=64 hd=128 s_k=1024 (bf16 out)  — the headline:
    attention TFLOP/s against the bf16 dense MFMA peak;
  * mqa_decode   B=32 T=1 n_h=128 hd=256 s_k=1024, 8-way split-KV + LSE merge
    (bf16 out) — HBM GB/s of algorithmic bytes against the HBM peak;
  * sparse_topk  B=4 T=512 n_h=128 hd=128, 1024 of 32768 pool rows gathered per
    token (bf16 out) — TFLOP/s and gathered GB/s.
Clocks are first brought to steady state with ~1 s of untimed cache flushes and
prefill calls, and each workload first runs ~0.5 s of untimed flush + call pairs
(the timed pattern) and its warm-up calls.  Each call is timed with its own pair of HIP events on the launch stream, with
L2 and the memory-side cache flushed (a read-only sweep of 512 MiB) before every
timed call, so every call reads its inputs from HBM.  Back-to-back ("warm") times are
reported beside them.  Rank 0 prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
FLUSH_BYTES = 512 << 20

# Sources the committed HBM traffic counters were taken on: every HIP source
# and header of the library (the ABI layer picks tile shapes and partial
# formats, so it can change the traffic too).  A changed source makes those
# counters stale and the traffic field null.
CSRC_DIR = os.path.join(ROOT, "fmha_mqa_fwd_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.relpath(os.path.join(CSRC_DIR, f), ROOT)
                        for f in os.listdir(CSRC_DIR) if f.endswith((".hip", ".h")))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# which attention kernels (by demangled name) serve each workload
WORKLOAD_KERNEL_SIG = {
    "mqa_prefill": lambda k: "fwd_kernel<128" in k and ", false," in k,
    "mqa_decode": lambda k: "chunk_kernel" in k or "merge_kernel" in k,
    "sparse_topk": lambda k: "fwd_gather_staged_kernel<128" in k,
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str):
    """Per-launch HBM bytes (FETCH+WRITE, copy-calibrated) for `workload` from
    the committed counter file, or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = rec.get("workloads", {}).get(workload)
    return None if ent is None else ent.get("bytes_per_launch")


def committed_kernel_stats(workload: str):
    """Effective clock / matrix-unit busy share of `workload`'s attention
    kernel from the committed counter file ({} when absent or stale)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return {}
    sig = WORKLOAD_KERNEL_SIG[workload]
    out = {}
    for k, v in rec.get("kernels", {}).items():
        if sig(k) and "merge_kernel" not in k:
            for key in ("effective_clock_GHz", "mfma_busy_frac", "lds_busy_frac",
                        "lds_bank_conflict_frac", "valu_active_frac", "mfma_valu_coexec_frac"):
                if key in v:
                    out[key] = v[key]
    return out


CASES = (("mqa_prefill", 4), ("mqa_decode", 3), ("sparse_topk", 5))
COPY_BYTES = 256 << 20   # calibration copy: reads and writes this many bytes


class Case:
    """One workload's inputs and outputs resident on the GPU; calling it
    launches the forward once.  `wl` is a config id or a Workload; `sink`
    optionally joins an attention sink of that many heads."""

    def __init__(self, wl, dev, sink=False):
        import fmha_mqa_fwd_amd as F

        self.F = F
        self.w = W.get(wl) if isinstance(wl, int) else wl
        q, k, v, idx = W.make_inputs(self.w)
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        self.idx = None if idx is None else idx.to(dev)
        self.out_dtype = torch.float32 if self.w.out_dtype == "f32" else torch.bfloat16
        w = self.w
        self.out = torch.empty((w.B, w.T, w.n_h, w.hd), dtype=self.out_dtype, device=dev)
        self.lse = torch.empty((w.B, w.T, w.n_h), dtype=torch.float32, device=dev)
        nb = F.workspace_bytes(w.B, w.T, w.n_h, w.hd, w.num_splits)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        self.sink = None
        if sink:
            g = torch.Generator().manual_seed(7)
            self.sink = (torch.randn(w.n_h, generator=g) * 2.0).to(dev)
        # arguments marshalled once: a timed call is the C launch itself
        self.plan = F.FwdPlan(self.q, self.k, self.v, self.idx, scale=w.scale,
                              out_dtype=self.out_dtype, num_splits=w.num_splits,
                              out=self.out, lse=self.lse, workspace=self.ws, sink=self.sink)

    def __call__(self):
        self.plan()


class FloorCase:
    """The gather-only floor of a gather workload: fmha_gather_floor reads the
    same K/V rows for the same index lists with no attention arithmetic."""

    def __init__(self, case):
        self.F = case.F
        self.k, self.v, self.idx = case.k, case.v, case.idx
        w = case.w
        self.out = torch.empty((w.B, w.T), dtype=torch.int32, device=case.k.device)
        self.bytes = 2 * w.B * w.T * w.s_k * w.hd * 2  # K and V rows, gathered

    def __call__(self):
        self.F.gather_floor(self.k, self.v, self.idx, out=self.out)


class ReadFloorCase:
    """The read floor of a dense split-KV workload: fmha_read_floor reads the
    bytes the split kernel reads (its q rows and its split's K/V rows), with
    the same workgroups and no arithmetic."""

    def __init__(self, case):
        self.F = case.F
        self.q, self.k, self.v = case.q, case.k, case.v
        w = case.w
        self.splits = w.num_splits
        n_wg = -(-(w.T * w.n_h) // 128) * w.B * w.num_splits
        self.out = torch.empty((n_wg,), dtype=torch.int32, device=case.q.device)
        self.bytes = w.rows * w.hd * 2 + 2 * w.B * w.s_k * w.hd * 2   # q once, K and V once

    def __call__(self):
        self.F.read_floor(self.q, self.k, self.v, self.splits, out=self.out)


MFMA_ITERS = 20000   # ~2.5-3.5 ms per launch: long enough for the clock to settle


def mfma_ceiling(dev, reps=20):
    """Sustained bf16 matrix-core rate on random operands (fmha_mfma_ceiling,
    one 8-wave workgroup per CU): median TFLOP/s over `reps` launches and the
    median effective shader clock read in the kernel."""
    import fmha_mqa_fwd_amd as F

    g = torch.Generator().manual_seed(11)
    ops = torch.randn(8, 8, 64, 8, generator=g).to(torch.bfloat16).to(dev)
    n_wg = torch.cuda.get_device_properties(dev).multi_processor_count
    flops = n_wg * 8 * 4 * MFMA_ITERS * 32768
    sums = torch.empty((n_wg, 8, 4), dtype=torch.float32, device=dev)
    clocks = torch.empty((n_wg, 2), dtype=torch.int64, device=dev)
    for _ in range(5):
        F.mfma_ceiling(ops, n_wg, MFMA_ITERS, sums=sums, clocks=clocks)
    torch.cuda.synchronize()
    ts, ghz = [], []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        F.mfma_ceiling(ops, n_wg, MFMA_ITERS, sums=sums, clocks=clocks)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
        c = clocks.cpu().double()
        ghz.append(float((c[:, 0] / c[:, 1]).median()) * 0.1)
    ts.sort()
    ghz.sort()
    return {"TFLOPs": flops / ts[len(ts) // 2] / 1e12, "clock_GHz": ghz[len(ghz) // 2],
            "workgroups": n_wg, "us_per_launch": ts[len(ts) // 2] * 1e6}


class SourcesCase:
    """Decode over two key sources — top-k rows gathered from a compressed
    pool plus a dense sliding window — in one softmax: one
    fmha_mqa_fwd_sources_partials call writes both sources' split partials
    into planes of one fp32 buffer (at hd 512, one launch), then one LSE merge
    over all planes (the composition fwd_sources runs), with every launch's
    arguments marshalled once."""

    def __init__(self, dev, B=32, n_h=64, hd=512, top_k=512, pool=32768, window=128,
                 splits=(4, 1)):
        import fmha_mqa_fwd_amd as F

        top = W.make_custom(B=B, T=1, n_h=n_h, hd=hd, s_k=top_k, pool=pool, out_dtype="bf16",
                            seed=3001, name="topk_source")
        win = W.make_custom(B=B, T=1, n_h=1, hd=hd, s_k=window, out_dtype="bf16", seed=3002,
                            name="window_source")
        q, kp, vp, idx = W.make_inputs(top)
        _, kw, vw, _ = W.make_inputs(win)
        self.q, kp, vp, idx, kw, vw = (t.to(dev) for t in (q, kp, vp, idx, kw, vw))
        self._keep = (kp, vp, idx, kw, vw)
        rows = B * n_h
        n_parts = splits[0] + splits[1]
        self.parts = torch.empty((n_parts, B, 1, n_h, hd), dtype=torch.float32, device=dev)
        self.lse_parts = torch.empty((n_parts, B, 1, n_h), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, 1, n_h, hd), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, 1, n_h), dtype=torch.float32, device=dev)
        # one token per sequence leaves a source's rows few: split its keys so
        # that each launch fills the chip; every split's partial goes to the
        # one merge
        srcs = [(kp, vp, idx, splits[0]), (kw, vw, None, splits[1])]
        self.plans = [F.SourcesPlan(self.q, srcs, scale=top.scale, o_parts=self.parts,
                                    lse_parts=self.lse_parts)]
        lib = F._binding._lib
        self._merge = lib.fmha_lse_merge
        self._margs = (self.parts.data_ptr(), self.lse_parts.data_ptr(), n_parts, rows, hd,
                       self.out.data_ptr(), F.FMHA_BF16, self.lse.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
        # bytes the method must move once: Q, gathered top-k K/V rows (+ idx),
        # window K/V, bf16 O and lse
        self.bytes = (rows * hd * 2 + 2 * B * top_k * hd * 2 + B * top_k * 4
                      + 2 * B * window * hd * 2 + rows * hd * 2 + rows * 4)
        self.flops = 4 * rows * (top_k + window) * hd
        self.desc = (f"decode over two sources: B={B} T=1 n_h={n_h} hd={hd}, top-k {top_k} of "
                     f"{pool} pool rows ({splits[0]} splits) + {window}-key window ({splits[1]} "
                     f"splits), bf16 out")

    def __call__(self):
        for plan in self.plans:
            plan()
        st = self._merge(*self._margs)
        if st != 0:
            raise RuntimeError(f"fmha_lse_merge failed: status {st}")


class IndexerCase:
    """The top-k indexer at the sparse top-k config's shape (B=4, T=512, a
    32768-entry pool, top-k 1024) with 64 index heads of width 128: `part`
    'scores' times fmha_index_scores, 'select' times fmha_topk_select on the
    scores it produced."""

    def __init__(self, dev, part, B=4, T=512, H=64, c=128, P=32768, top_k=1024):
        import fmha_mqa_fwd_amd as F

        g = torch.Generator().manual_seed(4001)
        self.q = torch.randn(B, T, H, c, generator=g).to(torch.bfloat16).to(dev)
        self.k = torch.randn(P, c, generator=g).to(torch.bfloat16).to(dev)
        self.w = (torch.rand(B, T, H, generator=g) * 2 - 1).to(dev)
        self.scores = torch.empty((B, T, P), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B, T, top_k), dtype=torch.int32, device=dev)
        self.F, self.part, self.top_k = F, part, top_k
        F.index_scores(self.q, self.k, self.w, scores=self.scores)
        tokens = B * T
        if part == "scores":
            self.flops = 2 * tokens * H * c * P
            self.bytes = tokens * H * c * 2 + P * c * 2 + tokens * H * 4 + tokens * P * 4
        else:
            self.flops = 0
            self.bytes = tokens * P * 4 + tokens * top_k * 4
        self.desc = (f"top-k indexer {part}: {tokens} tokens, {H} index heads x {c}, "
                     f"{P}-entry pool, top-k {top_k}")

    def __call__(self):
        if self.part == "scores":
            self.F.index_scores(self.q, self.k, self.w, scores=self.scores)
        else:
            self.F.topk_select(self.scores, self.top_k, idx=self.idx)


RAMP_SECONDS = 0.5  # untimed flush + call pairs before each workload's warm-up


def ramp(case, flush_buf, seconds=RAMP_SECONDS):
    """Untimed (cache flush, call) pairs for `seconds`: the pattern the timed
    loop runs.  Measured on MI355X, the first ~100 flushed prefill calls after
    back-to-back work or an idle host gap run up to 15% slower (310 us falling
    to 269.5 us) while the memory-side clocks settle."""
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            untimed_flush(flush_buf)
            case()
        torch.cuda.synchronize()


def untimed_flush(flush_buf):
    """The same 512 MiB read-only sweep as the timed loop's flush, by another
    reduction (max instead of sum), so that a kernel trace tells the timed
    calls (after a sum) from the ramp and warm-up calls (after a max)."""
    flush_buf.amax()


def time_case(case, steps, warmup, flush_buf):
    """Mean per-call time in ms: flushed (events around each call, cache
    flushed before it) and warm (events around `steps` back-to-back calls).
    The `warmup` untimed calls follow the same flush + call pattern, after the
    clock ramp of `ramp`."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    # torch creates the HIP event at its first record: do that now, not
    # inside the timed loop
    for ev in starts + ends:
        ev.record()
    torch.cuda.synchronize()
    ramp(case, flush_buf)
    for _ in range(warmup):
        untimed_flush(flush_buf)
        case()
    torch.cuda.synchronize()
    for i in range(steps):
        # read-only sweep: evicts L2/MALL (and writes back the previous call's
        # dirty output) before the timed call instead of leaving dirty lines
        # that drain inside it
        flush_buf.sum()
        starts[i].record()
        case()
        ends[i].record()
    torch.cuda.synchronize()
    flushed = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        case()
    e1.record()
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) / steps
    flushed.sort()
    return {"ms": sum(flushed) / len(flushed), "ms_median": flushed[len(flushed) // 2],
            "ms_p10": flushed[len(flushed) // 10], "ms_p90": flushed[(9 * len(flushed)) // 10],
            "ms_warm": warm}


def profile_mode(args, dev):
    """Runs one workload `warmup + steps` times back to back (and, with
    --copy-calibration, `steps` plain copies of COPY_BYTES) for a profiler."""
    names = [n for n, _ in CASES] if args.only == "all" else [args.only]
    for name in names:
        case = Case(dict(CASES)[name], dev)
        for _ in range(args.warmup + args.steps):
            case()
        torch.cuda.synchronize()
        del case
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] profile mode done: {args.only} x{args.warmup + args.steps}",
          file=sys.stderr, flush=True)


def _counter_rows(d):
    """(kernel name, counter name, value) per dispatch from a rocprofv3 --pmc
    output directory (its *counter_collection.csv)."""
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    out = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                dur = None
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
                out.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]),
                            r.get("Dispatch_Id"), dur))
    return out


N_XCD = 8          # GRBM_GUI_ACTIVE reads summed over the XCDs
N_SIMD = 1024      # 256 CUs x 4 SIMDs


def _busy_counters(d):
    """Per fmha kernel (median dispatch): effective shader clock
    (GRBM_GUI_ACTIVE / XCDs / dispatch duration) and the share of SIMD cycles
    the matrix units were busy (SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x
    GRBM_GUI_ACTIVE / XCDs))."""
    by = {}
    for kname, cn, val, disp, dur in _counter_rows(d):
        if "fmha" in kname:
            by.setdefault(kname, {}).setdefault(disp, {})[cn] = val
            by[kname][disp]["_dur"] = dur
    res = {}
    for k, disps in by.items():
        clk, mfma, flops = [], [], []
        for c in disps.values():
            g = c.get("GRBM_GUI_ACTIVE")
            # the dispatch timestamps are too coarse for short kernels
            if g and c.get("_dur") and c["_dur"] > 50e-6:
                clk.append(g / N_XCD / c["_dur"] / 1e9)
                if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                    mfma.append(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * g / N_XCD))
            if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
                # bf16 matrix FLOPs the dispatch executed (512 per counted op)
                flops.append(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512)
        if clk or flops:
            res[k] = {}
            if clk:
                res[k]["effective_clock_GHz"] = round(sorted(clk)[len(clk) // 2], 3)
            if mfma:
                res[k]["mfma_busy_frac"] = round(sorted(mfma)[len(mfma) // 2], 4)
            if flops:
                res[k]["mfma_flops_per_launch"] = sorted(flops)[len(flops) // 2]
    return res


N_CU = 256         # compute units


def _pipe_counters(d):
    """Per fmha kernel (median dispatch), from a run of GRBM_GUI_ACTIVE,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_VALU_MFMA_COEXEC_CYCLES, SQ_LDS_IDX_ACTIVE,
    SQ_LDS_BANK_CONFLICT, SQ_ACTIVE_INST_VALU, SQ_INSTS_LDS, SQ_INSTS_VALU:
    the share of CU cycles the LDS is busy with indexed accesses and the
    share of those stalled by bank conflicts; the SIMD cycles with vector
    instructions active (SQ_ACTIVE_INST_VALU counts quad-cycles); the share of
    matrix-busy cycles in which vector instructions execute too; LDS and
    vector instructions per dispatch."""
    by = {}
    for kname, cn, val, disp, _ in _counter_rows(d):
        if "fmha" in kname:
            by.setdefault(kname, {}).setdefault(disp, {})[cn] = val
    res = {}
    for k, disps in by.items():
        cols = {}
        for c in disps.values():
            g = c.get("GRBM_GUI_ACTIVE")
            if not g:
                continue
            cyc = g / N_XCD
            if "SQ_LDS_IDX_ACTIVE" in c:
                cols.setdefault("lds_busy_frac", []).append(c["SQ_LDS_IDX_ACTIVE"] / (N_CU * cyc))
                if c["SQ_LDS_IDX_ACTIVE"]:
                    cols.setdefault("lds_bank_conflict_frac", []).append(
                        c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_LDS_IDX_ACTIVE"])
            if "SQ_ACTIVE_INST_VALU" in c:
                cols.setdefault("valu_active_frac", []).append(
                    4 * c["SQ_ACTIVE_INST_VALU"] / (N_SIMD * cyc))
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
                cols.setdefault("mfma_busy_frac", []).append(
                    c["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc))
                if "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
                    cols.setdefault("mfma_valu_coexec_frac", []).append(
                        c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"])
            for key, cn in (("lds_insts", "SQ_INSTS_LDS"), ("valu_insts", "SQ_INSTS_VALU")):
                if cn in c:
                    cols.setdefault(key, []).append(c[cn])
        if cols:
            res[k] = {key: round(sorted(v)[len(v) // 2], 4 if "frac" in key else 0)
                      for key, v in cols.items()}
    return res


def ingest_counters(fetch_dir, write_dir, busy_dir=None, pipe_dir=None):
    """Per-launch HBM bytes of each attention kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a plain copy of COPY_BYTES (expected COPY_BYTES/1024 KiB each way);
    with busy_dir (a GRBM_GUI_ACTIVE + SQ_VALU_MFMA_BUSY_CYCLES run), also the
    effective clock and matrix-unit busy share of each kernel; with pipe_dir
    (see _pipe_counters), the LDS, vector and co-execution shares."""
    rec = {"kernel_source_hash": kernel_source_hash(), "copy_bytes": COPY_BYTES,
           "workloads": {}, "kernels": {}}
    scale = {}
    per_kernel = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        sums = {}
        for kname, cn, val, disp, _ in _counter_rows(d):
            if cn != cname:
                continue
            sums.setdefault(kname, []).append(val)
        copies = [v for k, vs in sums.items()
                  if "copy" in k.lower() and "fill" not in k.lower() for v in vs]
        if not copies:
            raise SystemExit(f"no copy-kernel dispatch found in {d}")
        copy_kib = sorted(copies)[len(copies) // 2]
        scale[cname] = (COPY_BYTES / 1024.0) / copy_kib
        for k, vs in sums.items():
            if "fmha" in k:
                per_kernel.setdefault(k, {})[cname] = sorted(vs)[len(vs) // 2]
    for k, c in per_kernel.items():
        kib_f, kib_w = c.get("FETCH_SIZE", 0.0), c.get("WRITE_SIZE", 0.0)
        rec["kernels"][k] = {
            "fetch_kib_raw": kib_f, "write_kib_raw": kib_w,
            "bytes_per_launch": kib_f * 1024 * scale["FETCH_SIZE"] + kib_w * 1024 * scale["WRITE_SIZE"]}
    rec["copy_scale"] = scale
    if busy_dir:
        for k, b in _busy_counters(busy_dir).items():
            rec["kernels"].setdefault(k, {}).update(b)
    if pipe_dir:
        for k, b in _pipe_counters(pipe_dir).items():
            ent = rec["kernels"].setdefault(k, {})
            if "mfma_busy_frac" in ent:   # the busy run's figure stays the reported one
                b.pop("mfma_busy_frac", None)
            ent.update(b)
    # map kernels to workloads: the attention kernel with the largest traffic
    # of each workload's run is recorded by its template signature
    for name, _ in CASES:
        sig = WORKLOAD_KERNEL_SIG.get(name)
        tot = sum(v.get("bytes_per_launch", 0) for k, v in rec["kernels"].items() if sig and sig(k))
        if tot:
            rec["workloads"][name] = {"bytes_per_launch": tot}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def copy_ceiling(dev, nbytes=1 << 30, reps=10):
    """Practical HBM ceiling: a plain device-to-device copy of `nbytes`
    (read + write bytes per second, median of `reps`)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * nbytes / sorted(ts)[len(ts) // 2] / 1e9


def trace_summary(trace_csv):
    """Markdown table of per-kernel durations from a rocprofv3 --kernel-trace
    CSV of a bench.py run: all dispatches, and the timed flushed calls alone
    (each dispatch that directly follows the timed loop's cache-flush sum; the
    ramp and warm-up flushes are a max reduction)."""
    import csv

    with open(trace_csv) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    allk, flushed = {}, {}
    prev = None
    for r in rows:
        name = r["Kernel_Name"]
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        allk.setdefault(name, []).append(us)
        if (prev is not None and "reduce_kernel" in prev["Kernel_Name"]
                and "sum_functor" in prev["Kernel_Name"] and "reduce_kernel" not in name):
            flushed.setdefault(name, []).append(us)
        prev = r

    def short(n):
        n = n.replace("void fmha::(anonymous namespace)::", "").split("(fmha::")[0]
        return n.split("(float const*")[0][:70]

    lines = ["| kernel | dispatches | avg us | min us | max us | flushed calls | flushed avg us |",
             "|---|---|---|---|---|---|---|"]
    for name, v in sorted(allk.items(), key=lambda kv: -sum(kv[1])):
        if "fmha" not in name and "copyBuffer" not in name:
            continue
        fl = flushed.get(name, [])
        fl_avg = f"{sum(fl) / len(fl):.1f}" if fl else "-"
        lines.append(f"| `{short(name)}` | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | "
                     f"{max(v):.1f} | {len(fl)} | {fl_avg} |")
    return "\n".join(lines)


def cpu_baseline(budget_s=12.0):
    """The float64 oracle on a bounded sample of the prefill workload's rows,
    on this host's cores; returns its attention TFLOP/s."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    w = W.get(4)
    q, k, v, idx = W.make_inputs(w)
    rng = np.random.default_rng(0)
    oracle.attention(q, k, v, w.scale, rows=np.arange(1024))       # warm the BLAS pool
    n = 16384
    t = time.perf_counter()
    oracle.attention(q, k, v, w.scale, rows=rng.choice(w.rows, n, replace=False))
    dt = time.perf_counter() - t
    n = int(min(w.rows, max(n, n * budget_s / max(dt, 1e-3))))
    rows = rng.choice(w.rows, n, replace=False)
    t = time.perf_counter()
    oracle.attention(q, k, v, w.scale, rows=rows)
    dt = time.perf_counter() - t
    flops = 4.0 * n * w.s_k * w.hd
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {w.rows} rows of {w.describe()} (float64 numpy), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=[n for n, _ in CASES] + ["all"],
                    help="profile mode: run one workload back to back, no JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="profile mode: also run a plain device copy of known size")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print per-kernel durations (all / flushed calls) of a "
                         "rocprofv3 --kernel-trace run of bench.py")
    ap.add_argument("--ingest-counters", nargs="+", metavar="DIR",
                    help="FETCH_DIR WRITE_DIR [BUSY_DIR [PIPE_DIR]]: turn rocprofv3 --pmc "
                         "runs (FETCH_SIZE; WRITE_SIZE; GRBM_GUI_ACTIVE + "
                         "SQ_VALU_MFMA_BUSY_CYCLES; the LDS/vector/co-execution counters of "
                         "_pipe_counters) of --only ... --copy-calibration into "
                         + TRAFFIC_FILE)
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.ingest_counters:
        if len(args.ingest_counters) not in (2, 3, 4):
            ap.error("--ingest-counters takes FETCH_DIR WRITE_DIR [BUSY_DIR [PIPE_DIR]]")
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention shards by batch/token with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.only:
        profile_mode(args, dev)
        return
    flush_buf = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
    # load both flush reductions now: the first use of a kernel stalls the GPU
    # for ~25 ms, and after such a gap the next calls ran up to 30% slower
    flush_buf.sum()
    untimed_flush(flush_buf)
    torch.cuda.synchronize()

    # Bring clocks to steady state before anything is timed: ~1 s of untimed
    # cache flushes and prefill calls (then each workload's own ramp).
    warm = Case(4, dev)
    ramp(warm, flush_buf, 1.0)
    del warm
    torch.cuda.empty_cache()

    res = {}
    for name, cid in CASES:
        case = Case(cid, dev)
        t = time_case(case, args.steps, args.warmup, flush_buf)
        w = case.w
        t["flops"] = w.flops
        t["bytes"] = w.algorithmic_bytes()
        t["tflops"] = w.flops / (t["ms"] * 1e-3) / 1e12
        t["gbps"] = w.algorithmic_bytes() / (t["ms"] * 1e-3) / 1e9
        t["workload"] = w.describe()
        res[name] = t
        print(f"[bench] {name}: {t['ms'] * 1e3:.1f} us/call flushed "
              f"({t['ms_warm'] * 1e3:.1f} warm), {t['tflops']:.1f} TFLOP/s, "
              f"{t['gbps']:.0f} GB/s", file=sys.stderr, flush=True)
        if name == "mqa_decode":
            # the split kernel's reads alone: its q rows and its split's K/V rows
            fl = ReadFloorCase(case)
            tf = time_case(fl, args.steps, args.warmup, flush_buf)
            t["read_floor_ms"], t["read_floor_ms_warm"] = tf["ms"], tf["ms_warm"]
            t["read_floor_gbps"] = fl.bytes / (tf["ms"] * 1e-3) / 1e9
            print(f"[bench] {name} read floor: {tf['ms'] * 1e3:.1f} us/call flushed "
                  f"({tf['ms_warm'] * 1e3:.1f} warm), {t['read_floor_gbps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
            del fl
        if case.idx is not None:
            # the memory side's floor for the same gathered rows
            fl = FloorCase(case)
            tf = time_case(fl, args.steps, args.warmup, flush_buf)
            t["floor_ms"], t["floor_ms_warm"] = tf["ms"], tf["ms_warm"]
            t["floor_gbps"] = fl.bytes / (tf["ms"] * 1e-3) / 1e9
            print(f"[bench] {name} gather-only floor: {tf['ms'] * 1e3:.1f} us/call flushed "
                  f"({tf['ms_warm'] * 1e3:.1f} warm), {t['floor_gbps']:.0f} GB/s gathered",
                  file=sys.stderr, flush=True)
            del fl
        del case
        torch.cuda.empty_cache()

    # the two correctness configs (one KV tile; two KV tiles of one head):
    # launch-latency bound, reported as time per call only
    small = {}
    for name, cid in (("single_head_decode", 1), ("single_head_prefill", 2)):
        case = Case(cid, dev)
        t = time_case(case, args.steps, args.warmup, flush_buf)
        small[name] = {"us_per_call": round(t["ms"] * 1e3, 2),
                       "us_median": round(t["ms_median"] * 1e3, 2),
                       "us_per_call_warm": round(t["ms_warm"] * 1e3, 2),
                       "workload": case.w.describe()}
        print(f"[bench] {name}: {small[name]['us_per_call']:.1f} us/call flushed "
              f"({small[name]['us_per_call_warm']:.1f} warm)", file=sys.stderr, flush=True)
        del case

    # the widened rows: head dim 512 (decode split and Flash top-k), the
    # attention sink fused into decode, attention over two key sources
    nxt = {}
    nxt_cases = (
        ("hd512_decode", lambda: Case(W.make_custom(B=32, T=1, n_h=128, hd=512, s_k=1024,
                                                    out_dtype="bf16", num_splits=4, seed=2001,
                                                    name="hd512_decode"), dev)),
        ("hd512_flash_topk", lambda: Case(W.make_custom(B=4, T=512, n_h=64, hd=512, s_k=512,
                                                        pool=32768, out_dtype="bf16", seed=2002,
                                                        name="hd512_flash_topk"), dev)),
        ("decode_sink", lambda: Case(3, dev, sink=True)),
        ("two_source_decode", lambda: SourcesCase(dev)),
        ("indexer_scores", lambda: IndexerCase(dev, "scores")),
        ("indexer_select", lambda: IndexerCase(dev, "select")),
    )
    for name, make in nxt_cases:
        case = make()
        t = time_case(case, args.steps, args.warmup, flush_buf)
        floor = None
        if isinstance(case, Case) and case.idx is not None:
            fl = FloorCase(case)
            floor = time_case(fl, args.steps, args.warmup, flush_buf)
            floor["gbps"] = fl.bytes / (floor["ms"] * 1e-3) / 1e9
            del fl
        if isinstance(case, (SourcesCase, IndexerCase)):
            flops, nbytes, desc = case.flops, case.bytes, case.desc
        else:
            flops, nbytes, desc = case.w.flops, case.w.algorithmic_bytes(), case.w.describe()
        ent = {"us_per_call": round(t["ms"] * 1e3, 2), "us_per_call_warm": round(t["ms_warm"] * 1e3, 2),
               "TFLOPs": round(flops / (t["ms"] * 1e-3) / 1e12, 2),
               "GBps": round(nbytes / (t["ms"] * 1e-3) / 1e9, 1), "workload": desc}
        ent["frac_of_mfma_peak"] = round(ent["TFLOPs"] / PEAK_BF16_TFLOPS, 4)
        ent["frac_of_hbm_peak"] = round(ent["GBps"] / PEAK_HBM_GBPS, 4)
        if floor is not None:
            # the gather-only floor of the same index lists (fmha_gather_floor)
            ent["gather_floor_us"] = round(floor["ms"] * 1e3, 2)
            ent["gather_floor_GBps"] = round(floor["gbps"], 1)
            ent["floor_over_call"] = round(floor["ms"] / t["ms"], 4)
        nxt[name] = ent
        print(f"[bench] {name}: {ent['us_per_call']:.1f} us/call flushed, {ent['TFLOPs']:.1f} "
              f"TFLOP/s, {ent['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
        del case
        torch.cuda.empty_cache()

    copy_gbps = copy_ceiling(dev)
    print(f"[bench] device copy: {copy_gbps:.0f} GB/s (read + write)", file=sys.stderr, flush=True)
    mc = mfma_ceiling(dev)
    print(f"[bench] sustained bf16 MFMA on random operands: {mc['TFLOPs']:.0f} TFLOP/s at "
          f"{mc['clock_GHz']:.2f} GHz", file=sys.stderr, flush=True)

    p, d, s = res["mqa_prefill"], res["mqa_decode"], res["sparse_topk"]
    traffic = committed_traffic("mqa_prefill")
    line = {
        "metric": "attention TFLOP/s (prefill) + HBM GB/s (decode), % of MI355X peak, hd=128/256",
        "value": round(p["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(p["ms"] + d["ms"] + s["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": p["workload"], "step": "mqa_prefill + mqa_decode + sparse_topk",
                   "global_batch": 2, "seq_len": 4096, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(p["tflops"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(p["tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "decode": {"value": round(d["gbps"], 1), "unit": "GB/s",
                   "frac_of_hbm_peak": round(d["gbps"] / PEAK_HBM_GBPS, 4),
                   "us_per_call": round(d["ms"] * 1e3, 2),
                   "us_median": round(d["ms_median"] * 1e3, 2),
                   "us_p10": round(d["ms_p10"] * 1e3, 2), "us_p90": round(d["ms_p90"] * 1e3, 2),
                   "us_per_call_warm": round(d["ms_warm"] * 1e3, 2),
                   "algorithmic_bytes": d["bytes"], "workload": d["workload"],
                   "hbm_copy_GBps": round(copy_gbps, 1),
                   "read_floor_us": round(d["read_floor_ms"] * 1e3, 2),
                   "read_floor_us_warm": round(d["read_floor_ms_warm"] * 1e3, 2),
                   "read_floor_GBps": round(d["read_floor_gbps"], 1),
                   "read_floor_over_call": round(d["read_floor_ms"] / d["ms"], 4),
                   "traffic": committed_traffic("mqa_decode")},
        "sparse_topk": {"value": round(s["tflops"], 2), "unit": "TFLOP/s",
                        "frac_of_mfma_peak": round(s["tflops"] / PEAK_BF16_TFLOPS, 4),
                        "gathered_GBps": round(s["gbps"], 1),
                        "gather_floor_us": round(s["floor_ms"] * 1e3, 2),
                        "gather_floor_us_warm": round(s["floor_ms_warm"] * 1e3, 2),
                        "gather_floor_GBps": round(s["floor_gbps"], 1),
                        "gather_floor_over_call": round(s["floor_ms"] / s["ms"], 4),
                        "us_per_call": round(s["ms"] * 1e3, 2),
                        "us_median": round(s["ms_median"] * 1e3, 2),
                        "us_p10": round(s["ms_p10"] * 1e3, 2), "us_p90": round(s["ms_p90"] * 1e3, 2),
                        "us_per_call_warm": round(s["ms_warm"] * 1e3, 2),
                        "workload": s["workload"]},
        "small_configs": small,
        "prefill_detail": {"us_per_call": round(p["ms"] * 1e3, 2),
                           "us_median": round(p["ms_median"] * 1e3, 2),
                           "us_p10": round(p["ms_p10"] * 1e3, 2),
                           "us_p90": round(p["ms_p90"] * 1e3, 2),
                           "us_per_call_warm": round(p["ms_warm"] * 1e3, 2),
                           "mfma_ceiling_TFLOPs": round(mc["TFLOPs"], 1),
                           "mfma_ceiling_clock_GHz": round(mc["clock_GHz"], 3),
                           "frac_of_mfma_ceiling": round(p["tflops"] / mc["TFLOPs"], 4),
                           **committed_kernel_stats("mqa_prefill")},
    }
    line["next"] = nxt
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
