"""Host-side logic of bench.py (no GPU): the kernel-trace summary that picks
out the timed calls, the counter ingest and its copy calibration, and the
staleness check of the committed counters."""
import csv
import json
import os

import pytest

import bench

FWD = "void fmha::(anonymous namespace)::fwd_kernel<128, 32, 32, 4, false, 3>(fmha::FwdParams)"
SUM = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<long, sum_functor<long> > >"
MAX = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<long, MaxNanFunctor<long> > >"
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_trace_summary_counts_only_the_timed_flushed_calls(tmp_path):
    # (kernel, duration ns): ramp pairs after a max flush, timed pairs after a
    # sum flush, then back-to-back calls
    seq = [(MAX, 100), (FWD, 300_000), (MAX, 100), (FWD, 310_000),
           (SUM, 100), (FWD, 280_000), (SUM, 100), (FWD, 290_000),
           (FWD, 270_000)]
    rows, t = [], 0
    for name, dur in seq:
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 1000
    path = tmp_path / "kt_kernel_trace.csv"
    _write_csv(path, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    table = bench.trace_summary(str(path))
    line = [ln for ln in table.splitlines() if "fwd_kernel<128" in ln]
    assert len(line) == 1
    cells = [c.strip() for c in line[0].strip("|").split("|")]
    # dispatches, avg, min, max, flushed calls, flushed avg
    assert cells[1] == "5"
    assert cells[2] == f"{(300 + 310 + 280 + 290 + 270) / 5:.1f}"
    assert cells[5] == "2" and cells[6] == "285.0"


def _counter_dir(tmp_path, name, counter, values):
    d = tmp_path / name
    d.mkdir()
    rows = [{"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v, "Dispatch_Id": i}
            for i, (k, v) in enumerate(values)]
    _write_csv(d / "p_counter_collection.csv",
               ["Kernel_Name", "Counter_Name", "Counter_Value", "Dispatch_Id"], rows)
    return str(d)


def test_ingest_scales_each_counter_by_the_copy_and_maps_workloads(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    copy_kib = bench.COPY_BYTES / 1024
    # the copy reads half of its bytes on FETCH_SIZE (factor 2) and all of
    # them on WRITE_SIZE (factor 1); medians are taken per kernel
    fetch = _counter_dir(tmp_path, "fetch", "FETCH_SIZE",
                         [(COPY, copy_kib / 2), (COPY, copy_kib / 2), (FWD, 900.0), (FWD, 1000.0),
                          (FWD, 1100.0)])
    write = _counter_dir(tmp_path, "write", "WRITE_SIZE",
                         [(COPY, copy_kib), (FWD, 500.0)])
    bench.ingest_counters(fetch, write)
    rec = json.loads(out.read_text())
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    assert rec["copy_scale"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert rec["copy_scale"]["WRITE_SIZE"] == pytest.approx(1.0)
    want = 1000.0 * 1024 * 2.0 + 500.0 * 1024 * 1.0
    assert rec["kernels"][FWD]["bytes_per_launch"] == pytest.approx(want)
    assert rec["workloads"]["mqa_prefill"]["bytes_per_launch"] == pytest.approx(want)
    assert "mqa_decode" not in rec["workloads"]  # no split or merge kernel in this run


def test_ingest_refuses_a_run_without_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    fetch = _counter_dir(tmp_path, "fetch", "FETCH_SIZE", [(FWD, 1.0)])
    write = _counter_dir(tmp_path, "write", "WRITE_SIZE", [(FWD, 1.0)])
    with pytest.raises(SystemExit):
        bench.ingest_counters(fetch, write)


def test_committed_traffic_is_null_once_a_kernel_source_changes(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    rec = {"kernel_source_hash": bench.kernel_source_hash(),
           "workloads": {"mqa_prefill": {"bytes_per_launch": 123.0}}}
    path.write_text(json.dumps(rec))
    assert bench.committed_traffic("mqa_prefill") == 123.0
    assert bench.committed_traffic("mqa_decode") is None
    rec["kernel_source_hash"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.committed_traffic("mqa_prefill") is None
    os.remove(path)
    assert bench.committed_traffic("mqa_prefill") is None


def test_the_hash_covers_every_library_source():
    """Every source build.py compiles, and every header beside them, is
    hashed with the committed counters: any change to the library's code
    turns them stale."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "fmha_mqa_build_for_test", os.path.join(bench.ROOT, "fmha_mqa_fwd_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)  # build.py only defines; it does not build on import
    hashed = {os.path.basename(p) for p in bench.KERNEL_SOURCES}
    for rel in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(bench.ROOT, rel)), rel
    for src in mod.SOURCES:
        assert src in hashed, src
    for hdr in ("fmha_device.h", "fmha_internal.h", "api.hip"):
        assert hdr in hashed, hdr


def test_pipe_counters_give_lds_vector_and_coexec_shares(tmp_path):
    """The LDS / vector / co-execution shares of a kernel from one counter
    run: per-XCD cycles are GRBM_GUI_ACTIVE / 8; LDS busy per CU cycle,
    vector-active quad-cycles x 4 per SIMD cycle, co-execution per matrix-busy
    cycle."""
    d = tmp_path / "pipe"
    d.mkdir()
    cyc = 1000.0
    vals = {"GRBM_GUI_ACTIVE": cyc * 8, "SQ_LDS_IDX_ACTIVE": 0.25 * 256 * cyc,
            "SQ_LDS_BANK_CONFLICT": 0.01 * 256 * cyc, "SQ_ACTIVE_INST_VALU": 0.5 * 1024 * cyc / 4,
            "SQ_VALU_MFMA_BUSY_CYCLES": 0.6 * 1024 * cyc,
            "SQ_VALU_MFMA_COEXEC_CYCLES": 0.3 * 0.6 * 1024 * cyc,
            "SQ_INSTS_LDS": 123.0, "SQ_INSTS_VALU": 456.0}
    rows = [{"Kernel_Name": FWD, "Counter_Name": c, "Counter_Value": v, "Dispatch_Id": 1}
            for c, v in vals.items()]
    _write_csv(d / "p_counter_collection.csv",
               ["Kernel_Name", "Counter_Name", "Counter_Value", "Dispatch_Id"], rows)
    r = bench._pipe_counters(str(d))[FWD]
    assert r["lds_busy_frac"] == pytest.approx(0.25)
    assert r["lds_bank_conflict_frac"] == pytest.approx(0.04)
    assert r["valu_active_frac"] == pytest.approx(0.5)
    assert r["mfma_busy_frac"] == pytest.approx(0.6)
    assert r["mfma_valu_coexec_frac"] == pytest.approx(0.3)
    assert r["lds_insts"] == 123 and r["valu_insts"] == 456
