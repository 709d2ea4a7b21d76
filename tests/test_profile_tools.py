"""CPU checks of the rocprofv3 summarizers whose figures the profiles report.

Each tool reads rocprofv3's csv outputs (counter collection, kernel trace,
kernel statistics).  Synthetic files with hand-computed answers pin their
arithmetic: the copy calibration of the byte counters, bytes per dispatch,
the clock and matrix-busy formulas, per-dispatch averages and LDS ratios,
per-kernel medians, and the kernel-name shortening that keys every table.
"""

import csv
import os

import pytest

from block_sparse_attention_qk_amd import profile_counters as PC
from block_sparse_attention_qk_amd import profile_kernels as PK
from block_sparse_attention_qk_amd import profile_mfma as PM
from block_sparse_attention_qk_amd import profile_traffic as PT

ATTN = "void sva::(anonymous namespace)::attn_kernel<128, 128, false, false, 1>(sva::(anonymous namespace)::AttnArgs)"
ATTN_SHORT = "attn_kernel<128, 128, false, false, 1>"
COPY = "void sva::(anonymous namespace)::stream_copy_kernel(u32x4 const*, u32x4*, long)"
COUNTER_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                  "Start_Timestamp", "End_Timestamp"]


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _counters(path, rows):
    _write(path, COUNTER_FIELDS,
           [dict(zip(COUNTER_FIELDS, (d, k, c, v, 0, 1000))) for d, k, c, v in rows])


def test_traffic_calibration_and_bytes(tmp_path):
    mib = 64
    calib = mib * (1 << 20)
    # the read counter sees half of the copy's bytes, the write counter all
    _counters(str(tmp_path / "f" / "run_counter_collection.csv"), [
        (1, COPY, "FETCH_SIZE", calib / 2 / 1024),
        (2, ATTN, "FETCH_SIZE", 1000.0),
        (3, ATTN, "FETCH_SIZE", 3000.0),
    ])
    _counters(str(tmp_path / "w" / "run_counter_collection.csv"), [
        (1, COPY, "WRITE_SIZE", calib / 1024),
        (2, ATTN, "WRITE_SIZE", 400.0),
        (3, ATTN, "WRITE_SIZE", 600.0),
    ])
    _write(str(tmp_path / "stats.csv"), ["Name", "AverageNs"], [{"Name": ATTN, "AverageNs": 2e6}])
    res = PT.summarize(str(tmp_path / "f"), str(tmp_path / "w"), mib, str(tmp_path / "stats.csv"))
    assert res["fetch_scale"] == pytest.approx(2.0)
    assert res["write_scale"] == pytest.approx(1.0)
    e = res["kernels"][ATTN_SHORT]
    assert set(res["kernels"]) == {ATTN_SHORT}          # the copy is not a step kernel
    assert e["fetch_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)   # mean KiB per dispatch, scaled
    assert e["write_bytes"] == pytest.approx(500.0 * 1024 * 1.0)
    assert e["traffic_gbs"] == pytest.approx((2000 * 2048 + 500 * 1024) / 2e-3 / 1e9)
    assert "k_attention.hip" in res["sources_sha256"]
    assert "k_attention.hip:flags" in res["sources_sha256"]


def test_traffic_needs_the_calibration_copy(tmp_path):
    _counters(str(tmp_path / "f" / "run_counter_collection.csv"), [(1, ATTN, "FETCH_SIZE", 1.0)])
    _counters(str(tmp_path / "w" / "run_counter_collection.csv"), [(1, ATTN, "WRITE_SIZE", 1.0)])
    with pytest.raises(ValueError):
        PT.summarize(str(tmp_path / "f"), str(tmp_path / "w"), 64)


def test_mfma_clock_and_busy(tmp_path):
    # one dispatch of 2 ms: 3.0e6 graphics-active cycles per XCD (1.5 GHz),
    # matrix units busy 2.1e6 of them on every SIMD (70 %)
    _counters(str(tmp_path / "run_counter_collection.csv"), [
        (1, ATTN, "GRBM_GUI_ACTIVE", 8 * 3.0e6),
        (1, ATTN, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 2.1e6),
    ])
    _write(str(tmp_path / "run_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [{"Dispatch_Id": 1, "Kernel_Name": ATTN, "Start_Timestamp": 10_000,
             "End_Timestamp": 10_000 + 2_000_000}])
    res = PM.summarize(str(tmp_path))
    e = res[ATTN_SHORT]
    assert e["avg_ms"] == pytest.approx(2.0)
    assert e["clock_ghz"] == pytest.approx(1.5)
    assert e["mfma_busy"] == pytest.approx(0.70)


def test_counter_averages_and_ratios(tmp_path):
    _counters(str(tmp_path / "run_counter_collection.csv"), [
        (1, ATTN, "SQ_LDS_BANK_CONFLICT", 10.0), (2, ATTN, "SQ_LDS_BANK_CONFLICT", 30.0),
        (1, ATTN, "SQ_LDS_IDX_ACTIVE", 100.0), (2, ATTN, "SQ_LDS_IDX_ACTIVE", 100.0),
        (1, ATTN, "SQ_WAIT_INST_LDS", 5.0), (2, ATTN, "SQ_WAIT_INST_LDS", 15.0),
        (1, ATTN, "SQ_WAVE_CYCLES", 200.0), (2, ATTN, "SQ_WAVE_CYCLES", 200.0),
        (1, ATTN, "GRBM_GUI_ACTIVE", 8 * 1000.0), (2, ATTN, "GRBM_GUI_ACTIVE", 8 * 1000.0),
        (1, ATTN, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 600.0),
        (2, ATTN, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 800.0),
        (1, ATTN, "SQ_VALU_MFMA_COEXEC_CYCLES", 1024 * 300.0),
        (2, ATTN, "SQ_VALU_MFMA_COEXEC_CYCLES", 1024 * 300.0),
    ])
    res = PC.read_run(str(tmp_path))
    cs = res[ATTN_SHORT]
    assert cs["SQ_LDS_BANK_CONFLICT"] == pytest.approx(20.0)      # per-dispatch average
    md = PC.to_markdown(res, "t", "c")
    row = [ln for ln in md.splitlines() if ATTN_SHORT in ln][0].split("|")
    # bank conflict / active 20/100, LDS wait / wave cycles 10/200, MFMA busy
    # 700/1000, co-execution 300/700 of the busy cycles
    assert [c.strip() for c in row[-5:-1]] == ["0.200", "0.050", "70.0 %", "42.9 %"]


def test_kernel_medians(tmp_path):
    path = str(tmp_path / "trace.csv")
    rows = []
    for i, ms in enumerate((1.0, 2.0, 10.0)):
        rows.append({"Kernel_Name": ATTN, "Start_Timestamp": 0, "End_Timestamp": int(ms * 1e6)})
    for i, ms in enumerate((1.0, 3.0)):
        rows.append({"Kernel_Name": COPY, "Start_Timestamp": 0, "End_Timestamp": int(ms * 1e6)})
    _write(path, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    med = PK.read_medians(path)
    assert med[ATTN_SHORT] == pytest.approx(2.0)
    assert med["stream_copy_kernel"] == pytest.approx(2.0)


def test_bench_traffic_only_for_the_measured_kernel(monkeypatch):
    """bench.py reports the committed attention traffic only while the
    attention source and its compiler options match the hashes the counter
    summary recorded; any change to either makes it None."""
    import json
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    with open(os.path.join(root, "profiles", "traffic_wan720p_sp75.json")) as f:
        rec = json.load(f)
    want = next(e["traffic_bytes"] for k, e in rec["kernels"].items()
                if k.startswith("attn_kernel<128, 128, "))
    now = PT.source_hashes()
    assert bench.measured_traffic("wan720p_sp75", 128, 128) == pytest.approx(round(want, 0))
    for f in ("k_attention.hip", "k_attention.hip:flags"):
        changed = dict(now, **{f: "0" * 64})
        monkeypatch.setattr(PT, "source_hashes", lambda c=changed: c)
        assert bench.measured_traffic("wan720p_sp75", 128, 128) is None, f
    monkeypatch.setattr(PT, "source_hashes", lambda: now)
    assert bench.measured_traffic("no_such_workload", 128, 128) is None
