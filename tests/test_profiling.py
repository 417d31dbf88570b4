"""The rocprofv3 summary tool (gemv_layers_amd.profiling) on small synthetic CSV files (CPU only)."""

import csv
import io
import contextlib

import pytest

from gemv_layers_amd import profiling


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        for r in rows:
            w.writerow(r)


def _run(argv):
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        profiling.main(argv)
    return out.getvalue()


def _kv(text):
    kv = {}
    for ln in text.splitlines():
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


TRACE_HEADER = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]


def test_window_takes_dispatches_in_order_after_the_skip(tmp_path):
    p = tmp_path / "trace.csv"
    rows = []
    t = 1000
    # dispatch ids out of file order; another kernel and another grid interleaved
    for i, (dur, grid) in enumerate([(10, 64), (20, 64), (30, 64), (40, 64), (50, 64), (99, 32)]):
        rows.append(["KERNEL_DISPATCH", 2 * i + 1, "void k<1>(A)", t, t + dur * 1000, grid])
        rows.append(["KERNEL_DISPATCH", 2 * i + 2, "other", t, t + 5000, grid])
        t += 100_000
    rows.reverse()
    _write(p, TRACE_HEADER, rows)
    kv = _kv(_run(["window", str(p), "--kernel", r"k<1>", "--skip", "1", "--count", "3", "--grid", "64"]))
    assert float(kv["mean_us"]) == pytest.approx(30.0)     # 20, 30, 40
    assert float(kv["min_us"]) == pytest.approx(20.0)
    assert float(kv["max_us"]) == pytest.approx(40.0)
    # span: start of the 2nd to end of the 4th dispatch = 2 gaps of 100 us + 40 us, over 3
    assert float(kv["span_over_count_us"]) == pytest.approx((200.0 + 40.0) / 3)


def test_window_refuses_a_short_trace(tmp_path):
    p = tmp_path / "trace.csv"
    _write(p, TRACE_HEADER, [["KERNEL_DISPATCH", 1, "k", 0, 1000, 64]])
    with pytest.raises(SystemExit):
        _run(["window", str(p), "--kernel", "k", "--count", "2"])


COUNTER_HEADER = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]


def test_traffic_scales_each_counter_by_the_copy_kernel(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    copy_bytes = 1 << 20
    # the copy kernel moves copy_bytes each way; FETCH_SIZE reads half (KiB), WRITE_SIZE exactly
    _write(fetch, COUNTER_HEADER, [["peak_copy_kernel", 256, "FETCH_SIZE", copy_bytes / 2048],
                                   ["tile_gemm_kernel<x>", 256, "FETCH_SIZE", 100.0],
                                   ["tile_gemm_kernel<x>", 256, "FETCH_SIZE", 300.0],
                                   ["tile_gemm_kernel<x>", 128, "FETCH_SIZE", 9999.0]])
    _write(write, COUNTER_HEADER, [["peak_copy_kernel", 256, "WRITE_SIZE", copy_bytes / 1024],
                                   ["tile_gemm_kernel<x>", 256, "WRITE_SIZE", 50.0]])
    kv = _kv(_run(["traffic", "--fetch", str(fetch), "--write", str(write), "--kernel", r"tile_gemm_kernel<x>",
                   "--grid", "256", "--copy-bytes", str(copy_bytes), "--workload", "w",
                   "--algorithmic-bytes", "1024"]))
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    assert int(kv["fetch_bytes_per_launch"]) == 200 * 1024 * 2    # mean 200 KiB, scaled by 2
    assert int(kv["write_bytes_per_launch"]) == 50 * 1024
    assert int(kv["traffic_bytes_per_launch"]) == (400 + 50) * 1024
    assert float(kv["traffic_over_algorithmic"]) == pytest.approx(450.0)
    assert kv["source_sha256"] == profiling.source_digest(profiling.TILE_SOURCES)


def test_stats_filters_by_kernel(tmp_path):
    p = tmp_path / "stats.csv"
    _write(p, ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"],
           [["glk::a_kernel", 4, 4000, 1000, 900, 1100, 60.0], ["other", 1, 2000, 2000, 2000, 2000, 40.0]])
    text = _run(["stats", str(p), "--kernel", "glk::"])
    assert "glk::a_kernel" in text and "other" not in text
    assert "1.000" in text  # average in microseconds


PMC_HEADER = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]


def test_counters_average_per_dispatch_and_derive_fractions(tmp_path):
    p1, p2 = tmp_path / "a.csv", tmp_path / "b.csv"
    k = "tile_gemm_kernel<256, 256, 2, 4, false>"
    _write(p1, PMC_HEADER, [
        [1, 131072, k, "GRBM_GUI_ACTIVE", 1000.0], [1, 131072, k, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0],
        [2, 131072, k, "GRBM_GUI_ACTIVE", 3000.0], [2, 131072, k, "SQ_VALU_MFMA_BUSY_CYCLES", 1536000.0],
        [3, 524288, k, "GRBM_GUI_ACTIVE", 9.0e9], [4, 131072, "other", "GRBM_GUI_ACTIVE", 1.0],
        [1, 131072, k, "SQ_WAVE_CYCLES", 400.0], [1, 131072, k, "SQ_WAIT_INST_ANY", 100.0],
        [2, 131072, k, "SQ_WAVE_CYCLES", 400.0], [2, 131072, k, "SQ_WAIT_INST_ANY", 300.0]])
    _write(p2, PMC_HEADER, [[5, 131072, k, "TA_TA_BUSY", 256000.0], [5, 131072, k, "GRBM_GUI_ACTIVE", 2000.0]])
    kv = _kv(_run(["counters", str(p1), str(p2), "--kernel", "tile_gemm", "--grid", "131072", "--cus", "256",
                   "--xcds", "1"]))
    assert float(kv["GRBM_GUI_ACTIVE"].split("#")[0]) == pytest.approx(2000.0)
    # 1024000 / (2000 * 256 * 4) = 0.5
    assert float(kv["mfma_busy_frac"]) == pytest.approx(0.5)
    assert float(kv["wave_wait_inst_frac"]) == pytest.approx(0.5)
    assert float(kv["ta_busy_frac"]) == pytest.approx(0.5)
