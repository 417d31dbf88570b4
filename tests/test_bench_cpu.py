"""Host-side checks of the benchmark: its one-GPU guard and the stored HBM-traffic summaries it
reports from (rocprofv3 FETCH_SIZE / WRITE_SIZE, each scaled by a copy kernel's readings). No GPU
is touched."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from synth import WORKLOADS  # noqa: E402

TRAFFIC_FILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt")))


def _read(path):
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that measured nothing


def test_every_traffic_summary_is_present():
    names = {os.path.basename(p) for p in TRAFFIC_FILES}
    # the dominant kernel of the headline, and each decode shape the bench reports a roofline for
    assert "tile_gemm_sq4096_traffic.txt" in names
    for proj in ("up", "down"):
        for m in (1, 16, 64):
            assert f"skinny_gemm_dec_{proj}_M{m}_traffic.txt" in names


@pytest.mark.parametrize("path", TRAFFIC_FILES, ids=os.path.basename)
def test_traffic_summary_arithmetic(path):
    kv = _read(path)
    copy = float(kv["copy_kernel_bytes_each_way"])
    fetch_scale, write_scale = float(kv["fetch_scale"]), float(kv["write_scale"])
    # the copy kernel reads and writes `copy` bytes: each counter's scale is what makes it say so
    assert fetch_scale == pytest.approx(copy / (float(kv["copy_fetch_kib_per_dispatch"]) * 1024), rel=1e-5)
    assert write_scale == pytest.approx(copy / (float(kv["copy_write_kib_per_dispatch"]) * 1024), rel=1e-5)
    fetch = int(kv["fetch_bytes_per_launch"])
    write = int(kv["write_bytes_per_launch"])
    # (the file prints KiB to 3 decimals and the scales to 6, hence the relative tolerance)
    assert fetch == pytest.approx(float(kv["kernel_fetch_kib_per_dispatch"]) * 1024 * fetch_scale, rel=2e-6, abs=2)
    assert write == pytest.approx(float(kv["kernel_write_kib_per_dispatch"]) * 1024 * write_scale, rel=2e-6, abs=2)
    assert abs(int(kv["traffic_bytes_per_launch"]) - (fetch + write)) <= 1  # each rounded on its own
    # a launch cannot move fewer bytes than the product must read and write (1% for counter noise)
    assert fetch + write >= 0.99 * int(kv["algorithmic_bytes_per_launch"])
    for rel in kv["sources"].split():
        assert os.path.exists(os.path.join(ROOT, rel)), rel
    assert len(kv["source_sha256"]) == 64


@pytest.mark.parametrize("path", [p for p in TRAFFIC_FILES if _read(p)["workload"] in WORKLOADS],
                         ids=os.path.basename)
def test_traffic_summary_algorithmic_bytes_match_the_workload(path):
    kv = _read(path)
    w = WORKLOADS[kv["workload"]]
    b_cols = 2 * w.N if w.glu else w.N  # the SwiGLU weight holds the gate and up halves side by side
    assert int(kv["algorithmic_bytes_per_launch"]) == 2 * (w.M * w.K + w.K * b_cols + w.M * w.N)


def test_bench_reports_stored_traffic_only_for_unchanged_sources():
    import bench
    from gemv_layers_amd.profiling import SKINNY_SOURCES, TILE_SOURCES, source_digest

    for kernel, workload, sources in (("tile", "sq4096", TILE_SOURCES), ("skinny", "dec_up_M1", SKINNY_SOURCES),
                                      ("skinny", "dec_down_M64", SKINNY_SOURCES)):
        kv = _read(os.path.join(ROOT, "profiles", f"{kernel}_gemm_{workload}_traffic.txt"))
        got = bench.measured_traffic(kernel, workload)
        if kv["source_sha256"] == source_digest(sources):
            assert got == int(kv["traffic_bytes_per_launch"])
        else:
            assert got is None
    assert bench.measured_traffic("tile", "no_such_workload") is None
