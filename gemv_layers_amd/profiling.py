"""Summaries of rocprofv3 CSV output for this library's kernels (plain Python, no GPU needed).

    python -m gemv_layers_amd.profiling stats  <run_kernel_stats.csv> [--kernel REGEX] [--command CMD]
    python -m gemv_layers_amd.profiling traffic --fetch <counter_collection.csv>
        --write <counter_collection.csv> --kernel REGEX --copy-bytes N --workload NAME
        [--algorithmic-bytes B] [--command CMD]

    python -m gemv_layers_amd.profiling window <run_kernel_trace.csv> --kernel REGEX --skip N
        --count K [--grid THREADS]
    python -m gemv_layers_amd.profiling counters <counter_collection.csv> [...] --kernel REGEX
        [--grid THREADS] [--cus N] [--command CMD]

`stats` prints the per-kernel table of a `--kernel-trace --stats --output-format csv` run (the
kernels matching REGEX only, when given).
`window` takes the dispatches of the matching kernel in dispatch order, skips the first N and
prints the mean, minimum and maximum duration of the next K, and their span (first start to
last end) divided by K: e.g. the timed region of a benchmark that runs N warm-up launches
first.
`counters` averages every counter of one or more `--pmc` passes over the dispatches of the
matching kernel and derives the busy fractions. GRBM_GUI_ACTIVE is summed over the XCDs, so the
kernel's cycles are G = GRBM_GUI_ACTIVE / XCDs; then MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES over
(G x CUs x 4 SIMDs), TA busy = TA_TA_BUSY over (G x CUs), TA address FIFO full =
SQ_VMEM_TA_ADDR_FIFO_FULL over (G x CUs), LDS busy = SQ_LDS_IDX_ACTIVE over (G x CUs), the wave
wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, LDS bank conflicts per LDS instruction, and the
L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS).
`traffic` turns two counter passes (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, both over a
command that also runs the library's copy kernel on `--copy-bytes` bytes, e.g.
`bench.py --copy-calibration`) into HBM bytes per launch of the kernel matching REGEX: each
counter's mean KiB per dispatch of that kernel, times (known copy bytes / what the same counter
read for the copy kernel). The output carries a sha256 of the kernel's sources so that a reader
can tell whether the readings still describe the current kernel.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

TILE_SOURCES = ("gemv_layers_amd/csrc/gemm_tile.hip", "gemv_layers_amd/csrc/common.h",
                "gemv_layers_amd/csrc/tile.h")
SKINNY_SOURCES = ("gemv_layers_amd/csrc/gemm_skinny.hip", "gemv_layers_amd/csrc/common.h",
                  "gemv_layers_amd/csrc/skinny.h", "gemv_layers_amd/csrc/stream_k.h")
MX_SOURCES = ("gemv_layers_amd/csrc/gemm_mx.hip", "gemv_layers_amd/csrc/common.h",
              "gemv_layers_amd/csrc/mx.h")
PACKED_SOURCES = ("gemv_layers_amd/csrc/gemm_packed.hip", "gemv_layers_amd/csrc/common.h",
                  "gemv_layers_amd/csrc/packed.h")
_SOURCES = {"tile": TILE_SOURCES, "skinny": SKINNY_SOURCES, "mx": MX_SOURCES, "packed": PACKED_SOURCES}
COPY_KERNEL = r"peak_copy_kernel"


def source_digest(paths=TILE_SOURCES) -> str:
    """sha256 over the given sources (paths relative to the repository root)."""
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_stats(path: str) -> list[dict]:
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                         "total_ns": float(r["TotalDurationNs"]), "avg_ns": float(r["AverageNs"]),
                         "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                         "percent": float(r["Percentage"])})
    return rows


def counter_per_dispatch(path: str, counter: str, kernel_regex: str, grid: int = 0) -> list[float]:
    """Values of `counter` for every dispatch whose kernel name matches `kernel_regex` (and whose
    grid has `grid` threads, when given)."""
    rx = re.compile(kernel_regex)
    out = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and rx.search(r["Kernel_Name"]) and \
                    (not grid or int(r["Grid_Size"]) == grid):
                out.append(float(r["Counter_Value"]))
    return out


def _mean(v: list[float]) -> float:
    if not v:
        raise SystemExit("no matching dispatches")
    return sum(v) / len(v)


def cmd_stats(a) -> None:
    rows = kernel_stats(a.csv)
    if a.kernel:
        rx = re.compile(a.kernel)
        rows = [r for r in rows if rx.search(r["name"])]
    if a.command:
        print(f"# command: {a.command}")
    print(f"{'calls':>7} {'avg_us':>11} {'min_us':>10} {'max_us':>10} {'time%':>7}  kernel")
    for r in rows[: a.top]:
        name = r["name"] if len(r["name"]) <= 110 else r["name"][:107] + "..."
        print(f"{r['calls']:7d} {r['avg_ns'] / 1e3:11.3f} {r['min_ns'] / 1e3:10.3f} "
              f"{r['max_ns'] / 1e3:10.3f} {r['percent']:7.3f}  {name}")


def cmd_window(a) -> None:
    rx = re.compile(a.kernel)
    rows = []
    with open(a.csv, newline="") as f:
        for r in csv.DictReader(f):
            if rx.search(r["Kernel_Name"]) and (not a.grid or int(r["Grid_Size_X"]) == a.grid):
                rows.append((int(r["Dispatch_Id"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    win = rows[a.skip:a.skip + a.count]
    if len(win) < a.count:
        raise SystemExit(f"only {len(rows)} matching dispatches")
    durs = [(e - b) / 1e3 for _, b, e in win]
    span = (win[-1][2] - win[0][1]) / 1e3
    print(f"# dispatches {a.skip} .. {a.skip + a.count - 1} of the kernel matching /{a.kernel}/"
          + (f", grid {a.grid} threads" if a.grid else "") + f" ({len(rows)} in the trace)")
    print(f"mean_us: {sum(durs) / len(durs):.3f}")
    print(f"min_us: {min(durs):.3f}")
    print(f"max_us: {max(durs):.3f}")
    print(f"span_over_count_us: {span / a.count:.3f}")


def cmd_traffic(a) -> None:
    kib = 1024.0
    f_copy = _mean(counter_per_dispatch(a.fetch, "FETCH_SIZE", COPY_KERNEL))
    w_copy = _mean(counter_per_dispatch(a.write, "WRITE_SIZE", COPY_KERNEL))
    f_k = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel, a.grid)
    w_k = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel, a.grid)
    fetch_scale = a.copy_bytes / (f_copy * kib)
    write_scale = a.copy_bytes / (w_copy * kib)
    fetch_b = _mean(f_k) * kib * fetch_scale
    write_b = _mean(w_k) * kib * write_scale
    srcs = _SOURCES[a.sources]
    print(f"# HBM traffic per launch of the kernel matching /{a.kernel}/ on workload {a.workload}")
    if a.command:
        for ln in a.command.split(" ;; "):
            print(f"# command: {ln}")
    print(f"workload: {a.workload}")
    print(f"kernel_regex: {a.kernel}")
    if a.grid:
        print(f"grid_threads: {a.grid}")
    print(f"sources: {' '.join(srcs)}")
    print(f"source_sha256: {source_digest(srcs)}")
    print(f"copy_kernel_bytes_each_way: {a.copy_bytes}")
    print(f"copy_fetch_kib_per_dispatch: {f_copy:.3f}")
    print(f"copy_write_kib_per_dispatch: {w_copy:.3f}")
    print(f"fetch_scale: {fetch_scale:.6f}")
    print(f"write_scale: {write_scale:.6f}")
    print(f"kernel_dispatches: {len(f_k)} fetch, {len(w_k)} write")
    print(f"kernel_fetch_kib_per_dispatch: {_mean(f_k):.3f}")
    print(f"kernel_write_kib_per_dispatch: {_mean(w_k):.3f}")
    print(f"fetch_bytes_per_launch: {fetch_b:.0f}")
    print(f"write_bytes_per_launch: {write_b:.0f}")
    print(f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}")
    if a.algorithmic_bytes:
        print(f"algorithmic_bytes_per_launch: {a.algorithmic_bytes}")
        print(f"traffic_over_algorithmic: {(fetch_b + write_b) / a.algorithmic_bytes:.3f}")


def counter_means(paths, kernel_regex: str, grid: int = 0) -> tuple[dict, dict]:
    """Mean per dispatch of every counter of the matching kernel over the given passes, and the
    number of dispatches each mean is over."""
    rx = re.compile(kernel_regex)
    vals: dict[str, list[float]] = {}
    for path in paths:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if rx.search(r["Kernel_Name"]) and (not grid or int(r["Grid_Size"]) == grid):
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: _mean(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def derived_fractions(m: dict, cus: int, xcds: int = 8) -> dict:
    out = {}
    gui = m.get("GRBM_GUI_ACTIVE")
    if gui:
        gui = gui / xcds
        out["kernel_cycles_per_xcd"] = gui
    if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        out["mfma_busy_frac"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * cus * 4)
    if "SQ_WAIT_INST_ANY" in m and m.get("SQ_WAVE_CYCLES"):
        out["wave_wait_inst_frac"] = m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]
    if "SQ_WAIT_ANY" in m and m.get("SQ_WAVE_CYCLES"):
        out["wave_wait_any_frac"] = m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"]
    if gui and "TA_TA_BUSY" in m:
        out["ta_busy_frac"] = m["TA_TA_BUSY"] / (gui * cus)
    if gui and "TA_ADDR_STALLED_BY_TC_CYCLES" in m:
        out["ta_addr_stalled_by_tc_frac"] = m["TA_ADDR_STALLED_BY_TC_CYCLES"] / (gui * cus)
    if gui and "SQ_VMEM_TA_ADDR_FIFO_FULL" in m:
        out["ta_addr_fifo_full_frac"] = m["SQ_VMEM_TA_ADDR_FIFO_FULL"] / (gui * cus)
    if gui and "SQ_LDS_IDX_ACTIVE" in m:
        out["lds_busy_frac"] = m["SQ_LDS_IDX_ACTIVE"] / (gui * cus)
    if m.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in m:
        out["lds_bank_conflict_cycles_per_lds_inst"] = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_INSTS_LDS"]
    if m.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in m:
        out["lds_bank_conflict_per_active_lds_cycle"] = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_ACTIVE_INST_LDS"]
    if m.get("TCC_HIT") is not None and m.get("TCC_MISS") is not None and (m["TCC_HIT"] + m["TCC_MISS"]) > 0:
        out["l2_hit_frac"] = m["TCC_HIT"] / (m["TCC_HIT"] + m["TCC_MISS"])
    return out


def cmd_counters(a) -> None:
    means, counts = counter_means(a.csv, a.kernel, a.grid)
    if not means:
        raise SystemExit("no matching dispatches")
    print(f"# mean per dispatch of the kernel matching /{a.kernel}/" + (f", grid {a.grid} threads" if a.grid else ""))
    if a.command:
        for ln in a.command.split(" ;; "):
            print(f"# command: {ln}")
    for k in sorted(means):
        print(f"{k}: {means[k]:.1f}   # {counts[k]} dispatches")
    for k, v in derived_fractions(means, a.cus, a.xcds).items():
        print(f"{k}: {v:.4f}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(prog="python -m gemv_layers_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--kernel", default="")
    s.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--sources", choices=("tile", "skinny", "mx", "packed"), default="tile")
    t.add_argument("--grid", type=int, default=0, help="only dispatches with this many threads")
    t.add_argument("--algorithmic-bytes", type=int, default=0)
    t.add_argument("--command", default="")
    w = sub.add_parser("window")
    w.add_argument("csv")
    w.add_argument("--kernel", required=True)
    w.add_argument("--skip", type=int, default=0)
    w.add_argument("--count", type=int, required=True)
    w.add_argument("--grid", type=int, default=0, help="only dispatches with this many threads")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--grid", type=int, default=0, help="only dispatches with this many threads")
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--command", default="")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "window": cmd_window, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main(sys.argv[1:])
