"""Benchmark: bf16 -> fp32 GEMM TFLOP/s and fraction of the MFMA roof at 4096^3, plus the
skinny decode shapes' HBM GB/s, on one MI355X. Prints ONE JSON line.

A step is one call of the library's dispatching entry point (gemm_bf16) on the 4096^3 workload
(A, B ~ N(0,1) bf16 from fixed seeds, already resident in HBM). Before anything is timed the card
runs at least 300 ms of back-to-back steps, so that its clock has settled (spark-kernels post,
"how things are measured": a 300 ms clock ramp). Then W counted warm-up steps, then `value`: the
throughput of exactly K steps run back to back on one stream between two synchronisations. The
dominant kernel's average duration over those K steps is measured with HIP events recorded on
the stream the kernel is launched on, and gives `roofline.achieved` = 2*M*N*K / duration.

Alongside (reported, not part of `value`):
* the card's measured roofs: sustained MFMA bf16->fp32 TFLOP/s and shader clock, HBM copy and
  read GB/s over 1 GiB buffers, the empty-launch floor, and a read-only kernel over exactly the
  decode weight's 90.2 MB (cold copies, single launch and back to back: "the decode kernel");
* every compute-bound workload (sq4096, sq8192, sq16384, mlp_up, mlp_down, sq512), each in >= 5
  rounds of >= 100 launches with hipBLASLt (torch.matmul) interleaved in rotated order, reporting
  the median and the minimum over rounds ("Benchmarks" page of gemm3, "Measurement conditions";
  "Kernel development on sm_120", section 6), the time with the Infinity Cache flushed before
  each launch, and its own roofline object;
* three shapes outside those configurations, one for each planner rule that none of them
  exercises (a sparse last wave cut off, one 128 x 128 tile per CU with K split, between one and
  two tiles per CU), against hipBLASLt in the same rounds (planner_cases);
* the shader clock and board power sampled every 250 ms over a sustained run of the 8192^3
  product ("the roof is the power limit");
* every decode workload (M = 1, 2, 16, 64 against the 7B MLP weights), over 12 rotating copies of
  the weights (> 1 GiB, more than the 256 MB Infinity Cache) so each call reads cold weights, as
  single launches between events, back to back and replayed from a captured graph;
* the fused SwiGLU and block-scaled (MX) decode workloads;
* the float64 CPU oracle timed on a bounded row sample of the 4096^3 product (cpu_baseline).
"""

from __future__ import annotations

import argparse
import ctypes
import glob
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "bf16→fp32 GEMM TFLOP/s & % MFMA peak at 4096³; skinny M≤64 HBM GB/s"
MI355X_PEAK_BF16_TFLOPS = 2500.0   # published dense bf16 MFMA peak
MI355X_PEAK_CLOCK_GHZ = 2.4        # the engine clock that peak is quoted at (256 CUs x 4 SIMDs x 1024 flop/clk)
MI355X_PEAK_HBM_GBPS = 8000.0      # published HBM3E bandwidth
RAMP_MS = 300.0                    # clock ramp before every timed arm
COMPUTE = ("sq4096", "sq8192", "sq16384", "mlp_up", "mlp_down", "sq512")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` ("tile" or "skinny") on `workload` from the stored
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes (each scaled by the copy-kernel calibration), or
    None when there is no stored reading for it or the kernel's sources changed since it was
    taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_gemm_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    from gemv_layers_amd.profiling import SKINNY_SOURCES, TILE_SOURCES, source_digest

    sources = TILE_SOURCES if kernel == "tile" else SKINNY_SOURCES
    if kv.get("source_sha256") != source_digest(sources) or "traffic_bytes_per_launch" not in kv:
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


class PowerSampler:
    """Board power (W) and shader clock (MHz) from the amdgpu hwmon files, every `period` s, in a
    host thread, while the GPU runs something else. Empty when the files are not readable."""

    def __init__(self, period: float = 0.25):
        self.period = period
        self.samples: list[tuple[float, float | None, float | None]] = []
        self._stop = threading.Event()
        self.power_file = self.clock_file = None
        for hw in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
            for name in ("power1_average", "power1_input"):
                if os.access(os.path.join(hw, name), os.R_OK):
                    self.power_file = os.path.join(hw, name)
                    break
            if os.access(os.path.join(hw, "freq1_input"), os.R_OK):
                self.clock_file = os.path.join(hw, "freq1_input")
            if self.power_file:
                break

    @staticmethod
    def _read(path, scale):
        try:
            with open(path) as f:
                return float(f.read().strip()) * scale
        except (OSError, ValueError):
            return None

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            w = self._read(self.power_file, 1e-6) if self.power_file else None
            mhz = self._read(self.clock_file, 1e-6) if self.clock_file else None
            self.samples.append((round(time.perf_counter() - t0, 3), w, mhz))
            self._stop.wait(self.period)

    def __enter__(self):
        self._t = threading.Thread(target=self._run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="sq4096")
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--no-peaks", action="store_true", help="skip the roof microbenchmarks")
    ap.add_argument("--no-compute", action="store_true",
                    help="skip the compute-bound workloads other than the headline")
    ap.add_argument("--only", default="", help="comma-separated compute workloads to time (default: all)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workloads")
    ap.add_argument("--decode", default="", help="comma-separated decode workloads to time (default: all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-torch", action="store_true", help="skip the torch.matmul comparison")
    ap.add_argument("--no-power", action="store_true", help="skip the sustained power/clock sample")
    ap.add_argument("--no-planner-cases", action="store_true",
                    help="skip the shapes outside the configurations that show the planner's rules")
    ap.add_argument("--no-swiglu", action="store_true",
                    help="skip the fused gate/up SwiGLU workloads")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the block-scaled (MXFP8 x MXFP4) decode workloads")
    ap.add_argument("--packed", action="store_true",
                    help="also time the decode workloads on packed bf16 weights")
    ap.add_argument("--swiglu-unfused-ours", action="store_true",
                    help="also time the unfused SwiGLU path on this library's own product (it runs "
                         "the plain kernels, which then also appear in a profile of this command)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run the copy kernel 3 times over 256 MiB (known traffic) so that a "
                         "counter pass over this command also calibrates FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gemv_layers_amd as g
    from synth import WORKLOADS, matrix

    torch.cuda.set_device(0)
    g.gemm_init(0)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def dev(h):
        return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).view(torch.bfloat16).cuda()

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def warm(fn, ms=RAMP_MS):
        """fn(i) back to back for about `ms` milliseconds (at least two calls), then synchronise:
        after an idle spell (host-side input generation, a lone-launch measurement) the card takes
        tens of milliseconds of sustained load to settle its clocks. Returns the call count."""
        fn(0)
        e0, e1 = events(2)
        e0.record(stream)
        fn(1)
        e1.record(stream)
        torch.cuda.synchronize()
        n = int(ms / max(e0.elapsed_time(e1), 1e-3)) + 1
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return n + 2

    def timed_rounds(arms: dict, n: int, rounds: int):
        """Every arm n times back to back between two events, per round, the arms in an order
        rotated each round; per-arm arrays of the per-launch mean (us) of each round."""
        names = list(arms)
        res = {k: [] for k in names}
        for r in range(rounds):
            order = names[r % len(names):] + names[:r % len(names)]
            for k in order:
                e0, e1 = events(2)
                e0.record(stream)
                for _ in range(n):
                    arms[k]()
                e1.record(stream)
                torch.cuda.synchronize()
                res[k].append(e0.elapsed_time(e1) * 1e3 / n)
        return {k: np.array(v) for k, v in res.items()}

    def clock_during(launch, launch_ms, n=32):
        """Median shader clock (GHz) while `launch` runs back to back: the clock probe runs on a
        second stream (default priority), one wave per workgroup beside the launches' workgroups,
        started after a few launches and lasting about a quarter of the stream of them."""
        blocks = 256
        clk = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
        side = torch.cuda.Stream()
        e0, e1 = events(2)
        e0.record(stream)
        g.gemm_peak_clock_launch(20000, blocks, P(clk), sh)
        e1.record(stream)
        torch.cuda.synchronize()
        per_iter_ms = max(e0.elapsed_time(e1), 1e-3) / 20000
        iters = int(max(2000, min(5e7, 0.25 * n * launch_ms / per_iter_ms)))
        for i in range(n):
            launch()
            if i == 3:
                g.gemm_peak_clock_launch(iters, blocks, P(clk), side.cuda_stream)
        torch.cuda.synchronize()
        cc = clk.view(-1, 2).double().cpu()
        return float((cc[:, 0] / cc[:, 1]).median()) * 0.1  # s_memrealtime runs at 100 MHz

    out = {}

    # the headline workload's inputs are generated (on the host) before the roof measurements, so
    # that its clock ramp follows the card's sustained load there rather than an idle spell
    w = WORKLOADS[args.workload]
    A = dev(matrix("normal", w.M, w.K, seed=w.seed_a, sigma=w.sigma_a))
    B = dev(matrix("normal", w.K, w.N, seed=w.seed_b, sigma=w.sigma_b))
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")

    # ---------------- measured roofs ----------------
    peaks = {}
    if not args.no_peaks:
        log("HBM copy/read")
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        g.gemm_fill_launch(P(src), nbytes, 0x12345678, sh)
        rsink = torch.zeros(65536, dtype=torch.int32, device="cuda")
        best_copy = best_read = 0.0
        for _ in range(10):
            e0, e1, e2 = events(3)
            e0.record(stream)
            g.gemm_peak_copy_launch(P(src), P(dst), nbytes, sh)
            e1.record(stream)
            g.gemm_peak_read_launch(P(src), nbytes, P(rsink), sh)
            e2.record(stream)
            torch.cuda.synchronize()
            best_copy = max(best_copy, 2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
            best_read = max(best_read, nbytes / (e1.elapsed_time(e2) * 1e-3) / 1e9)
        e0, e1 = events(2)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        peaks["hbm_copy_gbps"] = round(best_copy, 1)
        peaks["hbm_read_gbps"] = round(best_read, 1)
        peaks["hip_memcpy_d2d_gbps"] = round(2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del src, dst

        # launch floor: single launch between events, and back to back
        singles = []
        for _ in range(50):
            e0, e1 = events(2)
            e0.record(stream)
            g.gemm_peak_empty_launch(sh)
            e1.record(stream)
            torch.cuda.synchronize()
            singles.append(e0.elapsed_time(e1) * 1e3)
        e0, e1 = events(2)
        e0.record(stream)
        for _ in range(1000):
            g.gemm_peak_empty_launch(sh)
        e1.record(stream)
        torch.cuda.synchronize()
        peaks["empty_launch_us_single_median"] = round(float(np.median(singles)), 2)
        peaks["empty_launch_us_back_to_back"] = round(e0.elapsed_time(e1), 3)  # ms/1000 = us
        # the matrix-core roof last, so that the headline's ramp follows its sustained load
        log("MFMA peak")
        blocks = 512
        sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
        cyc = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
        flop_per_iter = blocks * 4 * 8 * 32768

        def mfma_run(iters):
            e0, e1 = events(2)
            e0.record(stream)
            g.gemm_peak_mfma_launch(iters, blocks, P(sink), P(cyc), sh)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            c = cyc.view(-1, 2).double()
            clk_ghz = float((c[:, 0] / c[:, 1]).mean()) * 0.1  # s_memrealtime runs at 100 MHz
            return flop_per_iter * iters / (ms * 1e-3) / 1e12, ms, clk_ghz

        mfma_run(20000)  # clock ramp
        t_end = time.time() + 0.3
        while time.time() < t_end:
            mfma_run(20000)
        burst = max(mfma_run(20000)[0] for _ in range(3))
        sampler = PowerSampler()
        with sampler:
            sus_tf, sus_ms, sus_clk = mfma_run(5_000_000)
        watts = [x[1] for x in sampler.samples[1:] if x[1] is not None]
        peaks["mfma_sustained_power_w_median"] = round(float(np.median(watts)), 1) if watts else None
        peaks["mfma_bf16_fp32_tflops_burst"] = round(burst, 1)
        peaks["mfma_bf16_fp32_tflops_sustained"] = round(sus_tf, 1)
        peaks["mfma_sustained_ms"] = round(sus_ms, 1)
        peaks["shader_clock_ghz_sustained"] = round(sus_clk, 3)
        out["measured_peaks"] = peaks
    mfma_meas = peaks.get("mfma_bf16_fp32_tflops_sustained")

    if args.copy_calibration:
        log("copy calibration: 3 x 256 MiB")
        nb = 256 << 20
        csrc = torch.empty(nb // 4, dtype=torch.int32, device="cuda")
        cdst = torch.empty_like(csrc)
        g.gemm_fill_launch(P(csrc), nb, 0x3C003C00, sh)
        for _ in range(3):
            g.gemm_peak_copy_launch(P(csrc), P(cdst), nb, sh)
        torch.cuda.synchronize()
        del csrc, cdst

    # ---------------- the headline workload ----------------
    log(f"workload {w.name} {w.M}x{w.N}x{w.K}")

    def step():
        g.gemm_bf16(w.M, w.N, w.K, P(A), w.K, P(B), w.N, P(C), w.N, sh)

    n_ramp = warm(lambda i: step())     # >= 300 ms: the clock settles before anything is counted
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    dispatches_before = n_ramp + args.warmup
    log(f"headline: {dispatches_before} dispatches before the timed region, {args.steps} timed")
    # the timed region: K steps back to back, bracketed by synchronisations (wall clock: `value`)
    # and by two HIP events on the launch stream (device time: the kernel's average launch
    # duration over the region, `roofline.achieved`)
    ev_t0, ev_t1 = events(2)
    t0 = time.perf_counter()
    ev_t0.record(stream)
    for _ in range(args.steps):
        step()
    ev_t1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    plan = g.gemm_last_plan()
    ms_per_step = elapsed * 1e3 / args.steps
    value = w.flops / (elapsed / args.steps) / 1e12
    kern_ms = ev_t0.elapsed_time(ev_t1) / args.steps
    achieved = w.flops / (kern_ms * 1e-3) / 1e12
    clock_ghz = clock_during(step, kern_ms)
    headline = {"dispatches_before_timed_region": dispatches_before,
                "kernel_us_mean": round(kern_ms * 1e3, 2),
                "plan": {k: plan.get(k) for k in ("kernel", "bm", "bn", "grid", "schedule",
                                                  "splits", "waves", "wave_eff")}}
    if mfma_meas:
        headline["frac_of_measured_mfma_peak"] = round(achieved / mfma_meas, 4)
    # Under this load the card runs below the clock the register-only MFMA loop holds, so the
    # matrix cores' ceiling during these launches is the measured (else published) peak scaled
    # by the clock ratio.
    headline["shader_clock_ghz_during_launches"] = round(clock_ghz, 3)
    if mfma_meas:
        at_clock = mfma_meas * clock_ghz / peaks["shader_clock_ghz_sustained"]
    else:
        at_clock = MI355X_PEAK_BF16_TFLOPS * clock_ghz / MI355X_PEAK_CLOCK_GHZ
    headline["mfma_peak_tflops_at_that_clock"] = round(at_clock, 1)
    headline["frac_of_mfma_peak_at_that_clock"] = round(achieved / at_clock, 4)
    del A, B, C

    # ---------------- every compute-bound workload ----------------
    flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB: evicts the Infinity Cache
    compute = {}
    names = [n for n in COMPUTE if not args.only or n in args.only.split(",")]
    if args.no_compute:
        names = [w.name]
    for name in names:
        wl = WORKLOADS[name]
        log(f"compute {name} {wl.M}x{wl.N}x{wl.K}")
        Al = dev(matrix("normal", wl.M, wl.K, seed=wl.seed_a, sigma=wl.sigma_a))
        Bl = dev(matrix("normal", wl.K, wl.N, seed=wl.seed_b, sigma=wl.sigma_b))
        Cl = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
        Ct = torch.empty_like(Cl)

        def ours(wl=wl, Al=Al, Bl=Bl, Cl=Cl):
            g.gemm_bf16(wl.M, wl.N, wl.K, P(Al), wl.K, P(Bl), wl.N, P(Cl), wl.N, sh)

        arms = {"ours": ours}
        if not args.no_torch:
            arms["hipblaslt"] = lambda Al=Al, Bl=Bl, Ct=Ct: torch.matmul(Al, Bl, out=Ct)
        for fn in arms.values():
            warm(lambda i, fn=fn: fn())
        t = timed_rounds(arms, 100, max(5, args.rounds))
        ours()
        torch.cuda.synchronize()
        pl = g.gemm_last_plan()
        # the same launches with the Infinity Cache flushed before each (a 1 GiB fill between
        # the launches, outside the events), so that A and B come from HBM
        cold = []
        for i in range(20):
            g.gemm_fill_launch(P(flush), 1 << 30, i, sh)
            e0, e1 = events(2)
            e0.record(stream)
            ours()
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1) * 1e3)
        med, mn = float(np.median(t["ours"])), float(t["ours"].min())
        tf = lambda us: wl.flops / (us * 1e-6) / 1e12  # noqa: E731
        rec = {"M": wl.M, "N": wl.N, "K": wl.K, "us_median": round(med, 2), "us_min": round(mn, 2),
               "us_rounds": [round(float(x), 2) for x in t["ours"]],
               "tflops_median": round(tf(med), 1), "tflops_best_round": round(tf(mn), 1),
               "us_cache_flushed_median": round(float(np.median(cold)), 2),
               "tflops_cache_flushed": round(tf(float(np.median(cold))), 1),
               "plan": {k: pl.get(k) for k in ("bm", "bn", "grid", "schedule", "splits", "waves", "wave_eff")}}
        if wl.bound == "mfma":
            rec["roofline"] = {"bound": "mfma", "achieved": round(tf(med), 1),
                               "peak": MI355X_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(tf(med) / MI355X_PEAK_BF16_TFLOPS, 4),
                               "achieved_cache_flushed": round(tf(float(np.median(cold))), 1),
                               "wave_eff": pl.get("wave_eff")}
            if mfma_meas:
                rec["frac_of_measured_mfma_peak"] = round(tf(med) / mfma_meas, 4)
                # a result above 1.05x the measured roof would be a measurement error
                rec["valid"] = bool(tf(mn) <= 1.05 * mfma_meas)
        if "hipblaslt" in t:
            hm = float(np.median(t["hipblaslt"]))
            rec.update({"hipblaslt_us_median": round(hm, 2),
                        "hipblaslt_us_min": round(float(t["hipblaslt"].min()), 2),
                        "hipblaslt_tflops_median": round(tf(hm), 1),
                        "speedup_vs_hipblaslt": round(hm / med, 3)})
        compute[name] = rec
        del Al, Bl, Cl, Ct
    del flush
    out["compute"] = compute
    if w.name in compute:
        hc = compute[w.name]
        headline["median_over_rounds_tflops"] = hc["tflops_median"]
        headline["tflops_cache_flushed"] = hc["tflops_cache_flushed"]
        if "hipblaslt_tflops_median" in hc:
            headline["torch_matmul_tflops"] = hc["hipblaslt_tflops_median"]
    out["headline"] = headline

    # ---------------- shapes outside the configurations, one per planner rule ----------------
    # (timing only, N(0,1) inputs drawn on the device; ours against hipBLASLt in the same rounds)
    PLANNER_CASES = [("last_wave_cut", 4096, 4352, 4096),     # 272 big tiles: the last 16 cut off
                     ("one_small_tile_per_cu", 1024, 4096, 11008),  # 256 tiles of 128 x 128, K split
                     ("small_tiles_1_to_2_per_cu", 512, 11008, 4096)]  # 344 tiles of 128 x 128
    if not args.no_compute and not args.no_planner_cases:
        cases = {}
        torch.manual_seed(0)
        for name, M, N, K in PLANNER_CASES:
            log(f"planner case {name} {M}x{N}x{K}")
            At = torch.randn(M, K, device="cuda").to(torch.bfloat16)
            Bt = torch.randn(K, N, device="cuda").to(torch.bfloat16)
            Ct = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            Ht = torch.empty_like(Ct)
            arms = {"ours": lambda: g.gemm_bf16(M, N, K, P(At), K, P(Bt), N, P(Ct), N, sh)}
            if not args.no_torch:
                arms["hipblaslt"] = lambda: torch.matmul(At, Bt, out=Ht)
            for f in arms.values():
                warm(lambda i, f=f: f(), ms=RAMP_MS / 2)
            arms["ours"]()
            torch.cuda.synchronize()
            pl = g.gemm_last_plan()
            t = timed_rounds(arms, 50, args.rounds)
            med = float(np.median(t["ours"]))
            flops = 2.0 * M * N * K
            rec = {"M": M, "N": N, "K": K, "us_median": round(med, 2),
                   "tflops_median": round(flops / (med * 1e-6) / 1e12, 1),
                   "plan": {k: pl.get(k) for k in ("bm", "bn", "grid", "schedule", "splits")},
                   "cut": ({"axis": pl["cut"]["axis"], "at": pl["cut"]["at"],
                            "rest": {k: pl["cut"]["rest"].get(k) for k in ("bm", "grid", "schedule", "splits")}}
                           if "cut" in pl else None)}
            if "hipblaslt" in t:
                hm = float(np.median(t["hipblaslt"]))
                rec.update({"hipblaslt_us_median": round(hm, 2), "speedup_vs_hipblaslt": round(hm / med, 3)})
            cases[name] = rec
            del At, Bt, Ct, Ht
        out["planner_cases"] = cases

    # ---------------- clock and power over a sustained product ----------------
    if not args.no_power:
        wl = WORKLOADS["sq8192"]
        log("sustained sq8192 with power/clock sampling")
        Al = dev(matrix("normal", wl.M, wl.K, seed=wl.seed_a, sigma=wl.sigma_a))
        Bl = dev(matrix("normal", wl.K, wl.N, seed=wl.seed_b, sigma=wl.sigma_b))
        Cl = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
        sampler = PowerSampler()
        e0, e1 = events(2)
        n = 0
        with sampler:
            e0.record(stream)
            t_end = time.perf_counter() + 1.5
            while time.perf_counter() < t_end:
                for _ in range(20):
                    g.gemm_bf16(wl.M, wl.N, wl.K, P(Al), wl.K, P(Bl), wl.N, P(Cl), wl.N, sh)
                n += 20
                # keep the host within a few hundred launches of the device
                if n % 200 == 0:
                    torch.cuda.synchronize()
            e1.record(stream)
            torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        watts = [s[1] for s in sampler.samples if s[1] is not None]
        out["sustained"] = {"workload": "sq8192", "launches": n, "us_mean": round(us, 2),
                            "tflops": round(wl.flops / (us * 1e-6) / 1e12, 1),
                            "sample_period_s": sampler.period,
                            "power_file": sampler.power_file, "clock_file": sampler.clock_file,
                            "samples_t_w_mhz": sampler.samples,
                            "power_w_median": round(float(np.median(watts)), 1) if watts else None}
        del Al, Bl, Cl

    # ---------------- the matrix cores on random operands ----------------
    # The register-only loop above toggles few operand bits, so it measures the matrix cores at
    # the clock limit. The products multiply random data, and under the board's power limit the
    # clock then drops: this loop (the large-tile kernel's MFMA shape and register layout, random
    # bf16 operands, no memory traffic) measures the ceiling for that data.
    if not args.no_peaks:
        log("MFMA rate on random operands")
        ops = torch.randn(3072 * 8, device="cuda").to(torch.bfloat16)
        dblocks = torch.cuda.get_device_properties(0).multi_processor_count
        dsink = torch.zeros(dblocks * 512, dtype=torch.float32, device="cuda")
        dcyc = torch.zeros(2 * dblocks, dtype=torch.int64, device="cuda")
        dflop_per_iter = dblocks * 8 * 32 * 16384

        def data_run(iters):
            e0, e1 = events(2)
            e0.record(stream)
            g.gemm_peak_mfma_data_launch(P(ops), iters, dblocks, P(dsink), P(dcyc), sh)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            c = dcyc.view(-1, 2).double()
            return dflop_per_iter * iters / (ms * 1e-3) / 1e12, ms, float((c[:, 0] / c[:, 1]).mean()) * 0.1

        t_end = time.time() + RAMP_MS / 1e3
        while time.time() < t_end:
            data_run(20000)
        sampler = PowerSampler()
        with sampler:
            rnd_tf, rnd_ms, rnd_clk = data_run(2_000_000)
        watts = [x[1] for x in sampler.samples[1:] if x[1] is not None]
        peaks["mfma_bf16_fp32_tflops_sustained_random_operands"] = round(rnd_tf, 1)
        peaks["mfma_random_operands_ms"] = round(rnd_ms, 1)
        peaks["shader_clock_ghz_random_operands"] = round(rnd_clk, 3)
        peaks["mfma_random_operands_power_w_median"] = round(float(np.median(watts)), 1) if watts else None
        headline["frac_of_random_operand_mfma_peak"] = round(achieved / rnd_tf, 4)
        for rec in compute.values():
            if "roofline" in rec:
                rec["frac_of_random_operand_mfma_peak"] = round(rec["tflops_median"] / rnd_tf, 4)
        del ops, dsink, dcyc

    # ---------------- decode workloads (HBM bound) ----------------
    if not args.no_decode:
        dec = {}
        copies = 12
        shapes = {}
        for name in sorted(n for n in WORKLOADS if n.startswith("dec_")
                           and (not args.decode or n in args.decode.split(","))):
            wd = WORKLOADS[name]
            key = (wd.K, wd.N)
            if key not in shapes:
                shapes.clear()
                log(f"decode weights {wd.K}x{wd.N} x{copies}")
                b0 = dev(matrix("normal", wd.K, wd.N, seed=wd.seed_b, sigma=wd.sigma_b))
                shapes[key] = [b0] + [b0.clone() for _ in range(copies - 1)]
                # the floor: a read-only kernel over exactly these weight bytes, cold copies,
                # single launch between events and back to back ("the decode kernel")
                wbytes = wd.K * wd.N * 2
                rsink = torch.zeros(65536, dtype=torch.int32, device="cuda")
                Bs = shapes[key]
                warm(lambda i: g.gemm_peak_read_launch(P(Bs[i % copies]), wbytes, P(rsink), sh), ms=60)
                singles = []
                for i in range(48):
                    e0, e1 = events(2)
                    e0.record(stream)
                    g.gemm_peak_read_launch(P(Bs[i % copies]), wbytes, P(rsink), sh)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    singles.append(e0.elapsed_time(e1) * 1e3)
                warm(lambda i: g.gemm_peak_read_launch(P(Bs[i % copies]), wbytes, P(rsink), sh), ms=20)
                e0, e1 = events(2)
                e0.record(stream)
                for i in range(96):
                    g.gemm_peak_read_launch(P(Bs[i % copies]), wbytes, P(rsink), sh)
                e1.record(stream)
                torch.cuda.synchronize()
                b2b = e0.elapsed_time(e1) * 1e3 / 96
                dec[f"read_floor_{wd.K}x{wd.N}"] = {
                    "bytes": wbytes, "us_single_median": round(float(np.median(singles)), 2),
                    "us_back_to_back": round(b2b, 2), "gbps_back_to_back": round(wbytes / (b2b * 1e-6) / 1e9, 1)}
            Bs = shapes[key]
            Ad = dev(matrix("normal", wd.M, wd.K, seed=wd.seed_a, sigma=wd.sigma_a))
            Cd = torch.empty((wd.M, wd.N), dtype=torch.bfloat16, device="cuda")

            def call(b):
                g.gemm_bf16(wd.M, wd.N, wd.K, P(Ad), wd.K, P(b), wd.N, P(Cd), wd.N, sh)

            warm(lambda i: call(Bs[i % copies]), ms=60)
            singles = []
            for i in range(48):
                e0, e1 = events(2)
                e0.record(stream)
                call(Bs[i % copies])
                e1.record(stream)
                torch.cuda.synchronize()
                singles.append(e0.elapsed_time(e1) * 1e3)
            nb = 96
            warm(lambda i: call(Bs[i % copies]), ms=20.0)  # (after the lone launches' idle gaps)
            b2b_rounds = []
            for _ in range(5):
                e0, e1 = events(2)
                e0.record(stream)
                for i in range(nb):
                    call(Bs[i % copies])
                e1.record(stream)
                torch.cuda.synchronize()
                b2b_rounds.append(e0.elapsed_time(e1) * 1e3 / nb)
            b2b_us = float(np.median(b2b_rounds))
            # the same calls replayed from a captured graph (one call per rotated copy), as a
            # serving loop would: launch gaps between kernels shrink, the kernels are the same
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                call(Bs[0])
            stream.wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(copies):
                    g.gemm_bf16(wd.M, wd.N, wd.K, P(Ad), wd.K, P(Bs[i]), wd.N, P(Cd), wd.N,
                                g.current_stream_handle())
            graph.replay()
            torch.cuda.synchronize()
            reps = 8
            e0, e1 = events(2)
            e0.record(stream)
            for _ in range(reps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            graph_us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
            del graph
            # a lone call replayed from a one-call graph, timed like the lone launch above
            lone = []
            for i in range(copies):
                gi = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gi):
                    g.gemm_bf16(wd.M, wd.N, wd.K, P(Ad), wd.K, P(Bs[i]), wd.N, P(Cd), wd.N,
                                g.current_stream_handle())
                lone.append(gi)
            for gi in lone:
                gi.replay()
            torch.cuda.synchronize()
            graph_singles = []
            for i in range(48):
                e0, e1 = events(2)
                e0.record(stream)
                lone[i % copies].replay()
                e1.record(stream)
                torch.cuda.synchronize()
                graph_singles.append(e0.elapsed_time(e1) * 1e3)
            del lone
            single_us = float(np.median(singles))
            gbps = wd.bytes / (b2b_us * 1e-6) / 1e9
            rec = {"us_single_median": round(single_us, 2),
                   "us_single_min": round(float(np.min(singles)), 2),
                   "us_back_to_back": round(b2b_us, 2),
                   "us_back_to_back_min": round(float(np.min(b2b_rounds)), 2),
                   "gbps_single": round(wd.bytes / (single_us * 1e-6) / 1e9, 1),
                   "gbps_back_to_back": round(gbps, 1),
                   "us_graph_replay": round(graph_us, 2),
                   "us_graph_single_median": round(float(np.median(graph_singles)), 2),
                   "gbps_graph_replay": round(wd.bytes / (graph_us * 1e-6) / 1e9, 1),
                   "algorithmic_bytes": wd.bytes,
                   "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": MI355X_PEAK_HBM_GBPS,
                                "unit": "GB/s", "frac": round(gbps / MI355X_PEAK_HBM_GBPS, 4),
                                "traffic": measured_traffic("skinny", name)},
                   "plan_splits": g.gemm_last_plan().get("splits")}
            if "hbm_copy_gbps" in peaks:
                rec["frac_of_measured_copy"] = round(gbps / peaks["hbm_copy_gbps"], 4)
                rec["valid"] = bool(gbps <= 1.05 * peaks["hbm_read_gbps"])
            fl = dec.get(f"read_floor_{wd.K}x{wd.N}")
            if fl:
                rec["us_over_read_floor_back_to_back"] = round(b2b_us - fl["us_back_to_back"], 2)
            dec[name] = rec
            del Ad, Cd
        del shapes
        out["decode"] = dec

    # ---------------- fused gate/up SwiGLU ----------------
    # silu(A Wg) * (A Wu) in one call on the K x 2N gate/up weight, against the same work in
    # PyTorch (torch.matmul into an M x 2N bf16 intermediate, then silu and multiply) and, with
    # --swiglu-unfused-ours, against this library's own product followed by the same two ops
    if not args.no_swiglu:
        import torch.nn.functional as F

        glu = {}
        for name in ("glu_prefill", "glu_dec_M1", "glu_dec_M16", "glu_dec_M64"):
            wg = WORKLOADS[name]
            log(f"swiglu {name}")
            M, N, K = wg.M, wg.N, wg.K
            copies = 1 if wg.bound == "mfma" else 12  # decode: cold weights, rotated
            b0 = dev(matrix("normal", K, 2 * N, seed=wg.seed_b, sigma=wg.sigma_b))
            Bs = [b0] + [b0.clone() for _ in range(copies - 1)]
            Ag = dev(matrix("normal", M, K, seed=wg.seed_a, sigma=wg.sigma_a))
            Hg = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            Gu = torch.empty((M, 2 * N), dtype=torch.bfloat16, device="cuda")
            Hu = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

            def fused(b):
                g.gemm_bf16_swiglu(M, N, K, P(Ag), K, P(b), 2 * N, P(Hg), N, sh)

            def unfused_ours(b):
                g.gemm_bf16(M, 2 * N, K, P(Ag), K, P(b), 2 * N, P(Gu), 2 * N, sh)
                torch.mul(F.silu(Gu[:, :N]), Gu[:, N:], out=Hu)

            def unfused_torch(b):
                torch.matmul(Ag, b, out=Gu)
                torch.mul(F.silu(Gu[:, :N]), Gu[:, N:], out=Hu)

            def per_call_us(fn, n, rounds=5):
                """Mean per call of n calls back to back between two events, per round."""
                warm(lambda i: fn(Bs[i % copies]), ms=100)
                res = []
                for _ in range(rounds):
                    e0, e1 = events(2)
                    e0.record(stream)
                    for i in range(n):
                        fn(Bs[i % copies])
                    e1.record(stream)
                    torch.cuda.synchronize()
                    res.append(e0.elapsed_time(e1) * 1e3 / n)
                return np.array(res)

            n = 20 if wg.bound == "mfma" else 96
            t_f = per_call_us(fused, n)
            plan = g.gemm_last_plan()
            med_f = float(np.median(t_f))
            rec = {"M": M, "N": N, "K": K, "us_median": round(med_f, 2),
                   "us_best_round": round(float(t_f.min()), 2),
                   "kernel": plan.get("kernel"), "strip": plan.get("strip"),
                   "grid": plan.get("grid")}
            if not args.no_torch:
                med_t = float(np.median(per_call_us(unfused_torch, n)))
                rec["torch_unfused_us_median"] = round(med_t, 2)
                rec["speedup_vs_torch_unfused"] = round(med_t / med_f, 3)
            if args.swiglu_unfused_ours:
                med_u = float(np.median(per_call_us(unfused_ours, n)))
                rec["unfused_ours_us_median"] = round(med_u, 2)
                rec["speedup_vs_unfused_ours"] = round(med_u / med_f, 3)
            if wg.bound == "mfma":
                tf = wg.flops / (med_f * 1e-6) / 1e12
                rec.update({"tflops": round(tf, 1),
                            "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                         "peak": MI355X_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                         "frac": round(tf / MI355X_PEAK_BF16_TFLOPS, 4)}})
            else:
                gb = wg.bytes / (med_f * 1e-6) / 1e9
                rec.update({"gbps": round(gb, 1),
                            "roofline": {"bound": "hbm", "achieved": round(gb, 1),
                                         "peak": MI355X_PEAK_HBM_GBPS, "unit": "GB/s",
                                         "frac": round(gb / MI355X_PEAK_HBM_GBPS, 4)}})
                if "hbm_copy_gbps" in peaks:
                    rec["frac_of_measured_copy"] = round(gb / peaks["hbm_copy_gbps"], 4)
            glu[name] = rec
            del Bs, b0, Ag, Hg, Gu, Hu
        out["swiglu"] = glu

    # ---------------- decode on packed bf16 weights (opt-in) ----------------
    if args.packed:
        pkd = {}
        copies = 12
        packed_w = {}
        for name in sorted(n for n in WORKLOADS if n.startswith("dec_")):
            wd = WORKLOADS[name]
            M, N, K = wd.M, wd.N, wd.K
            log(f"packed {name}")
            if (K, N) not in packed_w:
                packed_w.clear()
                Bh = dev(matrix("normal", K, N, seed=wd.seed_b, sigma=wd.sigma_b))
                p0 = torch.empty(K * N, dtype=torch.bfloat16, device="cuda")
                g.gemm_pack_weight_bf16(K, N, P(Bh), N, P(p0), sh)
                del Bh
                packed_w[(K, N)] = [p0] + [p0.clone() for _ in range(copies - 1)]
            ps = packed_w[(K, N)]
            Ad = dev(matrix("normal", M, K, seed=wd.seed_a, sigma=wd.sigma_a))
            Cd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

            def pk_call(i):
                g.gemm_bf16_packed(M, N, K, P(Ad), K, P(ps[i]), P(Cd), N, g.current_stream_handle())

            warm(lambda i: pk_call(i % copies), ms=60)
            e0, e1 = events(2)
            nb = 96
            e0.record(stream)
            for i in range(nb):
                pk_call(i % copies)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / nb
            plan = g.gemm_last_plan()
            gbps = wd.bytes / (us * 1e-6) / 1e9
            rec = {"us_back_to_back": round(us, 2), "gbps_back_to_back": round(gbps, 1),
                   "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": MI355X_PEAK_HBM_GBPS,
                                "unit": "GB/s", "frac": round(gbps / MI355X_PEAK_HBM_GBPS, 4)},
                   "splits": plan.get("splits"), "grid": plan.get("grid")}
            if "hbm_copy_gbps" in peaks:
                rec["frac_of_measured_copy"] = round(gbps / peaks["hbm_copy_gbps"], 4)
            pkd[name] = rec
            del Ad, Cd
        del packed_w
        out["packed_decode"] = pkd

    # ---------------- block-scaled decode (MXFP8 activations x MXFP4 weights) ----------------
    # the decode shapes with the weight in the nn.Linear layout (N x K) packed to MXFP4 once;
    # timed on pre-quantised activations (the product alone) and from bf16 activations
    # (quantisation launch + product), 16 rotated weight copies (384 MB) so every call reads cold
    if not args.no_mx:
        mxd = {}
        copies = 16
        packed = {}
        for name in ("dec_up_M1", "dec_up_M16", "dec_up_M64", "dec_down_M1", "dec_down_M64"):
            wd = WORKLOADS[name]
            M, N, K = wd.M, wd.N, wd.K
            log(f"mx {name}")
            if (N, K) not in packed:
                packed.clear()
                W = dev(matrix("normal", N, K, seed=wd.seed_b, sigma=wd.sigma_b))
                wb, sb = g.gemm_mx_packed_sizes(N, K)
                wp0 = torch.empty(wb, dtype=torch.uint8, device="cuda")
                sp0 = torch.empty(sb, dtype=torch.uint8, device="cuda")
                g.gemm_mx_pack_weight(N, K, P(W), K, P(wp0), P(sp0), sh)
                del W
                packed[(N, K)] = ([wp0] + [wp0.clone() for _ in range(copies - 1)],
                                  [sp0] + [sp0.clone() for _ in range(copies - 1)], wb, sb)
            wps, sps, wb, sb = packed[(N, K)]
            Ad = dev(matrix("normal", M, K, seed=wd.seed_a, sigma=wd.sigma_a))
            aq = torch.empty(M * K, dtype=torch.uint8, device="cuda")
            asc = torch.empty(M * K // 32, dtype=torch.uint8, device="cuda")
            g.gemm_mx_quantize_act(M, K, P(Ad), K, P(aq), K, P(asc), K // 32, sh)
            Cd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

            def b2b_us(fn, n=160):
                warm(lambda i: fn(i % copies), ms=60)
                e0, e1 = events(2)
                e0.record(stream)
                for i in range(n):
                    fn(i % copies)
                e1.record(stream)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / n

            def mx_call(i):
                g.gemm_mx_decode(M, N, K, P(aq), K, P(asc), K // 32, P(wps[i]), P(sps[i]), P(Cd), N,
                                 g.current_stream_handle())

            def mx_bf16_call(i):
                g.gemm_mx_decode_bf16(M, N, K, P(Ad), K, P(wps[i]), P(sps[i]), P(Cd), N,
                                      g.current_stream_handle())

            def graph_us(fn, reps=10):
                """Per call, the calls over every weight copy captured once and replayed: the
                device time back to back, without the host's per-call cost (a call here takes
                about as long to issue from Python as the kernel takes to run)."""
                side = torch.cuda.Stream()
                side.wait_stream(stream)
                with torch.cuda.stream(side):
                    fn(0)
                stream.wait_stream(side)
                torch.cuda.synchronize()
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    for i in range(copies):
                        fn(i)
                gr.replay()
                torch.cuda.synchronize()
                e0, e1 = events(2)
                e0.record(stream)
                for _ in range(reps):
                    gr.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                del gr
                return e0.elapsed_time(e1) * 1e3 / (reps * copies)

            us_eager = b2b_us(lambda i: g.gemm_mx_decode(M, N, K, P(aq), K, P(asc), K // 32, P(wps[i]),
                                                         P(sps[i]), P(Cd), N, sh))
            plan = g.gemm_last_plan()
            us = graph_us(mx_call)
            us_q = graph_us(mx_bf16_call)
            nbytes = wb + sb + M * K + M * K // 32 + 2 * M * N
            gbps = nbytes / (us * 1e-6) / 1e9
            rec = {"M": M, "N": N, "K": K, "us_graph_replay": round(us, 2),
                   "us_eager_back_to_back": round(us_eager, 2),
                   "us_with_activation_quantisation_graph_replay": round(us_q, 2),
                   "algorithmic_bytes": nbytes, "gbps": round(gbps, 1),
                   "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": MI355X_PEAK_HBM_GBPS,
                                "unit": "GB/s", "frac": round(gbps / MI355X_PEAK_HBM_GBPS, 4)},
                   "tiles_per_group": plan.get("strip", 0) // 16, "splits": plan.get("splits"),
                   "grid": plan.get("grid")}
            if "hbm_copy_gbps" in peaks:
                rec["frac_of_measured_copy"] = round(gbps / peaks["hbm_copy_gbps"], 4)
            bf = out.get("decode", {}).get(name, {}).get("us_graph_replay")
            if bf:
                rec["bf16_skinny_us_graph_replay"] = bf
                rec["speedup_vs_bf16"] = round(bf / us, 3)
                rec["speedup_vs_bf16_with_quantisation"] = round(bf / us_q, 3)
            mxd[name] = rec
            del Ad, aq, asc, Cd
        del packed
        out["mx_decode"] = mxd

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu:
        import oracle

        log("cpu oracle baseline")
        Ah = matrix("normal", w.M, w.K, seed=w.seed_a, sigma=w.sigma_a)
        Bh = matrix("normal", w.K, w.N, seed=w.seed_b, sigma=w.sigma_b)
        threads = oracle.default_threads()
        rows_done, t_cpu = 0, 0.0
        block = 64
        while t_cpu < args.cpu_seconds and rows_done < w.M:
            nr = min(block, w.M - rows_done)
            t1 = time.perf_counter()
            oracle.gemm_rows(Ah, Bh, rows_done, nr, w.N, w.K, with_abs=True, threads=threads)
            t_cpu += time.perf_counter() - t1
            rows_done += nr
        flops = 2.0 * rows_done * w.N * w.K
        cpu = {"value": round(flops / t_cpu / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle",
               "sample": f"rows 0..{rows_done - 1} of the {w.name} product "
                         f"({rows_done}x{w.N}x{w.K}, float64 value and |a*b| sums), {t_cpu:.1f} s"}

    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MI355X_PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MI355X_PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("tile", w.name)}
    if w.name in compute:
        roofline["achieved_cache_flushed"] = compute[w.name]["tflops_cache_flushed"]
        roofline["frac_cache_flushed"] = round(compute[w.name]["tflops_cache_flushed"] / MI355X_PEAK_BF16_TFLOPS, 4)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "inputs": f"A~N(0,{w.sigma_a}), B~N(0,{w.sigma_b}) bf16, seeds "
                             f"{w.seed_a:#x}/{w.seed_b:#x}", "parallelism": "none"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    line.update(out)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
