"""Parity of the HIP path with the float64 oracle, through the C ABI, on an MI355X.

Every product is checked element by element: for floating inputs against
|c - ref| <= 2^-8 |ref| + 2^-16 sum|a b| and a relative Frobenius error <= 4e-3 (the oracle's
check); for integer-valued inputs (all partial sums exact in float32) bit for bit against the
oracle's round-to-nearest-even of the exact result. Outputs are poisoned with NaN before each
call so a skipped tile cannot pass on stale data. Full-size workloads run in the launch
configuration the benchmark times (the dispatching entry point) and are compared on sampled
rows, plus closed-form properties (all-ones gives K everywhere) over every element.
"""

import ctypes

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemv_layers_amd as g  # noqa: E402

POISON = 0x7FC07FC0  # two bf16 quiet NaNs


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    g.gemm_init(0)
    yield


def dev(h: np.ndarray) -> "torch.Tensor":
    t = torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def host(t: "torch.Tensor") -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


ENTRIES = {"auto": g.gemm_bf16, "tiled": g.gemm_bf16_tiled, "skinny": g.gemm_bf16_skinny}


def run(entry, A, B, M, N, K, ldc=None, C=None):
    """Call the library on host bf16-bit arrays A (M x lda) and B (K x ldb); returns C bits."""
    ldc = N if ldc is None else ldc
    dA, dB = dev(A), dev(B)
    if C is None:
        n = -(-max(M * ldc, 8) // 8) * 8      # whole 16-byte units for the poison fill
        C = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        g.gemm_fill_launch(ctypes.c_void_p(C.data_ptr()), C.numel() * 2, POISON)
    s = g.current_stream_handle()
    ENTRIES[entry](M, N, K, ctypes.c_void_p(dA.data_ptr()), A.shape[1] if A.size else max(K, 1),
                   ctypes.c_void_p(dB.data_ptr()), B.shape[1] if B.size else max(N, 1),
                   ctypes.c_void_p(C.data_ptr()), ldc, s)
    torch.cuda.synchronize()
    return host(C)[: M * ldc].reshape(M, ldc)[:, :N]


def check_float(C, A, B, M, N, K, what=""):
    ref, sabs = oracle.gemm(A, B, M=M, N=N, K=K)
    res = oracle.check(C, ref, sabs)
    assert res.ok, f"{what} {res.summary()}"
    return res


def check_exact(C, A, B, M, N, K, what=""):
    ref, _ = oracle.gemm(A, B, M=M, N=N, K=K, with_abs=False)
    want = oracle.bf16_rne(ref)
    bad = np.argwhere(C != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[0].tolist()}"


# ---- small and ragged shapes, each kernel family --------------------------------------------

TILE_SHAPES = [(256, 256, 64), (512, 512, 512), (300, 520, 328), (1000, 1000, 1000),
               (65, 264, 72), (1, 8, 8), (257, 264, 4104), (513, 1032, 136),
               # 128 x 128 tiles up to two per CU (320 and 371 tiles), ragged in M, N and K
               (1000, 5000, 328), (777, 6704, 200),
               # 256 x 256 tiles in a partial wave (144 and 172 tiles), ragged in M, N and K
               (1000, 9000, 328), (777, 11000, 200),
               # exactly one 128 x 128 tile per CU (256) and 97 k-steps: K split in two, ragged
               (1000, 4000, 3080)]


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_tile_kernel_float_and_exact(M, N, K):
    A = matrix("normal", M, K, seed=1000 + M)
    B = matrix("normal", K, N, seed=2000 + N, sigma=0.5)
    check_float(run("tiled", A, B, M, N, K), A, B, M, N, K, f"tiled {M}x{N}x{K}")
    Ai = matrix("int", M, K, seed=3000 + M)
    Bi = matrix("int", K, N, seed=4000 + N)
    check_exact(run("tiled", Ai, Bi, M, N, K), Ai, Bi, M, N, K, f"tiled int {M}x{N}x{K}")
    big, small = (-(-M // 256)) * (-(-N // 256)), (-(-M // 128)) * (-(-N // 128))
    # 256 x 256 tiles from one full wave of them, or when 128 x 128 ones would need three per CU
    plan = g.gemm_last_plan()
    assert plan["bm"] == (256 if big >= 256 or small > 512 else 128)
    if (M, N, K) == (1000, 4000, 3080):
        assert plan["splits"] == 2 and plan["grid"] == 512


SKINNY_SHAPES = [(m, n, k) for m in (1, 2, 3, 16, 17, 33, 64)
                 for (n, k) in ((1000, 1000), (264, 4104), (4104, 320))]


@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_skinny_kernel_float_and_exact(M, N, K):
    A = matrix("normal", M, K, seed=5000 + M)
    B = matrix("normal", K, N, seed=6000 + N, sigma=0.02)
    check_float(run("skinny", A, B, M, N, K), A, B, M, N, K, f"skinny {M}x{N}x{K}")
    Ai = matrix("int", M, K, seed=7000 + M)
    Bi = matrix("int", K, N, seed=8000 + N)
    check_exact(run("skinny", Ai, Bi, M, N, K), Ai, Bi, M, N, K, f"skinny int {M}x{N}x{K}")


# Stream-K ranges of the skinny kernel that cross strip boundaries: with too few strips of
# either width for an aligned grid to fill two thirds of the CUs (more than 256 strips of 128
# columns and 129..170 of 256), or, for three or more 16-row tiles of M, an aligned grid that
# leaves a sixteenth of the CUs idle, 256 ranges cut the strips wherever they fall. A range may end
# inside a strip (announced at the range's end) or contain a strip's end (announced mid-stream);
# ragged N and K included.
STREAMK_SHAPES = [(3, 256 * 150 + 8, 64 * 17 + 8), (1, 256 * 140, 64 * 20), (2, 256 * 135 + 24, 64 * 15 + 24),
                  (33, 128 * 131, 2056), (64, 128 * 145, 64 * 16)]


@pytest.mark.parametrize("M,N,K", STREAMK_SHAPES)
def test_skinny_stream_k_boundaries(M, N, K):
    plan = g.gemm_plan_describe(M, N, K, 256, 1)
    assert plan["kernel"] == "skinny"
    U, G, ks = plan["strips"] * plan["ks"], plan["grid"], plan["ks"]
    ranges = [(w * U // G, (w + 1) * U // G) for w in range(G)]
    crossing = [(b, e) for b, e in ranges if b // ks != (e - 1) // ks]
    assert crossing, "some range must span two strips"
    A = matrix("normal", M, K, seed=5100 + M)
    B = matrix("normal", K, N, seed=6100 + N, sigma=0.02)
    check_float(run("skinny", A, B, M, N, K), A, B, M, N, K, f"skinny {M}x{N}x{K}")
    Ai = matrix("int", M, K, seed=7100 + M)
    Bi = matrix("int", K, N, seed=8100 + N)
    check_exact(run("skinny", Ai, Bi, M, N, K), Ai, Bi, M, N, K, f"skinny int {M}x{N}x{K}")


# Aligned layouts (grid = strips x pieces, every range one piece of one strip), with 128- and
# 256-column strips: few pieces on two thirds of the CUs, and strips cut into many pieces (long
# fixups in batches), for one to four 16-row tiles of M.
ALIGNED_SHAPES = [(1, 128 * 65, 4096), (5, 128 * 65 + 8, 1000), (64, 128 * 9, 64 * 300), (1, 128 * 7, 64 * 400),
                  (17, 128 * 7 + 40, 64 * 300 + 8), (40, 128 * 11, 12872)]


@pytest.mark.parametrize("M,N,K", ALIGNED_SHAPES)
def test_skinny_aligned_layouts(M, N, K):
    plan = g.gemm_plan_describe(M, N, K, 256, 1)
    assert plan["kernel"] == "skinny" and plan["grid"] % plan["strips"] == 0
    A = matrix("normal", M, K, seed=5200 + M)
    B = matrix("normal", K, N, seed=6200 + N, sigma=0.02)
    check_float(run("skinny", A, B, M, N, K), A, B, M, N, K, f"skinny {M}x{N}x{K}")
    Ai = matrix("int", M, K, seed=7200 + M)
    Bi = matrix("int", K, N, seed=8200 + N)
    check_exact(run("skinny", Ai, Bi, M, N, K), Ai, Bi, M, N, K, f"skinny int {M}x{N}x{K}")


# Aligned layouts with 2, 4 or 8 pieces per strip at one or two 16-row tiles keep the hardware's
# round-robin dealing of workgroups to XCDs (no remap): grids that are and are not multiples of 8,
# ragged N and K.
HW_ORDER_SHAPES = [(1, 128 * 112 + 8, 1000), (3, 128 * 64 - 8, 64 * 50 + 8), (2, 128 * 32, 64 * 100 + 24),
                   (32, 128 * 31 + 40, 64 * 90 + 8), (9, 128 * 120, 520)]


@pytest.mark.parametrize("M,N,K", HW_ORDER_SHAPES)
def test_skinny_hardware_xcd_order(M, N, K):
    plan = g.gemm_plan_describe(M, N, K, 256, 1)
    assert plan["kernel"] == "skinny" and plan["nxcd"] == 1 and plan["grid"] == plan["strips"] * plan["splits"]
    A = matrix("normal", M, K, seed=5300 + M)
    B = matrix("normal", K, N, seed=6300 + N, sigma=0.02)
    check_float(run("skinny", A, B, M, N, K), A, B, M, N, K, f"skinny {M}x{N}x{K}")
    Ai = matrix("int", M, K, seed=7300 + M)
    Bi = matrix("int", K, N, seed=8300 + N)
    check_exact(run("skinny", Ai, Bi, M, N, K), Ai, Bi, M, N, K, f"skinny int {M}x{N}x{K}")
    assert g.gemm_last_plan()["nxcd"] == 1


GENERIC_SHAPES = [(17, 15, 63), (5, 33, 1), (70, 9, 100), (1, 1, 1), (130, 67, 255)]


@pytest.mark.parametrize("M,N,K", GENERIC_SHAPES)
def test_general_kernel_odd_shapes(M, N, K):
    A = matrix("normal", M, K, seed=9000 + M)
    B = matrix("normal", K, N, seed=9100 + N)
    C = run("auto", A, B, M, N, K)
    assert g.gemm_last_plan()["kernel"] == "generic"
    check_float(C, A, B, M, N, K, f"generic {M}x{N}x{K}")
    Ai, Bi = matrix("int", M, K, seed=9200), matrix("int", K, N, seed=9300)
    check_exact(run("auto", Ai, Bi, M, N, K), Ai, Bi, M, N, K)


@pytest.mark.parametrize("entry", ["tiled", "skinny", "auto"])
def test_leading_dimensions_never_read_padding(entry):
    # padding columns hold NaN: a kernel that reads them produces NaN and fails
    M, N, K = (48, 264, 200) if entry != "tiled" else (300, 264, 200)
    A = matrix("normal", M, K, seed=11, ld=K + 24)
    B = matrix("normal", K, N, seed=12, ld=N + 16)
    C = run(entry, A, B, M, N, K, ldc=N + 8)
    ref, sabs = oracle.gemm(A, B, M=M, N=N, K=K)
    assert oracle.check(C, ref, sabs).ok


@pytest.mark.parametrize("entry,M,ld_extra,kernel", [("tiled", 256, 0, "tile"), ("skinny", 64, 0, "skinny"),
                                                     ("auto", 256, 8, "generic")])
def test_largest_leading_dimensions(entry, M, ld_extra, kernel):
    # the fast kernels take leading dimensions up to 2^20 elements (32-bit buffer offsets over
    # a tile's rows); one more 16-byte unit sends the call to the general kernel
    LD = (1 << 20) + ld_extra
    N, K = 136, 72
    A = matrix("normal", M, K, seed=21, ld=LD)
    B = matrix("normal", K, N, seed=22, ld=LD)
    C = run(entry, A, B, M, N, K, ldc=LD)
    assert g.gemm_last_plan()["kernel"] == kernel
    check_float(C, A, B, M, N, K, f"{entry} ld={LD}")


def test_dispatch_on_m():
    A64, A65 = matrix("int", 64, 512, seed=1), matrix("int", 65, 512, seed=1)
    B = matrix("int", 512, 1024, seed=2)
    check_exact(run("auto", A64, B, 64, 1024, 512), A64, B, 64, 1024, 512)
    assert g.gemm_last_plan()["kernel"] == "skinny"
    check_exact(run("auto", A65, B, 65, 1024, 512), A65, B, 65, 1024, 512)
    assert g.gemm_last_plan()["kernel"] == "tile"


def test_degenerate_shapes():
    A = np.zeros((8, 8), np.uint16)
    B = np.zeros((8, 16), np.uint16)
    C = run("auto", A, B, 8, 16, 0)             # K = 0: the empty sum
    assert np.all(C == 0)
    Cd = torch.empty(64, dtype=torch.bfloat16, device="cuda")
    g.gemm_fill_launch(ctypes.c_void_p(Cd.data_ptr()), 128, POISON)
    dA, dB = dev(A), dev(B)
    g.gemm_bf16(0, 16, 8, ctypes.c_void_p(dA.data_ptr()), 8, ctypes.c_void_p(dB.data_ptr()), 16,
                ctypes.c_void_p(Cd.data_ptr()), 16, g.current_stream_handle())
    torch.cuda.synchronize()
    assert np.all(host(Cd) == 0x7FC0)           # M = 0: nothing written


def _rne_golden():
    import os
    rows = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "rne_ties.txt")):
        line = line.split("#")[0].strip()
        if line:
            x, bits = line.split()[:2]
            rows.append((float(x), int(bits, 16)))
    return rows


@pytest.mark.parametrize("entry,M", [("tiled", 256), ("skinny", 16), ("auto", 5)])
def test_epilogue_rounds_to_nearest_even(entry, M):
    # c = a0*b0 + a1*b1 with a = [1, 1]: b0 = 4096, b1 = x - 4096 gives the golden tie cases
    ties = [(x, b) for x, b in _rne_golden() if 4096 <= abs(x) <= 4160]
    N, K = 264, 64
    A = np.zeros((M, K), np.uint16)
    A[:, 0] = 0x3F80
    A[:, 1] = 0x3F80
    B = np.zeros((K, N), np.uint16)
    want = np.zeros(N, np.uint16)
    for j in range(N):
        x, bits = ties[j % len(ties)]
        sgn = -1.0 if x < 0 else 1.0
        B[0, j] = oracle.bf16_rne(sgn * 4096.0)[0]
        B[1, j] = oracle.bf16_rne(x - sgn * 4096.0)[0]
        want[j] = bits
    C = run(entry, A, B, M, N, K)
    assert np.all(C == want[None, :])


# ---- a sparse last wave of 256 x 256 tiles cut off as a strip -----------------------------
# (the planner keeps the whole waves' rectangle and plans the strip left over on its own; both
# launches write C, so every row sampled crosses the column cut, and rows on both sides of a row
# cut are sampled)
CUT_SHAPES = [(4096, 4352, 1024, "n", 4096),   # 272 tiles: 16 in the last wave
              (4000, 4400, 1000, "n", 4096),   # ragged M, N, K: 288 tiles
              (4352, 4096, 1024, "m", 4096),   # a row cut keeps 256 tiles, a column cut 255
              (8192, 8448, 512, "n", 8192)]    # after four full waves


@pytest.mark.parametrize("M,N,K,axis,at", CUT_SHAPES)
def test_sparse_last_wave_cut(M, N, K, axis, at):
    A = matrix("normal", M, K, seed=7000 + M)
    B = matrix("normal", K, N, seed=8000 + N, sigma=0.5)
    C = run("auto", A, B, M, N, K)
    plan = g.gemm_last_plan()
    assert plan["bm"] == 256 and plan["cut"]["axis"] == axis and plan["cut"]["at"] == at, plan
    assert plan["cut"]["rest"]["bm"] == 128
    rows = np.unique(np.concatenate([_sample_rows(M, 24), [at - 1, at, min(at + 1, M - 1)]]))
    rows = rows[rows < M]
    ref, sabs = oracle.gemm(np.ascontiguousarray(A[rows]), B, M=len(rows), N=N, K=K)
    res = oracle.check(np.ascontiguousarray(C[rows]), ref, sabs)
    assert res.ok, f"cut {M}x{N}x{K} {res.summary()}"
    Ai = matrix("int", M, K, seed=7100 + M)
    Bi = matrix("int", K, N, seed=8100 + N)
    Ci = run("auto", Ai, Bi, M, N, K)
    ref, _ = oracle.gemm(np.ascontiguousarray(Ai[rows]), Bi, M=len(rows), N=N, K=K, with_abs=False)
    bad = np.argwhere(Ci[rows] != oracle.bf16_rne(ref))
    assert bad.size == 0, f"cut int {M}x{N}x{K}: {len(bad)} mismatches, first {bad[0].tolist()}"


# Ragged products whose plan cuts a sparse last wave off, three per direction, drawn once from
# a seeded generator (M and N uniform in 2000-9000, multiples of 8; K a multiple of 8 up to 1024,
# so sampled rows stay cheap for the oracle) and kept as data so that collecting the tests needs
# no library: (M, N, K, direction, position of the cut). One leaves a strip of 8 rows.
RANDOM_CUT_CASES = [(5376, 3312, 400, "n", 3072), (4792, 3800, 992, "m", 4352),
                    (6408, 4936, 584, "m", 6400), (4152, 8616, 320, "n", 7680),
                    (2792, 7592, 416, "n", 5888), (5088, 4120, 304, "m", 3840)]


@pytest.mark.parametrize("M,N,K,axis,at", RANDOM_CUT_CASES)
def test_random_cut_shapes_integer_exact(M, N, K, axis, at):
    Ai = matrix("int", M, K, seed=7200 + M)
    Bi = matrix("int", K, N, seed=8200 + N)
    C = run("auto", Ai, Bi, M, N, K)
    plan = g.gemm_last_plan()
    assert (plan["cut"]["axis"], plan["cut"]["at"]) == (axis, at), plan
    rows = np.unique(np.concatenate([_sample_rows(M, 12), [at - 1, at, min(at + 1, M - 1)] if axis == "m" else []]))
    rows = rows[(rows >= 0) & (rows < M)].astype(np.int64)
    ref, _ = oracle.gemm(np.ascontiguousarray(Ai[rows]), Bi, M=len(rows), N=N, K=K, with_abs=False)
    bad = np.argwhere(C[rows] != oracle.bf16_rne(ref))
    assert bad.size == 0, f"cut int {M}x{N}x{K} {axis}@{at}: {len(bad)} mismatches, first {bad[0].tolist()}"


# ---- full-size workloads, in the benchmark's launch configuration -------------------------

FULL = ["sq512", "sq4096", "sq8192", "sq16384", "mlp_up", "mlp_down"] + \
       [n for n in WORKLOADS if n.startswith("dec_")]


def _sample_rows(M, n):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(M)
    return np.unique(np.concatenate([[0, M - 1, M // 2], rng.choice(M, n - 3, replace=False)]))


@pytest.mark.parametrize("name", FULL)
def test_workload_full_size(name):
    w = WORKLOADS[name]
    A = matrix("normal", w.M, w.K, seed=w.seed_a, sigma=w.sigma_a)
    B = matrix("normal", w.K, w.N, seed=w.seed_b, sigma=w.sigma_b)
    C = run("auto", A, B, w.M, w.N, w.K)
    # every row where the host oracle (float64 value and |a b| sums) takes seconds, up to 8192^3;
    # 16384^3 on sampled rows (its every element is checked against a closed form below)
    rows = np.arange(w.M) if w.flops <= 1.2e12 else _sample_rows(w.M, 24)
    As = np.ascontiguousarray(A[rows])
    ref, sabs = oracle.gemm(As, B, M=len(rows), N=w.N, K=w.K)
    res = oracle.check(np.ascontiguousarray(C[rows]), ref, sabs)
    assert res.ok, f"{name} rows={len(rows)} {res.summary()}"


@pytest.mark.parametrize("name", FULL)
def test_workload_all_ones_every_element(name):
    w = WORKLOADS[name]
    A = np.full((w.M, w.K), 0x3F80, np.uint16)
    B = np.full((w.K, w.N), 0x3F80, np.uint16)
    C = run("auto", A, B, w.M, w.N, w.K)
    want = oracle.bf16_rne(float(w.K))
    bad = np.count_nonzero(C != want)
    assert bad == 0, f"{name}: {bad} elements differ from K = {w.K}"


# Integer-valued inputs in {-4 .. 4}: every partial sum is an integer below 16 K <= 2^18, exact in
# float32 in any order, so the result must equal the oracle's rounding of the exact sum bit for
# bit. Every workload shape, plus ragged shapes at the same scale (a partial last tile in M, N and
# K, and a decode shape whose N and K are not multiples of the strip or the stage).
INT_SHAPES = [(n, WORKLOADS[n].M, WORKLOADS[n].N, WORKLOADS[n].K) for n in FULL] + \
             [("ragged_prefill", 4000, 11000, 4104), ("ragged_square", 8200, 8200, 8200),
              ("ragged_decode", 37, 11000, 4100)]


@pytest.mark.parametrize("name,M,N,K", INT_SHAPES)
def test_workload_integer_exact_sampled(name, M, N, K):
    seed = WORKLOADS[name].seed_a if name in WORKLOADS else 0x5EED1000 + M
    A = matrix("int", M, K, seed=seed)
    B = matrix("int", K, N, seed=seed + 1)
    C = run("auto", A, B, M, N, K)
    rows = _sample_rows(M, 32 if M * N <= (1 << 26) else 16)
    ref, _ = oracle.gemm(np.ascontiguousarray(A[rows]), B, M=len(rows), N=N, K=K, with_abs=False)
    want = oracle.bf16_rne(ref)
    bad = np.argwhere(C[rows] != want)
    assert bad.size == 0, f"{name}: {len(bad)} mismatches, first {bad[0].tolist()}"


# ---- determinism and workspace hygiene -------------------------------------------------------

@pytest.mark.parametrize("name", ["sq4096", "sq512", "dec_down_M64", "dec_up_M1"])
def test_bitwise_deterministic_and_workspace_clean(name):
    w = WORKLOADS[name]
    A = matrix("normal", w.M, w.K, seed=w.seed_a, sigma=w.sigma_a)
    B = matrix("normal", w.K, w.N, seed=w.seed_b, sigma=w.sigma_b)
    first = run("auto", A, B, w.M, w.N, w.K)
    # interleave other shapes that use the same workspace, then repeat
    other = matrix("normal", 3, 1000, seed=5)
    ob = matrix("normal", 1000, 4104, seed=6)
    for _ in range(3):
        run("skinny", other, ob, 3, 4104, 1000)
        again = run("auto", A, B, w.M, w.N, w.K)
        assert np.array_equal(first, again), name


def test_many_back_to_back_calls_stay_correct():
    # 200 launches on one stream with no synchronisation in between; the split-K counters must
    # return to zero every time or later calls would lose their fixup
    M, N, K = 16, 4096, 11008
    A = matrix("int", M, K, seed=1)
    B = matrix("int", K, N, seed=2)
    dA, dB = dev(A), dev(B)
    outs = [torch.empty(M * N, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    s = g.current_stream_handle()
    for i in range(200):
        C = outs[i % 4]
        g.gemm_fill_launch(ctypes.c_void_p(C.data_ptr()), C.numel() * 2, POISON, s)
        g.gemm_bf16(M, N, K, ctypes.c_void_p(dA.data_ptr()), K, ctypes.c_void_p(dB.data_ptr()), N,
                    ctypes.c_void_p(C.data_ptr()), N, s)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(A, B, with_abs=False)
    want = oracle.bf16_rne(ref)
    for C in outs:
        assert np.array_equal(host(C).reshape(M, N), want)


# ---- graph capture ---------------------------------------------------------------------------
# The kernels allocate nothing and need no memset: split counters return to zero inside the
# kernel, so one captured call replays correctly any number of times. Each case mixes the
# counter-using layouts (aligned split pieces, Stream-K ranges across strips, tile split-K);
# between replays, eager work poisons the output and runs other shapes over the shared
# workspace, and every replay must equal the eager result bit for bit.
GRAPH_CASES = [("auto", 1, 4096, 11008), ("skinny", 3, 128 * 141 + 8, 64 * 37 + 8),
               ("auto", 64, 11008, 4096), ("tiled", 1000, 1000, 1000),
               ("auto", 4096, 4352, 1024)]  # a sparse last wave cut off: two kernels


class _KernelNodeParams(ctypes.Structure):  # hipKernelNodeParams
    _fields_ = [("blockDim", ctypes.c_uint * 3), ("extra", ctypes.c_void_p), ("func", ctypes.c_void_p),
                ("gridDim", ctypes.c_uint * 3), ("kernelParams", ctypes.c_void_p),
                ("sharedMemBytes", ctypes.c_uint)]


def graph_nodes(graph):
    """(node type, kernel name or None) for every node of a captured, kept graph.

    Uses the HIP runtime the process already has mapped (torch's), so the graph handle is valid
    for it. Node type 0 is a kernel node, 2 a memset node.
    """
    paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln})
    assert len(paths) == 1, f"expected one HIP runtime in the process, found {paths}"
    hip = ctypes.CDLL(paths[0])
    hip.hipKernelNameRefByPtr.restype = ctypes.c_char_p
    hip.hipKernelNameRefByPtr.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    handle = ctypes.c_void_p(graph.raw_cuda_graph())
    count = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(handle, None, ctypes.byref(count)) == 0
    nodes = (ctypes.c_void_p * max(count.value, 1))()
    assert hip.hipGraphGetNodes(handle, nodes, ctypes.byref(count)) == 0
    out = []
    for i in range(count.value):
        kind = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(kind)) == 0
        name = None
        if kind.value == 0:
            prm = _KernelNodeParams()
            assert hip.hipGraphKernelNodeGetParams(ctypes.c_void_p(nodes[i]), ctypes.byref(prm)) == 0
            raw = hip.hipKernelNameRefByPtr(prm.func, None)
            name = raw.decode() if raw else ""
        out.append((kind.value, name))
    return out


@pytest.mark.parametrize("entry,M,N,K", GRAPH_CASES)
def test_graph_replay_matches_eager(entry, M, N, K):
    A = matrix("normal", M, K, seed=9100 + M)
    B = matrix("normal", K, N, seed=9200 + N, sigma=0.02)
    eager = run(entry, A, B, M, N, K)
    check_float(eager, A, B, M, N, K, f"{entry} {M}x{N}x{K} eager")
    dA, dB = dev(A), dev(B)
    C = torch.empty(M * N, dtype=torch.bfloat16, device="cuda")
    other = [(2, 8320, 4096), (300, 520, 328)]
    oA = [dev(matrix("normal", m, k, seed=9300 + m)) for m, n, k in other]
    oB = [dev(matrix("normal", k, n, seed=9400 + n)) for m, n, k in other]
    oC = [torch.empty(m * n, dtype=torch.bfloat16, device="cuda") for m, n, k in other]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture expects
        ENTRIES[entry](M, N, K, ctypes.c_void_p(dA.data_ptr()), K, ctypes.c_void_p(dB.data_ptr()), N,
                       ctypes.c_void_p(C.data_ptr()), N, g.current_stream_handle())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g.gemm_fill_launch(ctypes.c_void_p(C.data_ptr()), C.numel() * 2, POISON)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(graph):
        ENTRIES[entry](M, N, K, ctypes.c_void_p(dA.data_ptr()), K, ctypes.c_void_p(dB.data_ptr()), N,
                       ctypes.c_void_p(C.data_ptr()), N, g.current_stream_handle())
    torch.cuda.synchronize()
    # the capture recorded the product as its kernel nodes (one, or two for a plan cut in two; no
    # memset node), and ran nothing
    nodes = graph_nodes(graph)
    family = "skinny_gemm_kernel" if entry == "skinny" or (entry == "auto" and M <= 64) else "tile_"
    launches = 2 if "cut" in g.gemm_plan_describe(M, N, K, skinny=entry == "skinny") else 1
    assert len(nodes) == launches and all(k == 0 for k, _ in nodes), \
        f"{entry} {M}x{N}x{K}: captured nodes {nodes}"
    assert all(family in name for _, name in nodes), f"{entry} {M}x{N}x{K}: captured kernels {nodes}"
    assert np.all(host(C) == np.uint16(POISON & 0xFFFF)), "capture wrote C"
    graph.instantiate()
    for rep in range(4):
        g.gemm_fill_launch(ctypes.c_void_p(C.data_ptr()), C.numel() * 2, POISON)
        (m, n, k), a, b, c = other[rep % 2], oA[rep % 2], oB[rep % 2], oC[rep % 2]
        g.gemm_bf16(m, n, k, ctypes.c_void_p(a.data_ptr()), k, ctypes.c_void_p(b.data_ptr()), n,
                    ctypes.c_void_p(c.data_ptr()), n, g.current_stream_handle())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host(C).reshape(M, N)
        assert np.array_equal(got, eager), f"replay {rep} of {entry} {M}x{N}x{K} differs from eager"


# ---- measurement kernels ---------------------------------------------------------------------

def _check_mfma_sink(sink, iters):
    """The peak loop's accumulators in closed form. Each wave runs 8 identical chains of
    v_mfma_f32_32x32x16_bf16 on fixed operands: lane l holds row (A) or column (B) l % 32 and
    k = 8 (l // 32) + e in its element e, with a = 1 + ((l + e) & 7) / 128 and
    b = 1/2 - ((3 l + e) & 7) / 128. After `iters` steps every chain holds iters * (A B), and
    lanes l and l + 32 together hold all 32 rows of column l % 32, so the two lanes' sinks add up
    to 8 * iters * (column sum of A B)."""
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for lane in range(64):
        for e in range(8):
            k = 8 * (lane // 32) + e
            A[lane % 32, k] = 1.0 + ((lane + e) & 7) / 128.0
            B[k, lane % 32] = 0.5 - ((3 * lane + e) & 7) / 128.0
    colsum = (A @ B).sum(axis=0)  # exact: multiples of 2^-14 well inside float64
    want = 8.0 * iters * colsum
    for wave in range(4):
        w = sink[:, 64 * wave:64 * wave + 64]
        got = w[:, :32] + w[:, 32:]
        assert np.all(np.abs(got - want[None, :]) <= 1e-4 * want[None, :]), \
            f"wave {wave}: sink {got[0, :4]} against closed form {want[:4]}"


def test_measurement_kernels_run_and_copy_is_exact():
    n = 64 << 20
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    s = g.current_stream_handle()
    g.gemm_peak_copy_launch(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, s)
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    g.gemm_peak_read_launch(ctypes.c_void_p(src.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), s)
    g.gemm_peak_empty_launch(s)
    blocks = 256
    fs = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    g.gemm_peak_mfma_launch(1000, blocks, ctypes.c_void_p(fs.data_ptr()),
                            ctypes.c_void_p(cyc.data_ptr()), s)
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    g.gemm_peak_clock_launch(2000, blocks, ctypes.c_void_p(clk.data_ptr()), s)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert torch.all(cyc > 0)
    _check_mfma_sink(fs.cpu().double().numpy().reshape(blocks, 256), 1000)
    c = clk.view(-1, 2).double().cpu()
    assert torch.all(c > 0)
    ghz = c[:, 0] / c[:, 1] * 0.1  # s_memrealtime ticks at 100 MHz
    assert 0.3 < float(ghz.median()) < 3.0


def test_mfma_data_peak_closed_form():
    """The operand-from-memory MFMA loop: A words all 1.0 and B words all 2.0 make every
    16 x 16 x 32 product add 64 to each accumulator, so after `iters` iterations each lane's sum
    of its 128 accumulators is 128 * 64 * iters exactly (a wrong operand word or a dropped
    instruction changes it)."""
    words = torch.empty(3072 * 8, dtype=torch.bfloat16, device="cuda")
    words[: 2048 * 8] = 1.0
    words[2048 * 8:] = 2.0
    blocks, iters = 256, 100
    sink = torch.zeros(blocks * 512, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    g.gemm_peak_mfma_data_launch(ctypes.c_void_p(words.data_ptr()), iters, blocks,
                                 ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(cyc.data_ptr()),
                                 g.current_stream_handle())
    torch.cuda.synchronize()
    assert torch.all(sink == 128 * 64 * iters)
    assert torch.all(cyc > 0)


# ---- concurrent streams and XCD placement ------------------------------------------------------

def test_split_layouts_on_two_streams_at_once():
    # Each stream gets its own workspace region, so split products enqueued on two streams with
    # no synchronisation between them cannot meet in the partial slots or the arrival counters.
    # Integer inputs: every result must equal the oracle's rounding of the exact sum bit for bit.
    cases = [("auto", 16, 4096, 11008),                     # skinny, K split 8 ways
             ("skinny", 3, 128 * 141 + 8, 64 * 37 + 8),     # Stream-K ranges across strips
             ("tiled", 1000, 1000, 1000)]                   # 128 x 128 tiles, K split
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for entry, M, N, K in cases:
        ins, wants, outs = [], [], []
        for si in range(2):
            A = matrix("int", M, K, seed=12000 + 10 * si + M)
            B = matrix("int", K, N, seed=13000 + 10 * si + N)
            ref, _ = oracle.gemm(A, B, with_abs=False)
            wants.append(oracle.bf16_rne(ref))
            ins.append((dev(A), dev(B)))
            outs.append([torch.empty(M * N, dtype=torch.bfloat16, device="cuda") for _ in range(3)])
        assert g.gemm_plan_describe(M, N, K, 256, entry == "skinny")["splits"] > 1
        torch.cuda.synchronize()
        for rep in range(12):
            for si in range(2):
                dA, dB = ins[si]
                C = outs[si][rep % 3]
                with torch.cuda.stream(streams[si]):
                    h = g.current_stream_handle()
                    g.gemm_fill_launch(ctypes.c_void_p(C.data_ptr()), C.numel() * 2, POISON, h)
                    ENTRIES[entry](M, N, K, ctypes.c_void_p(dA.data_ptr()), K, ctypes.c_void_p(dB.data_ptr()),
                                   N, ctypes.c_void_p(C.data_ptr()), N, h)
        torch.cuda.synchronize()
        for si in range(2):
            for C in outs[si]:
                got = host(C).reshape(M, N)
                bad = np.argwhere(got != wants[si])
                assert bad.size == 0, f"{entry} {M}x{N}x{K} stream {si}: {len(bad)} mismatches"


def test_workgroups_are_dealt_to_xcds_round_robin():
    # the tile and strip orders keep each XCD's share contiguous on the assumption that the
    # dispatcher deals consecutive workgroups to the XCDs in turn; measure it, and check that
    # the planner took the device's XCD count
    blocks = 4096
    out = torch.full((blocks,), 0xFFFF, dtype=torch.int32, device="cuda")
    g.gemm_peak_xcc_launch(blocks, ctypes.c_void_p(out.data_ptr()), g.current_stream_handle())
    torch.cuda.synchronize()
    x = out.cpu().numpy()
    A = matrix("int", 256, 256, seed=1)
    B = matrix("int", 256, 256, seed=2)
    run("tiled", A, B, 256, 256, 256)
    nxcd = g.gemm_last_plan()["nxcd"]
    assert nxcd == len(set(x.tolist())), f"planner nxcd {nxcd}, probe saw XCDs {sorted(set(x.tolist()))}"
    assert len(set(x[:nxcd].tolist())) == nxcd
    assert np.array_equal(x, np.tile(x[:nxcd], blocks // nxcd)), "workgroups not dealt round robin"


def test_tile_schedules_give_the_same_bits():
    # the two-group schedule and the all-waves-in-step schedule feed every accumulator the same
    # MFMAs in the same K order, so their outputs must agree bit for bit; the older schedule is
    # selected in a child process through the planner's debug override
    import os
    import subprocess
    import sys
    M, N, K = 777, 11000, 1000
    A = matrix("normal", M, K, seed=31000)
    B = matrix("normal", K, N, seed=32000, sigma=0.5)
    mine = run("tiled", A, B, M, N, K)
    assert g.gemm_last_plan()["bm"] == 256
    code = f"""
import ctypes, sys, numpy as np, torch
sys.path.insert(0, {os.path.dirname(os.path.dirname(os.path.abspath(__file__)))!r})
import gemv_layers_amd as g
from synth import matrix
torch.cuda.set_device(0); g.gemm_init(0)
A = matrix("normal", {M}, {K}, seed=31000); B = matrix("normal", {K}, {N}, seed=32000, sigma=0.5)
dA = torch.from_numpy(A.view(np.int16)).cuda(); dB = torch.from_numpy(B.view(np.int16)).cuda()
C = torch.empty({M} * {N}, dtype=torch.bfloat16, device="cuda")
g.gemm_bf16_tiled({M}, {N}, {K}, ctypes.c_void_p(dA.data_ptr()), {K}, ctypes.c_void_p(dB.data_ptr()), {N},
                  ctypes.c_void_p(C.data_ptr()), {N}, g.current_stream_handle())
torch.cuda.synchronize()
sys.stdout.buffer.write(C.cpu().view(torch.int16).numpy().tobytes())
"""
    env = dict(os.environ, GEMM_BF16_FORCE_TILE="0")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, timeout=240)
    assert r.returncode == 0, r.stderr.decode()[-2000:]
    other = np.frombuffer(r.stdout, dtype=np.uint16).reshape(M, N)
    assert np.array_equal(mine, other)


# ---- every element at full size ----------------------------------------------------------------
# Integer inputs make the exact result the expected bits (see above); for the workloads the host
# oracle finishes in seconds, every element is compared, not a row sample. 16384^3 (8.8 TFLOP in
# float64) is checked on every element against a closed form instead.

@pytest.mark.parametrize("name", ["sq512", "sq4096", "mlp_up", "mlp_down", "sq8192"] +
                         [n for n in WORKLOADS if n.startswith("dec_")])
def test_workload_integer_exact_every_element(name):
    w = WORKLOADS[name]
    A = matrix("int", w.M, w.K, seed=w.seed_a + 0x100)
    B = matrix("int", w.K, w.N, seed=w.seed_b + 0x100)
    C = run("auto", A, B, w.M, w.N, w.K)
    ref, _ = oracle.gemm(A, B, with_abs=False)
    want = oracle.bf16_rne(ref)
    bad = np.count_nonzero(C != want)
    assert bad == 0, f"{name}: {bad} of {C.size} elements differ"


def test_sq16384_rank_one_closed_form_every_element():
    # A[i][k] = a_i x_k and B[k][j] = y_k b_j with small integers: C[i][j] = a_i b_j (x . y), a
    # value that depends on the row and the column, so a misplaced row, column or k slice shows.
    # x . y = 2^10 and a_i b_j <= 15: every result and partial sum (|.| <= 15 K < 2^24) is exact
    # in float32 and in bf16.
    n = 16384
    i = np.arange(n)
    a = (1 + (i * 7) % 5).astype(np.float32)            # 1 .. 5
    b = (1 + (i * 11) % 3).astype(np.float32)           # 1 .. 3
    x = np.where(i % 3 == 0, 1.0, np.where(i % 3 == 1, -1.0, 0.0)).astype(np.float32)
    y = np.where(i % 3 == 0, 1.0, np.where(i % 3 == 1, 1.0, 0.0)).astype(np.float32)
    # make x . y exactly 2^10: zero every contribution past the first 1024 + 1024 matched pairs
    ones = np.flatnonzero(i % 3 == 0)[:1024 + 1024]
    negs = np.flatnonzero(i % 3 == 1)[:1024]
    x[:] = 0.0
    y[:] = 0.0
    x[ones] = 1.0
    y[ones] = 1.0
    x[negs] = -1.0
    y[negs] = 1.0
    s = float(x.astype(np.float64) @ y.astype(np.float64))
    assert s == 1024.0
    from synth import f32_to_bf16_bits
    A = f32_to_bf16_bits(np.outer(a, x).astype(np.float32))
    B = f32_to_bf16_bits(np.outer(y, b).astype(np.float32))
    C = run("auto", A, B, n, n, n)
    want = f32_to_bf16_bits((np.outer(a, b) * s).astype(np.float32))
    bad = np.count_nonzero(C != want)
    assert bad == 0, f"{bad} of {C.size} elements differ from a_i b_j (x . y)"


# ---- seeded random shapes across every dispatch regime ---------------------------------------

def _random_cases(n, seed=20251202):
    """(entry, M, N, K, lda, ldb, ldc) drawn from a fixed seed: M in the skinny, small-tile and
    large-tile ranges; N and K multiples of 8 with padded leading dimensions (the fast kernels)
    or arbitrary (the general kernel); at most 1.5e9 multiply-adds so the oracle takes a moment."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        regime = rng.choice(3, p=[0.4, 0.3, 0.3])
        M = int(rng.integers(1, 65) if regime == 0 else rng.integers(65, 400) if regime == 1
                else rng.integers(400, 1300))
        fast = rng.random() < 0.75
        N, K = int(rng.integers(1, 3000)), int(rng.integers(1, 2100))
        if fast:
            N, K = max(8, N - N % 8), max(8, K - K % 8)
            pads = [0, 0, 8, 64]
        else:
            pads = [0, 1, 3, 13]
        if M * N * K > 1.5e9:
            continue
        lda, ldb, ldc = (d + int(rng.choice(pads)) for d in (K, N, N))
        entry = rng.choice(["auto", "auto", "tiled"] + (["skinny"] if M <= 64 else []))
        cases.append((str(entry), M, N, K, lda, ldb, ldc))
    return cases


RANDOM_CASES = _random_cases(48)


def test_random_cases_reach_every_kernel_family():
    """The drawn cases cover the skinny, large-tile and general kernels (the dispatch rule,
    checked on the host)."""
    kinds = set()
    for entry, M, N, K, lda, ldb, ldc in RANDOM_CASES:
        fast = all(x % 8 == 0 for x in (N, K, lda, ldb, ldc))
        kinds.add("generic" if not fast else "skinny" if (entry == "skinny" or (entry == "auto" and M <= 64)) else "tile")
    assert kinds == {"generic", "skinny", "tile"}


@pytest.mark.parametrize("case", range(len(RANDOM_CASES)))
def test_random_shapes_integer_exact(case):
    """Integer-valued operands with NaN in every padding column: the product must equal the
    oracle's exact result rounded to bf16, bit for bit, whatever kernel the shape lands on."""
    entry, M, N, K, lda, ldb, ldc = RANDOM_CASES[case]
    A = matrix("int", M, K, seed=1000 + case, ld=lda)
    B = matrix("int", K, N, seed=2000 + case, ld=ldb)
    C = run(entry, A, B, M, N, K, ldc=ldc)
    kernel = g.gemm_last_plan()["kernel"]
    check_exact(C, A, B, M, N, K, f"{entry} {M}x{N}x{K} ld {lda},{ldb},{ldc} ({kernel})")


def _large_random_cases(n, seed=0x50A4):
    """Seeded shapes at prefill and decode scale through gemm_bf16: decode (M <= 64, N up to
    16000, K up to 12000), mid-size grids of small tiles with or without a K split, large grids,
    and products with a sparse last wave of 256 x 256 tiles (a whole number of waves plus up to
    half of one, so the planner cuts the product in two); 85% on the fast kernels (multiples of
    8, padded leading dimensions), the rest on the general kernel."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        kind = str(rng.choice(["decode", "mid", "big", "cut"], p=[0.3, 0.25, 0.2, 0.25]))
        if kind == "decode":
            M, N, K = int(rng.integers(1, 65)), int(rng.integers(8, 16000)), int(rng.integers(8, 12000))
        elif kind == "mid":
            M, N, K = int(rng.integers(65, 2200)), int(rng.integers(64, 6000)), int(rng.integers(64, 6000))
        elif kind == "big":
            M, N, K = int(rng.integers(2000, 7000)), int(rng.integers(2000, 9000)), int(rng.integers(64, 3000))
        else:
            w, tm = int(rng.integers(1, 4)), int(rng.integers(8, 33))
            tn = -(-256 * w // tm) + int(rng.integers(1, max(2, 128 // tm + 1)))
            M, N = 256 * tm - int(rng.integers(0, 200)), 256 * tn - int(rng.integers(0, 200))
            K = int(rng.integers(64, 2500))
        if rng.random() < 0.85:
            N, K = max(8, N - N % 8), max(8, K - K % 8)
            pads = [0, 0, 8, 64]
        else:
            pads = [0, 1, 3, 13]
        lda, ldb, ldc = (d + int(rng.choice(pads)) for d in (K, N, N))
        cases.append((kind, M, N, K, lda, ldb, ldc))
    return cases


LARGE_RANDOM_CASES = _large_random_cases(64)


def test_large_random_cases_reach_every_regime():
    """The drawn cases include products the planner cuts in two, split-K and unsplit tiles,
    skinny layouts in both XCD orders and the general kernel (checked on the host)."""
    seen = set()
    for kind, M, N, K, lda, ldb, ldc in LARGE_RANDOM_CASES:
        if not all(x % 8 == 0 for x in (N, K, lda, ldb, ldc)):
            seen.add("generic")
            continue
        p = g.gemm_plan_describe(M, N, K)
        if "cut" in p:
            seen.add("cut " + p["cut"]["axis"])
        if p["kernel"] == "tile":
            seen.add("split-k" if p["schedule"] == "split-k" else "tile")
        if p["kernel"] == "skinny":
            seen.add("skinny hardware order" if p["nxcd"] == 1 else "skinny remapped")
    assert seen >= {"generic", "cut n", "cut m", "split-k", "tile", "skinny hardware order", "skinny remapped"}, seen


@pytest.mark.parametrize("case", range(len(LARGE_RANDOM_CASES)))
def test_large_random_shapes_integer_exact(case):
    """Integer operands in {-4 .. 4} with NaN padding: on sampled rows (both sides of a row cut
    among them) every column equals the oracle's exact sum rounded to bf16, and C's padding
    columns keep their poison."""
    kind, M, N, K, lda, ldb, ldc = LARGE_RANDOM_CASES[case]
    A = matrix("int", M, K, seed=30000 + case, ld=lda)
    B = matrix("int", K, N, seed=40000 + case, ld=ldb)
    Cd = torch.empty(-(-max(M * ldc, 8) // 8) * 8, dtype=torch.bfloat16, device="cuda")
    g.gemm_fill_launch(ctypes.c_void_p(Cd.data_ptr()), Cd.numel() * 2, POISON)
    C = run("auto", A, B, M, N, K, ldc=ldc, C=Cd)
    plan = g.gemm_last_plan()
    rows = set(_sample_rows(M, 12).tolist())
    if "cut" in plan and plan["cut"]["axis"] == "m":
        at = plan["cut"]["at"]
        rows |= {at - 1, at, min(M - 1, at + 1)}
    rows = np.array(sorted(rows))
    ref, _ = oracle.gemm(np.ascontiguousarray(A[rows, :K]), np.ascontiguousarray(B[:, :N]), M=len(rows), N=N, K=K,
                         with_abs=False)
    bad = np.argwhere(C[rows] != oracle.bf16_rne(ref))
    what = f"{kind} {M}x{N}x{K} ld {lda},{ldb},{ldc} {plan['kernel']} cut={plan.get('cut', {}).get('at')}"
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[0].tolist()}"
    if ldc > N:
        full = host(Cd)[: M * ldc].reshape(M, ldc)
        assert np.all(full[rows, N:] == 0x7FC0), f"{what}: padding written"
