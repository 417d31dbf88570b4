"""The host planner: page-printed wave figures, and the plans at the workload shapes on 256 CUs."""

import math
import os

import pytest

import gemv_layers_amd as g
from synth import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixtures():
    out = []
    for line in open(os.path.join(GOLDEN, "planner_fixtures.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, s, w, e, tol = line.split()[:5]
            out.append((int(c), int(s), int(w), float(e), float(tol)))
    return out


@pytest.mark.parametrize("ctas,slots,waves,eff,tol", _fixtures())
def test_wave_efficiency_matches_printed_figures(ctas, slots, waves, eff, tol):
    e, w = g.gemm_wave_efficiency(ctas, slots)
    assert w == waves
    assert abs(e - eff) <= tol


def test_two_factor_decomposition_of_printed_example():
    # "Kernel development on sm_120", section 4: 82.4% of the ceiling = 86.1% waves x 95.7% pipe
    e, _ = g.gemm_wave_efficiency(1024, 170)
    assert abs(e - 0.861) < 0.001
    assert abs(e * 0.957 - 0.824) < 0.001


def _cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("name", ["sq4096", "sq8192", "sq16384", "mlp_up", "mlp_down"])
def test_large_shapes_use_256_tiles(name):
    w = WORKLOADS[name]
    p = g.gemm_plan_describe(w.M, w.N, w.K, 256)
    assert p["kernel"] == "tile" and (p["bm"], p["bn"]) == (256, 256)
    tiles = _cdiv(w.M, 256) * _cdiv(w.N, 256)
    assert p["tiles"] == tiles and p["grid"] == tiles and p["schedule"] == "data-parallel"
    e, waves = g.gemm_wave_efficiency(tiles, 256)
    assert p["waves"] == waves and abs(p["wave_eff"] - e) < 1e-6


def test_mlp_up_wave_quantization():
    # 688 tiles on 256 slots fill 688 / 768 = 89.6% of three waves (the closed form)
    e, waves = g.gemm_wave_efficiency(688, 256)
    assert waves == 3 and abs(e - 688 / 768) < 1e-12
    p = g.gemm_plan_describe(4096, 11008, 4096, 256)
    assert p["tiles"] == 688 and p["waves"] == 3
    assert abs(p["wave_eff"] - 688 / 768) < 1e-6


def test_small_square_splits_k():
    p = g.gemm_plan_describe(512, 512, 512, 256)
    assert p["kernel"] == "tile" and (p["bm"], p["bn"]) == (128, 128)
    assert p["schedule"] == "split-k" and p["splits"] > 1
    kt = 512 // p["bk"]
    assert p["splits"] * p["kt_per_split"] >= kt
    assert (p["splits"] - 1) * p["kt_per_split"] < kt  # no empty piece


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (1000, 1000, 1000), (257, 264, 4104),
                                   (300, 520, 328), (128, 128, 96), (200, 2000, 20000),
                                   (2048, 2048, 2048), (1024, 1024, 8192), (128, 128, 65536),
                                   (2048, 1024, 4096), (1536, 1536, 4096), (1664, 1664, 4096),
                                   (1536, 1536, 96), (2048, 1920, 4096), (1536, 1536, 1024),
                                   (1792, 1792, 2048), (1536, 1536, 3072), (1024, 4096, 4096),
                                   (1024, 4096, 11008), (2048, 2048, 8192), (1024, 4096, 2048)])
def test_split_count_follows_the_measured_rule(M, N, K):
    # each piece costs the last arriver one memory round trip, about three k-steps of a lone
    # workgroup, so with one workgroup per CU K is cut into about sqrt(kt / 3) pieces; when only
    # one piece per tile would fit that way, up to two per CU, about sqrt(kt / 8) pieces and only
    # from 96 k-steps; grids with more tiles than CUs stay whole; no piece is empty
    p = g.gemm_plan_describe(M, N, K, 256)
    kt = -(-K // p["bk"])

    def root(c):
        r = 1
        while c * (r + 1) ** 2 <= kt:
            r += 1
        return r

    want = 1
    if p["bm"] == 128 and p["tiles"] <= 256:
        per_cu = 256 // p["tiles"]
        if per_cu >= 2:
            want = min(root(3), per_cu)
        elif kt >= 96:
            want = min(root(8), 512 // p["tiles"])
    if want > 1:
        per = -(-kt // want)
        assert p["schedule"] == "split-k" and p["kt_per_split"] == per and p["splits"] == -(-kt // per)
        assert (p["splits"] - 1) * p["kt_per_split"] < kt <= p["splits"] * p["kt_per_split"]
        assert p["grid"] == p["tiles"] * p["splits"] <= 512
    else:
        assert p["splits"] == 1 and p["schedule"] == "data-parallel"


@pytest.mark.parametrize("name", [n for n in WORKLOADS if n.startswith("dec_")])
def test_decode_shapes_stream_weights(name):
    w = WORKLOADS[name]
    p = g.gemm_plan_describe(w.M, w.N, w.K, 256)
    assert p["kernel"] == "skinny"
    assert p["mtiles"] == _cdiv(w.M, 16)
    assert p["strip"] in (128, 256) and p["strips"] == _cdiv(w.N, p["strip"])
    assert p["ks"] == _cdiv(w.K, 64)
    # at most one workgroup per CU: either every range is one piece of one strip on at least two
    # thirds of the CUs, or Stream-K ranges over all of them
    assert p["grid"] <= 256 and p["waves"] == 1
    assert (p["grid"] % p["strips"] == 0 and 3 * p["grid"] >= 2 * 256) or p["grid"] == 256


# (M, N, K) -> (strip width, grid): the largest aligned grid (strips x the most pieces per strip
# that fit 256) that fills two thirds of the CUs (one or two 16-row tiles of M; 256-column strips
# only there) or fifteen sixteenths (more rows), ties to fewer pieces per strip; else Stream-K
# ranges over min(units, 256) workgroups with 128-column strips
LAYOUTS = [((1, 4096, 11008), (128, 256)),      # 32 x 8 ties 16 x 16 at 256: fewer pieces
           ((1, 11008, 4096), (256, 215)),      # 43 x 5 beats 86 x 2 = 172
           ((64, 11008, 4096), (128, 256)),     # 86 x 2 is too few for four tiles of M: Stream-K
           ((1, 128 * 65, 4096), (256, 231)),   # 33 x 7 beats 65 x 3 = 195
           ((1, 256 * 140, 4096), (128, 256)),  # 280 strips of 128, 140 of 256: Stream-K
           ((3, 256, 128), (128, 4)),           # 2 strips x 2 stages: one unit per workgroup
           ((1, 4096, 64), (128, 32))]          # one stage per strip


@pytest.mark.parametrize("shape,want", LAYOUTS)
def test_skinny_layout_choice(shape, want):
    p = g.gemm_plan_describe(*shape, 256)
    assert (p["strip"], p["grid"]) == want


@pytest.mark.parametrize("M,N,K,glu,nxcd", [
    (1, 4096, 11008, False, 1), (16, 4096, 11008, False, 1), (32, 4096, 11008, False, 1),  # 8 pieces
    (1, 8192, 4096, False, 1), (1, 14336, 4096, False, 1),  # 4 and 2 pieces
    (64, 4096, 11008, False, 8),  # four 16-row tiles
    (1, 11008, 4096, False, 8),  # 5 pieces
    (1, 2048, 8192, False, 8), (1, 1024, 4096, False, 8),  # 16 and 32 pieces
    (64, 11008, 4096, False, 8),  # unit ranges across strips
    (1, 11008, 4096, True, 8), (16, 11008, 4096, True, 8)])  # SwiGLU
def test_skinny_xcd_order(M, N, K, glu, nxcd):
    # aligned grids whose pieces per strip divide the XCD count keep the hardware's dealing
    # (nxcd 1: no remap) at one or two 16-row tiles of the plain product
    p = g.gemm_plan_describe(M, N, K, 256, swiglu=glu)
    assert p["kernel"] == "skinny" and p["nxcd"] == nxcd, p
    if nxcd == 1:
        assert p["grid"] == p["strips"] * p["splits"] and 8 % p["splits"] == 0 and p["splits"] >= 2


@pytest.mark.parametrize("cus", [80, 228, 256, 304])
@pytest.mark.parametrize("M,N,K,glu", [(1, 4096, 11008, False), (16, 8192, 4096, False), (32, 14336, 4096, False),
                                       (64, 4096, 11008, False), (1, 11008, 4096, True), (2, 2048, 8192, False)])
def test_skinny_xcd_order_follows_the_cu_count(cus, M, N, K, glu):
    p = g.gemm_plan_describe(M, N, K, cus, swiglu=glu)
    dev_nxcd = 8 if cus % 8 == 0 else 1  # the XCD count the library assumes without a device
    hw_order = (not glu and p["mtiles"] <= 2 and p["grid"] == p["strips"] * p["splits"]
                and p["splits"] >= 2 and dev_nxcd % p["splits"] == 0)
    assert p["nxcd"] == (1 if hw_order else dev_nxcd), p


def test_skinny_small_problem_has_one_unit_per_workgroup():
    p = g.gemm_plan_describe(3, 256, 128, 256)
    assert p["kernel"] == "skinny" and p["grid"] == 2 * 2


def test_dispatch_threshold_and_degenerate():
    assert g.gemm_plan_describe(64, 4096, 4096, 256)["kernel"] == "skinny"
    assert g.gemm_plan_describe(65, 4096, 4096, 256)["kernel"] == "tile"
    assert g.gemm_plan_describe(65, 4096, 4096, 256, skinny=False)["kernel"] == "tile"
    assert g.gemm_plan_describe(0, 8, 8, 256)["kernel"] == "none"
    assert g.gemm_plan_describe(8, 8, 0, 256)["kernel"] == "zero"
    with pytest.raises(g.GemmError):
        g.gemm_plan_describe(65, 8, 8, 256, skinny=True)


# ---- the SwiGLU form: the fast kernels are planned over the 2N weight columns --------------

@pytest.mark.parametrize("M,N,K", [(4096, 11008, 4096), (1000, 1000, 1000), (300, 520, 328)])
def test_swiglu_tile_plan_covers_both_halves(M, N, K):
    p = g.gemm_plan_describe(M, N, K, swiglu=True)
    q = g.gemm_plan_describe(M, 2 * N, K)
    assert p["kernel"] == "tile" and p["op"] == "swiglu" and p["N"] == N
    if "cut" in q and q["cut"]["axis"] == "n":
        # the plain product may cut a sparse last wave off as a column strip; the SwiGLU form
        # cannot (its up half sits N weight columns after the gate half), so it keeps the tiles
        assert "cut" not in p or p["cut"]["axis"] == "m"
        assert p["bm"] == q["bm"] and p["tiles_m"] == q["tiles_m"]
    else:
        for key in ("bm", "bn", "tiles_m", "tiles_n", "grid", "splits", "schedule"):
            assert p[key] == q[key], key
    # a BN-wide tile makes BN / 2 outputs
    if "cut" not in p:
        assert p["tiles_n"] == _cdiv(N, p["bn"] // 2)


@pytest.mark.parametrize("M", [1, 2, 16, 17, 64])
def test_swiglu_skinny_plan_covers_both_halves(M):
    N, K = 11008, 4096
    p = g.gemm_plan_describe(M, N, K, swiglu=True)
    q = g.gemm_plan_describe(M, 2 * N, K)
    assert p["kernel"] == "skinny" and p["op"] == "swiglu"
    assert p["ks"] == q["ks"] and p["mtiles"] == q["mtiles"]
    assert p["strips"] == _cdiv(N, p["strip"] // 2)
    assert p["grid"] == q["grid"]  # the same aligned grid, or Stream-K over every CU
    # a grid tie goes to the wider strip: gate and up segments of a row stay 256 bytes
    if M <= 32:
        assert (p["strip"], p["grid"]) == (256, 172) and (q["strip"], q["grid"]) == (128, 172)
    else:
        assert p["strip"] == q["strip"] == 128 and p["grid"] == 256


# ---- the block-scaled decode product --------------------------------------------------------

def _mx_groups(tiles, K, tn, cus=256):
    """Groups of tn column tiles and K pieces as the decode plans them: K whole when the groups
    cover 60% of the CUs, else just enough pieces to cover them all (at least 4 k-steps a piece)."""
    strips = _cdiv(tiles, tn)
    want = 1 if 5 * strips >= 3 * cus else _cdiv(cus, strips)
    return strips, min(want, max(1, (K // 128) // 4))


@pytest.mark.parametrize("cus", [80, 228, 256, 304])
@pytest.mark.parametrize("M,N,K", [(1, 11008, 4096), (64, 4096, 11008), (1, 12288, 4096), (16, 1040, 1152),
                                   (1, 65520, 65536)])
def test_mx_group_width_follows_the_cu_count(cus, M, N, K):
    # the width whose grid leaves the fewest CUs idle in its last round of CUs, four on a tie
    p = g.gemm_plan_describe(M, N, K, cus, mx=True)
    tiles = N // 16

    def fill(t):
        strips, s = _mx_groups(tiles, K, t, cus)
        grid = strips * s
        return grid / (_cdiv(grid, cus) * cus)

    tn = 3 if fill(3) > fill(4) + 1e-9 else 4
    assert p["strip"] == 16 * tn, p
    assert (p["strips"], p["splits"]) == _mx_groups(tiles, K, tn, cus)


@pytest.mark.parametrize("M,N,K", [(1, 11008, 4096), (16, 11008, 4096), (64, 11008, 4096),
                                   (1, 4096, 11008), (64, 4096, 11008), (3, 80, 640), (2, 128, 128),
                                   (1, 12288, 4096), (1, 4096, 4096)])
def test_mx_plan(M, N, K):
    p = g.gemm_plan_describe(M, N, K, mx=True)
    assert p["kernel"] == "mx" and p["op"] == "mx"
    tiles = N // 16
    tn = p["strip"] // 16
    assert tn in (3, 4)
    assert p["tiles_n"] == tiles and p["ks"] == K // 128
    assert (p["strips"], p["splits"]) == _mx_groups(tiles, K, tn)
    assert p["grid"] == p["strips"] * p["splits"]

    # the group width whose grid leaves the fewest CUs idle in its last round; four on a tie
    def fill(t):
        strips, s = _mx_groups(tiles, K, t)
        grid = strips * s
        return grid / (_cdiv(grid, 256) * 256)

    assert tn == (3 if fill(3) > fill(4) else 4)
    assert p["nxcd"] == 1  # groups dealt to the XCDs in the hardware's order
    if (N, K) == (11008, 4096):
        assert (tn, p["grid"]) == (3, 230)  # 172 groups of four would leave 84 CUs idle
    if (N, K) == (4096, 11008):
        assert (tn, p["splits"], p["grid"]) == (4, 4, 256)


def test_mx_plan_rejects_other_shapes():
    for (M, N, K) in ((65, 4096, 4096), (1, 4100, 4096), (1, 4096, 4000)):
        with pytest.raises(g.GemmError):
            g.gemm_plan_describe(M, N, K, mx=True)


@pytest.mark.parametrize("M,N,K,bm", [(1024, 11008, 4096, 256), (512, 11008, 4096, 128), (3072, 4096, 4096, 256),
                                      (2048, 2048, 2048, 128), (1024, 4096, 11008, 128),
                                      (1024, 4352, 4096, 128), (1024, 4096, 4096, 128),
                                      (1000, 4104, 512, 128), (1000, 4096, 512, 128),
                                      (2048, 4096, 4096, 128), (2048, 4224, 4096, 256),
                                      (4096, 4096, 4096, 256)])
def test_small_tiles_up_to_two_per_cu(M, N, K, bm):
    # below one wave of 256 x 256 tiles, 128 x 128 tiles as long as at most two share a CU (two
    # fit in a CU's LDS and registers and run together); otherwise 256 x 256 tiles
    p = g.gemm_plan_describe(M, N, K, 256)
    assert p["kernel"] == "tile" and p["bm"] == bm, p
    big = -(-M // 256) * -(-N // 256)
    small = -(-M // 128) * -(-N // 128)
    assert (big < 256 and small <= 512) == (bm == 128)
    assert p["slots"] == (512 if bm == 128 else 256)
    if bm == 256 or small > 256:
        assert p["splits"] == 1 and p["schedule"] == "data-parallel"


@pytest.mark.parametrize("cus", [80, 228, 256, 304])
@pytest.mark.parametrize("M,N,K", [(1024, 4352, 4096), (2048, 2048, 4096), (1536, 1536, 4096),
                                   (1024, 11008, 4096), (4096, 4096, 4096), (512, 512, 8192)])
def test_tile_rules_follow_the_cu_count(cus, M, N, K):
    # the tile choice and the K split scale with the queried CU count: 256 x 256 tiles from one
    # full wave of them, else 128 x 128 tiles while at most two share a CU; a K split only while
    # the small tiles are no more than the CUs, and then at most two pieces per CU
    p = g.gemm_plan_describe(M, N, K, cus)
    big = -(-M // 256) * -(-N // 256)
    small = -(-M // 128) * -(-N // 128)
    want_bm = 256 if (big >= cus or small > 2 * cus) else 128
    assert p["bm"] == want_bm, p
    assert p["slots"] == (2 * cus if want_bm == 128 else cus)
    if p["schedule"] == "split-k":
        assert want_bm == 128 and p["tiles"] <= cus
        assert p["grid"] <= 2 * cus
        if cus // p["tiles"] >= 2:
            assert p["grid"] <= cus


# ---- a sparse last wave of 256 x 256 tiles cut off as a strip ------------------------------

@pytest.mark.parametrize("M,N,K,glu,want", [
    (4096, 4352, 4096, False, ("n", 4096)), (4352, 4352, 4096, False, ("n", 3840)),
    (4352, 4096, 1024, False, ("m", 4096)), (8192, 8448, 4096, False, ("n", 8192)),
    (4608, 4608, 4608, False, ("n", 3584)), (4096, 11008, 4096, False, None),
    (5120, 5120, 5120, False, None), (4096, 4096, 4096, False, None), (8192, 8192, 8192, False, None),
    (4608, 2304, 4096, True, ("m", 3584)), (4096, 11008, 4096, True, None),
    # the seeded ragged cases of the GPU parity tests
    (5376, 3312, 400, False, ("n", 3072)), (4792, 3800, 992, False, ("m", 4352)),
    (6408, 4936, 584, False, ("m", 6400)), (4152, 8616, 320, False, ("n", 7680)),
    (2792, 7592, 416, False, ("n", 5888)), (5088, 4120, 304, False, ("m", 3840))])
def test_sparse_last_wave_cut_at_256_cus(M, N, K, glu, want):
    p = g.gemm_plan_describe(M, N, K, 256, swiglu=glu)
    if want is None:
        assert "cut" not in p, p
    else:
        assert (p["cut"]["axis"], p["cut"]["at"]) == want, p


@pytest.mark.parametrize("cus", [80, 228, 256, 304])
@pytest.mark.parametrize("M,N,K,glu", [
    (4096, 4352, 4096, False), (4352, 4352, 4096, False), (4352, 4096, 1024, False),
    (4000, 4400, 1000, False), (8192, 8448, 4096, False), (4608, 4608, 4608, False),
    (6144, 6144, 6144, False), (4096, 11008, 4096, False), (2560, 3072, 2048, False),
    (3000, 9000, 512, False), (4608, 2304, 4096, True), (4096, 11008, 4096, True),
    (3000, 2000, 1000, True)])
def test_sparse_last_wave_cut_rule(cus, M, N, K, glu):
    # with the 256 x 256 tiles of a data-parallel plan leaving a last wave at most half full, the
    # largest rectangle of whole tile rows or columns that fits in the full waves is kept (a
    # column cut only outside the SwiGLU form) and the strip left over is planned on its own; the
    # cut is taken only when that strip comes out as 128 x 128 tiles
    W = 2 * N if glu else N
    bm_, bn_ = -(-M // 256), -(-W // 256)
    full, last = divmod(bm_ * bn_, cus)
    tn = (full * cus) // bm_ if not glu else 0
    tm = (full * cus) // bn_
    cands = []
    if not glu and 1 <= tn < bn_:
        cands.append((tn * bm_, "n", tn * 256))
    if 1 <= tm < bm_ and (not cands or tm * bn_ > cands[0][0]):
        cands = [(tm * bn_, "m", tm * 256)]
    p = g.gemm_plan_describe(M, N, K, cus, swiglu=glu)
    uncut = p.get("cut") is None
    sparse = p["bm"] == 256 and full >= 1 and 0 < last and 2 * last <= cus and cands
    if not uncut:
        kept, axis, at = cands[-1]
        c = p["cut"]
        assert sparse and (c["axis"], c["at"]) == (axis, at), p
        assert p["bm"] == 256 and p["tiles"] == kept <= full * cus
        assert c["rest"]["bm"] == 128 and c["rest"]["kernel"] == "tile"
        if axis == "n":
            assert c["rest"]["M"] == M and c["rest"]["N"] == N - at
        else:
            assert c["rest"]["M"] == M - at and c["rest"]["N"] == N
        assert p["ws_floats"] >= c["rest"]["ws_floats"]
    elif sparse:
        # the strip would not have come out as small tiles
        kept, axis, at = cands[-1]
        rest = (g.gemm_plan_describe(M, N - at, K, cus, swiglu=glu) if axis == "n"
                else g.gemm_plan_describe(M - at, N, K, cus, swiglu=glu))
        assert rest["bm"] != 128 or rest["kernel"] != "tile", (p, rest)
