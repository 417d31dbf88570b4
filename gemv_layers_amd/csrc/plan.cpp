// Host planner. The choices follow the pages' closed forms:
// * wave efficiency (tiles / slots) / ceil(tiles / slots) decides whether a tile shape fills the
//   card ("Kernel development on sm_120", section 4, budget 4; spark-kernels "170 is 2 times 5
//   times 17": a grid that leaves a partial last wave wastes the idle slots for a whole wave);
// * the tile is picked per call: the big tile when its grid fills at least one wave, otherwise
//   a smaller tile, otherwise K is split across the idle slots (spark-kernels, "1024 cubed and the
//   decode shapes" and "170 is 2 times 5 times 17");
// * M <= 64 streams the weights with the skinny kernel, one workgroup per column strip, K split
//   just enough to give the card enough workgroups (spark-kernels, "the decode kernel").
// No autotuning at run time: fixed constants, one closed form per decision ("Kernel development
// on sm_120", section 6, "Autotune").

#include "plan.h"

#include <stdio.h>

#include <algorithm>

#include "kernels.h"

namespace glk {

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

void wave_efficiency(int64_t ctas, int64_t slots, double* eff, int64_t* waves) {
    if (ctas <= 0 || slots <= 0) {
        if (eff) *eff = 0.0;
        if (waves) *waves = 0;
        return;
    }
    const int64_t w = cdiv(ctas, slots);
    if (waves) *waves = w;
    if (eff) *eff = ((double)ctas / (double)slots) / (double)w;
}

bool fast_path_ok(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                  int64_t ldb, const void* C, int64_t ldc) {
    const int64_t kMaxLd = int64_t(1) << 20, kMaxDim = int64_t(1) << 26;
    auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return false;
    if ((N & 7) || (K & 7) || (lda & 7) || (ldb & 7) || (ldc & 7)) return false;
    if (lda > kMaxLd || ldb > kMaxLd || ldc > kMaxLd) return false;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return false;
    return true;
}

static void finish_waves(Plan& p) { wave_efficiency(p.grid, p.slots, &p.wave_eff, &p.waves); }

// The split of the strip-major list of (strip, stage) units into `grid` balanced ranges puts
// every range boundary on a strip boundary whenever grid = strips * S: each workgroup then holds
// one piece of one strip, and a strip has exactly S pieces (S = 1: no partials at all), so no
// piece ends mid-range and the fixup is as short as it gets. For each strip width the aligned
// grid takes the most pieces per strip that fit one wave of workgroups; it counts when it
// occupies enough of the CUs: two thirds for up to two 16-row tiles of M, all but a sixteenth
// above that (wider M does more work per byte and wants every CU). The planner takes the largest
// counting grid, and on a tie the one with fewer pieces per strip (less float32 partial traffic).
// 256-column strips are considered only up to two tiles of M: their stages are twice as big, and
// with wider A the ring would be too shallow. Without an aligned grid, Stream-K ranges over one
// workgroup per CU cut 128-column strips wherever they fall.
// The SwiGLU form reads each strip row as two segments, gate and up, of half the strip each:
// there a tie goes to the wider strip instead, which keeps the segments 256 bytes long
// (measured on the 4096 x 22016 gate/up weight at M = 1 and 16: 256-column strips in 2 pieces
// 37.0-37.2 us against 40.2-41.9 us for whole 128-column strips).
static void skinny_layout(int64_t N, int ks, int mtiles, int cus, bool glu, int* strip, int64_t* grid) {
    int best_sw = 0;
    int64_t best_grid = 0, best_s = 0;
    for (int sw : {128, 256}) {
        if (sw == 256 && mtiles > 2) continue;
        const int64_t strips = cdiv(N, sw);
        const int64_t s = std::min<int64_t>(cus / strips, ks);
        if (s < 1) continue;
        const int64_t g = strips * s;
        const bool enough = (mtiles <= 2) ? 3 * g >= 2 * (int64_t)cus : 16 * g >= 15 * (int64_t)cus;
        if (!enough) continue;
        if (g > best_grid || (g == best_grid && (glu ? sw > best_sw : s < best_s))) {
            best_sw = sw;
            best_grid = g;
            best_s = s;
        }
    }
    if (best_sw) {
        *strip = best_sw;
        *grid = best_grid;
    } else {
        *strip = kSkinnyStripMin;
        *grid = std::min<int64_t>(cdiv(N, kSkinnyStripMin) * ks, cus);
    }
}

static Plan plan_skinny(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev, bool glu) {
    Plan p;
    p.kernel = kKernSkinny;
    p.nxcd = dev.nxcd;
    p.mtiles = (int)cdiv(M, 16);
    p.threads = 256;
    p.ks = (int)cdiv(K, kSkinnyStage);
    // one workgroup per CU at most: every launch asks for more than half of a CU's LDS
    p.slots = dev.cus;
    skinny_layout(N, p.ks, p.mtiles, dev.cus, glu, &p.strip, &p.grid);
    p.strips = (int)cdiv(N, p.strip);
    const int64_t units = (int64_t)p.strips * p.ks;
    const int64_t slot_floats = skinny_slot_floats(p.mtiles, p.strip);
    // two partial slots per workgroup; fall back to one unit range per strip (no partials) if
    // the workspace or the counters cannot hold them
    if (2 * p.grid * slot_floats > dev.ws_floats || p.strips > dev.ws_counters) p.grid = p.strips;
    p.ws_floats = 2 * p.grid * slot_floats;
    p.counters = p.strips;
    p.splits = (int)cdiv(p.grid, p.strips);  // pieces per strip, about
    // With 2, 4 or 8 pieces per strip (a divisor of the XCD count) the hardware's round-robin
    // dealing alone gives each XCD the same pieces of many strips: whole rows of one K slice of
    // the weight, where the remap gives it all of K for a few strips, one narrow column block of
    // each row. Measured with one or two 16-row tiles, us: 4096 x 11008 weight 20.8 -> 20.4,
    // 4096 x 4096 12.5 -> 11.0, 8192 x 4096 18.2 -> 16.2, 14336 x 4096 25.4 -> 24.7. Not taken at
    // four tiles (neutral to 2% slower), for the SwiGLU form (1% slower), nor with 16 or 32
    // pieces (1-4% slower).
    if (!glu && p.mtiles <= 2 && p.grid == (int64_t)p.strips * p.splits && p.splits >= 2 &&
        dev.nxcd % p.splits == 0)
        p.nxcd = 1;
    finish_waves(p);
    p.reason = "M <= 64: weights streamed once, " + std::to_string(p.grid) +
               ((p.grid % p.strips == 0) ? " workgroups, each one piece of one strip, over "
                                         : " workgroups over ") +
               std::to_string(units) + " stages of " + std::to_string(p.strip) + "-column strips";
    return p;
}

static void set_tile(Plan& p, int cfg, int64_t M, int64_t N) {
    const TileShape t = tile_shape(cfg);
    p.tile_cfg = cfg;
    p.bm = t.bm;
    p.bn = t.bn;
    p.bk = t.bk;
    p.threads = t.threads;
    p.tiles_m = cdiv(M, t.bm);
    p.tiles_n = cdiv(N, t.bn);
    p.tiles = p.tiles_m * p.tiles_n;
}

static Plan plan_tile(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev) {
    Plan p;
    p.kernel = kKernTile;
    p.nxcd = dev.nxcd;
    // the 256 x 256 tile runs the kernel whose two wave groups alternate MFMA and memory phases:
    // 1.6-2.7% faster than all eight waves in step on every large workload, same bits as far as
    // the tests see (measured interleaved, settled clocks: sq8192 807 against 828 us, mlp_up 300
    // against 309 us, mlp_down 271 against 278 us)
    set_tile(p, kTile256x256pp, M, N);
    // Below one wave of 256x256 tiles, 128x128 tiles: one alone on a CU takes about 60% as long
    // as a 256x256 one (46 against 77 us at K = 4096), and two share a CU (72 KB of LDS and at
    // most 256 registers per lane each), taking about 1.35 times as long together as one alone.
    // So up to two small tiles per CU beat one partial wave of big ones; beyond that the big
    // tiles' lower bytes per flop win (measured, settled clocks: 2048^3 as 256 small tiles 26 us
    // against 41 us as 64 big ones; at K = 4096, 272 to 344 small tiles 61-63 us against 76-77
    // us as 68 to 86 big ones, 512 small tiles 74-76 us against 77 us as 128 big ones, 768
    // small tiles 112 us against 86 us as 192 big ones).
    const int64_t small_tiles = cdiv(M, tile_shape(kTile128x128w4).bm) * cdiv(N, tile_shape(kTile128x128w4).bn);
    if (p.tiles >= dev.cus) {
        p.reason = "256x256 tiles fill at least one wave";
    } else if (small_tiles > 2 * (int64_t)dev.cus) {
        p.reason = "128x128 tiles would need more than two per CU: 256x256 tiles";
    } else {
        set_tile(p, kTile128x128w4, M, N);
        p.reason = small_tiles > dev.cus ? "128x128 tiles, up to two per CU" : "128x128 tiles in one wave";
    }
    if (dev.force_tile_cfg >= 0 && dev.force_tile_cfg < kTileConfigCount) {
        set_tile(p, dev.force_tile_cfg, M, N);
        p.reason = "tile configuration forced";
    }
    const int64_t kt_total = cdiv(K, p.bk);
    p.group_m = (int)std::min<int64_t>(4, p.tiles_m);
    p.sched = kSchedDataParallel;
    p.splits = 1;
    p.kt_per_split = (int)kt_total;
    // workgroups resident at once: one per CU for the 256-wide tile (it takes all of LDS), two for
    // the 128x128 one
    p.slots = (int64_t)dev.cus * (p.tile_cfg == kTile128x128w4 ? 2 : 1);
    // only the smaller tiles carry the split fixup, and only grids of at most one tile per CU
    if (p.tiles <= dev.cus && kt_total > 1 && p.tile_cfg == kTile128x128w4) {
        // split K over the idle CUs; pieces are summed in K order by the last arriver, which
        // reads every other piece's float32 tile (BM*BN*4 bytes), one memory round trip per piece
        // (about 1.2 us), against about 0.4 us per k-step of a lone 128x128 workgroup. So with
        // at most one piece per CU the pieces number about sqrt(kt / 3) (measured, settled
        // clocks: 1024 x 1024 x 8192 in 4 pieces 32 us against 36 us in 8, two per CU; 1024 x
        // 2048 x 4096 in 2 pieces 30 us against 32 us in 4). When more than half the CUs hold a
        // tile, one piece per CU cannot split at all, and two per CU pay: co-resident pieces
        // run together at about 1.35 times a lone one's time, but each costs about 3.5-4 us of
        // fixup, so about sqrt(kt / 8) pieces, and none below 96 k-steps (K = 4096: 144 tiles in
        // 3 pieces 33 us against 46 us, 169 in 3 35.5 against 46, 240 in 2 42 against 46.6, 256
        // (one per CU) in 2 42.4 against 46.2; 256 tiles at K = 11008 in 2 94.9 against 116.2,
        // at K = 3072 35.2 against 36.1, at K = 2048 28.0 against 25.9; 144 tiles at K = 1024 in
        // 3 pieces 19.8 against 15.7 us, 196 at K = 2048 in 2 26.4 against 26.1).
        const int64_t per_cu = dev.cus / p.tiles;
        int64_t s = 1;
        if (per_cu >= 2) {
            int64_t root = 1;
            while ((root + 1) * (root + 1) * 3 <= kt_total) ++root;
            s = std::min<int64_t>(root, per_cu);
        } else if (kt_total >= 96) {
            int64_t root = 1;
            while ((root + 1) * (root + 1) * 8 <= kt_total) ++root;
            s = std::min<int64_t>(root, 2 * dev.cus / p.tiles);
        }
        s = std::max<int64_t>(s, 1);
        const int64_t slot_floats = (int64_t)p.bm * p.bn;
        while (s > 1 && p.tiles * s * slot_floats > dev.ws_floats) --s;
        if (s > 1 && p.tiles > dev.ws_counters) s = 1;
        if (s > 1) {
            p.kt_per_split = (int)cdiv(kt_total, s);
            p.splits = (int)cdiv(kt_total, p.kt_per_split);
            if (p.splits > 1) {
                p.sched = kSchedSplitK;
                p.ws_floats = p.tiles * p.splits * slot_floats;
                p.counters = p.tiles;
                p.reason += ", K split " + std::to_string(p.splits) + " ways";
            }
        }
    }
    p.grid = p.tiles * (p.sched == kSchedSplitK ? p.splits : 1);
    finish_waves(p);
    return p;
}

// A last wave of 256 x 256 tiles that is at most half full takes most of a full wave's time for a
// fraction of its work. Such a product is cut into the largest rectangle of whole tile rows or
// columns that fits in the full waves, planned as before, and the strip left over, planned on its
// own, which must come out as 128 x 128 tiles (at most two per CU, K split over idle CUs). Measured
// against one launch, interleaved, settled clocks, us (last wave's tiles in brackets): 4096 x 4352
// x 4096 (16) 121.7 against 170.5 (hipBLASLt 166.5), 4096 x 4608 x 4096 (32) 134.0 against 172.2,
// 4352^2 x 4096 (33) 136.1 against 172.3, 4096 x 4864 x 4096 (48) 144.1 against 175.7, 4096 x
// 5120 x 4096 (64) 147.1 against 173.3, 4608^3 (68) 181.0 against 194.3, 4096 x 5632 x 4096 (96)
// 168.8 against 178.0, 4096 x 6144 x 4096 (128) 174.3 against 180.1, 6144^3 (64, after two full
// waves) 379.5 against 391.1, 8192 x 8448 x 4096 (32, after four) 428.1 against 458.5; a fuller
// last wave lost (4096 x 11008 x 4096, 176: 284.8 against 278.2; 5120^3, 144: 219.4 against
// 217.2). The SwiGLU form is cut only across rows: its up half sits N weight columns after the
// gate half, so a column strip would need both halves' offsets.
static void cut_sparse_last_wave(Plan& p, int64_t M, int64_t W, int64_t K, const DeviceInfo& dev, bool glu) {
    if (p.kernel != kKernTile || p.tile_cfg != kTile256x256pp || p.sched != kSchedDataParallel) return;
    if (dev.force_tile_cfg >= 0) return;
    const int64_t slots = p.slots;
    const int64_t full = p.tiles / slots, last = p.tiles - full * slots;
    if (full < 1 || last == 0 || 2 * last > slots) return;
    const int64_t room = full * slots;
    int axis = 0;
    int64_t kept = 0, cut = 0;
    if (!glu) {  // keep the first tn tile columns
        const int64_t tn = room / p.tiles_m;
        if (tn >= 1 && tn < p.tiles_n) {
            axis = 1;
            kept = tn * p.tiles_m;
            cut = tn * p.bn;
        }
    }
    {  // keep the first tm tile rows
        const int64_t tm = room / p.tiles_n;
        if (tm >= 1 && tm < p.tiles_m && tm * p.tiles_n > kept) {
            axis = 2;
            kept = tm * p.tiles_n;
            cut = tm * p.bm;
        }
    }
    if (axis == 0) return;
    Plan rest = axis == 1 ? plan_tile(M, W - cut, K, dev) : plan_tile(M - cut, W, K, dev);
    if (rest.tile_cfg != kTile128x128w4) return;
    Plan q = axis == 1 ? plan_tile(M, cut, K, dev) : plan_tile(cut, W, K, dev);
    q.glu = rest.glu = glu;
    q.cut_axis = axis;
    q.cut_at = cut;
    q.ws_floats = std::max(q.ws_floats, rest.ws_floats);
    q.counters = std::max(q.counters, rest.counters);
    q.reason = "a last wave of " + std::to_string(last) + " of " + std::to_string(slots) +
               " 256x256 tiles is cut off: " + q.reason + " over the first " + std::to_string(cut) +
               (axis == 1 ? " columns" : " rows") + ", then the rest: " + rest.reason;
    q.rest.push_back(std::move(rest));
    p = std::move(q);
}

Plan make_plan(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev, bool fast_ok, int force,
               bool glu) {
    Plan p;
    p.glu = glu;
    if (M == 0 || N == 0) {
        p.kernel = kKernNone;
        p.reason = "empty output";
        return p;
    }
    if (K == 0) {
        p.kernel = kKernZero;
        p.grid = 1;
        p.reason = glu ? "K == 0: gate and up are empty sums, silu(0) * 0 = 0" : "K == 0: C is the empty sum";
        return p;
    }
    if (!fast_ok) {
        p.kernel = kKernGeneric;
        p.grid = cdiv(M, 64) * cdiv(N, 64);
        p.threads = 256;
        p.slots = (int64_t)dev.cus * 4;
        finish_waves(p);
        p.reason = "alignment, leading dimension or size outside the fast kernels";
        return p;
    }
    // the fast kernels of the SwiGLU form stream gate and up columns side by side: they are
    // planned over the 2N weight columns
    const int64_t W = glu ? 2 * N : N;
    // the skinny kernel counts its (strip, stage) units in 32 bits
    const bool units_fit = cdiv(W, kSkinnyStripMin) * cdiv(K, kSkinnyStage) <= INT32_MAX;
    const bool skinny = units_fit && ((force == 1) || (force == 0 && M <= 64));
    Plan q = skinny ? plan_skinny(M, W, K, dev, glu) : plan_tile(M, W, K, dev);
    q.glu = glu;
    if (!skinny) cut_sparse_last_wave(q, M, W, K, dev, glu);
    return q;
}

// Block-scaled decode: a workgroup streams the packed weights of 4 column tiles (64 columns) over
// one of S pieces of K, its 4 waves each holding two k-steps of loads in flight in registers.
// Splitting K costs a float32 fixup (about 2 us per call on the 11008 x 4096 weight, measured),
// so K stays whole when one piece per group already covers 60% of the CUs (the 172 groups of an
// 11008-wide weight: 8.3 us at M = 1 against 9.7 at S = 2) and is otherwise cut just far enough to
// cover them all (the 64 groups of a 4096-wide weight: S = 4, 9.7 us, against 14.6 at S = 1 and
// 10.1 at S = 3). Every wave keeps at least one k-step.
// groups of `tpg` column tiles times K pieces over `ks` k-steps (see the comment above)
static Plan decode_groups_plan(int kind, int64_t M, int64_t N, int64_t K, int64_t ks, int tpg,
                               const DeviceInfo& dev) {
    Plan p;
    p.kernel = kind;
    if (M == 0 || N == 0) {
        p.kernel = kKernNone;
        p.reason = "empty output";
        return p;
    }
    if (K == 0) {
        p.kernel = kKernZero;
        p.grid = 1;
        p.reason = "K == 0: C is the empty sum";
        return p;
    }
    // the block-scaled decode's groups go to the XCDs in the hardware's round-robin order: measured
    // against keeping a group's pieces (and neighbouring groups) on one XCD, us, same bits:
    // 4096-wide weight at M = 1, 16, 64 9.75 -> 9.50, 10.27 -> 10.13, 19.21 -> 19.04; 11008-wide
    // at M = 1 7.92 -> 7.62
    p.nxcd = kind == kKernMx ? 1 : dev.nxcd;
    p.threads = 256;
    p.mtiles = (int)cdiv(M, 16);
    p.tiles_n = N / 16;
    p.strips = (int)cdiv(p.tiles_n, tpg);
    p.strip = 16 * tpg;
    p.ks = (int)ks;
    const int64_t per_cu = p.mtiles <= 2 ? 2 : 1;  // waves' registers: two workgroups per CU
    p.slots = per_cu * dev.cus;
    int64_t s = (5 * p.strips >= 3 * (int64_t)dev.cus) ? 1 : cdiv(dev.cus, p.strips);
    s = std::min<int64_t>(s, std::max<int64_t>(1, p.ks / 4));
    const int64_t slot_floats = (int64_t)tpg * p.mtiles * 256;
    while (s > 1 && p.strips * s * slot_floats > dev.ws_floats) --s;
    if (s > 1 && p.strips > dev.ws_counters) s = 1;
    p.splits = (int)s;
    p.grid = p.strips * s;
    p.ws_floats = s > 1 ? p.strips * s * slot_floats : 0;
    p.counters = s > 1 ? p.strips : 0;
    finish_waves(p);
    p.reason = std::string(kind == kKernMx ? "MXFP8 x MXFP4 decode: " : "packed bf16 decode: ") +
               std::to_string(p.strips) + " groups of " + std::to_string(tpg) + " column tiles, K in " +
               std::to_string(s) + " pieces";
    return p;
}

// Workgroups of four column tiles, or of three where that spreads the weight over more CUs: the
// product streams the weight, and a CU left without a workgroup adds nothing to the read rate
// (11008 columns: 172 groups of four against 230 of three, 6% faster at 16 and 64 rows; 4096
// columns: 64 groups of four in 4 K pieces fill 256 CUs exactly and stay).
Plan make_mx_plan(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev) {
    Plan best;
    double best_fill = -1.0;
    for (int tn : {4, 3}) {
        Plan q = decode_groups_plan(kKernMx, M, N, K, K / 128, tn, dev);
        if (q.kernel != kKernMx) return q;
        // how full the rounds of CUs are: the grid over rounds x CUs
        const int64_t rounds = cdiv(q.grid, (int64_t)dev.cus);
        const double fill = (double)q.grid / (double)(rounds * dev.cus);
        if (fill > best_fill + 1e-9) {
            best = q;
            best_fill = fill;
        }
    }
    return best;
}

// The packed bf16 decode reads the same kind of 1 KB operand blocks over 32-k steps.
Plan make_packed_plan(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev) {
    return decode_groups_plan(kKernPacked, M, N, K, K / 32, pk_decode_tiles_per_group(M), dev);
}

static const char* kernel_name(int k) {
    switch (k) {
        case kKernNone: return "none";
        case kKernZero: return "zero";
        case kKernGeneric: return "generic";
        case kKernTile: return "tile";
        case kKernSkinny: return "skinny";
        case kKernMx: return "mx";
        case kKernPacked: return "packed";
        default: return "?";
    }
}

std::string plan_json(const Plan& p, int64_t M, int64_t N, int64_t K) {
    char buf[4096];
    snprintf(buf, sizeof buf,
             "{\"M\": %lld, \"N\": %lld, \"K\": %lld, \"kernel\": \"%s\", \"bm\": %d, \"bn\": %d, "
             "\"bk\": %d, \"threads\": %d, \"tiles_m\": %lld, \"tiles_n\": %lld, \"tiles\": %lld, "
             "\"schedule\": \"%s\", \"splits\": %d, \"kt_per_split\": %d, \"group_m\": %d, "
             "\"nxcd\": %d, \"mtiles\": %d, \"strip\": %d, \"strips\": %d, \"ks\": %d, \"grid\": %lld, "
             "\"slots\": %lld, \"waves\": %lld, \"wave_eff\": %.6f, \"ws_floats\": %lld, "
             "\"op\": \"%s\", \"reason\": \"%s\"}",
             (long long)M, (long long)N, (long long)K, kernel_name(p.kernel), p.bm, p.bn, p.bk,
             p.threads, (long long)p.tiles_m, (long long)p.tiles_n, (long long)p.tiles,
             p.kernel == kKernTile ? (p.sched == kSchedSplitK ? "split-k" : "data-parallel")
                                   : (p.kernel == kKernSkinny || p.kernel == kKernMx || p.kernel == kKernPacked
                                          ? "strips"
                                          : "-"),
             p.splits, p.kt_per_split, p.group_m, p.nxcd, p.mtiles, p.strip, p.strips, p.ks,
             (long long)p.grid, (long long)p.slots, (long long)p.waves, p.wave_eff,
             (long long)p.ws_floats,
             p.kernel == kKernMx ? "mx" : (p.kernel == kKernPacked ? "packed" : (p.glu ? "swiglu" : "gemm")),
             p.reason.c_str());
    std::string s(buf);
    if (p.cut_axis != 0 && !p.rest.empty()) {
        // the strip left over: its own plan, over its own sizes
        const int64_t Mr = p.cut_axis == 2 ? M - p.cut_at : M;
        const int64_t Nr = p.cut_axis == 1 ? N - p.cut_at : N;
        s.pop_back();
        s += ", \"cut\": {\"axis\": \"" + std::string(p.cut_axis == 1 ? "n" : "m") +
             "\", \"at\": " + std::to_string(p.cut_at) + ", \"rest\": " + plan_json(p.rest[0], Mr, Nr, K) + "}}";
    }
    return s;
}

}  // namespace glk
