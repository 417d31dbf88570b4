// Host planner: closed-form choice of kernel, tile, schedule and split for one product.
// Plain C++ (no HIP), so it runs and is tested on machines without a GPU.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

namespace glk {

enum KernelKind : int {
    kKernNone = 0, kKernZero = 1, kKernGeneric = 2, kKernTile = 3, kKernSkinny = 4, kKernMx = 5,
    kKernPacked = 6
};

struct Plan {
    int kernel = kKernNone;
    bool glu = false;        // the SwiGLU form: outputs N, weight columns 2N
    // large-tile kernel
    int tile_cfg = 0;
    int bm = 0, bn = 0, bk = 64;
    int threads = 0;
    int64_t tiles_m = 0, tiles_n = 0, tiles = 0;
    int sched = 0;           // 0 data-parallel, 1 split-K
    int splits = 1;          // pieces per tile (tile) or K slices per strip (skinny)
    int kt_per_split = 0;    // k-steps per piece (tile)
    int group_m = 1;
    int nxcd = 1;
    // skinny kernel
    int mtiles = 0;          // 16-row tiles of M
    int strip = 128;         // skinny strip width: 128 or 256 columns
    int strips = 0;          // column strips
    int ks = 0;              // 64-row stages per strip (skinny: units = strips * ks)
    // launch
    int64_t grid = 0;
    int64_t slots = 0;       // workgroups resident at once
    int64_t waves = 0;       // ceil(grid / slots)
    double wave_eff = 0.0;   // (grid / slots) / waves
    int64_t ws_floats = 0;   // workspace floats the launch uses
    int64_t counters = 0;    // workspace counters the launch uses
    // A product whose last wave of 256 x 256 tiles would be at most half full is cut in two: this
    // plan then covers the first `cut_at` output columns (cut_axis 1) or rows (cut_axis 2), and
    // rest[0] the remaining strip, launched after it on the same stream (ws_floats and counters
    // are then the larger of the two parts' needs).
    int cut_axis = 0;
    int64_t cut_at = 0;
    std::vector<Plan> rest;
    std::string reason;
};

struct DeviceInfo {
    int cus = 256;
    int nxcd = 8;
    int64_t ws_floats = 0;   // workspace capacity
    int64_t ws_counters = 0;
    int force_tile_cfg = -1; // debug: force a large-tile configuration (GEMM_BF16_FORCE_TILE)
};

// Wave quantization ("Kernel development on sm_120", section 4, budget 4):
// efficiency = (ctas / slots) / ceil(ctas / slots).
void wave_efficiency(int64_t ctas, int64_t slots, double* eff, int64_t* waves);

// True when the fast kernels can take these operands (alignment, multiples of 8, 32-bit offsets).
bool fast_path_ok(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                  int64_t ldb, const void* C, int64_t ldc);

// force: 0 = dispatch on M, 1 = skinny kernel, 2 = large-tile family. glu: plan the SwiGLU form,
// whose kernels stream 2N weight columns (gate, then up) for N outputs.
Plan make_plan(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev, bool fast_ok, int force,
               bool glu = false);

// The block-scaled decode product (1 <= M <= 64, N % 16 == 0, K % 128 == 0): groups of column
// tiles (strips) times K pieces (splits), one workgroup each.
Plan make_mx_plan(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev);

// The decode product on a packed bf16 weight (1 <= M <= 64, N % 16 == 0, K % 32 == 0): the same
// decomposition over 32-k steps.
Plan make_packed_plan(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev);

std::string plan_json(const Plan& p, int64_t M, int64_t N, int64_t K);

}  // namespace glk
