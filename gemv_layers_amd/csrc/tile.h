// Launch interface of the large-tile MFMA GEMM kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glk {

// ---- large-tile MFMA GEMM -------------------------------------------------------------------

// How the flattened work of a launch is cut. Data-parallel: one workgroup per output tile.
// Split: tile t's K range is cut into `splits` contiguous pieces of `kt_per_split` k-steps, one
// workgroup per piece; pieces meet in a per-tile float32 fixup summed in K order.
enum TileSchedule : int { kSchedDataParallel = 0, kSchedSplitK = 1 };

struct TileArgs {
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* C;
    int M, N, K;
    int lda, ldb, ldc;
    int tiles_m, tiles_n;
    int group_m;        // tile rows per group of the grouped (L2-friendly) tile order
    int nxcd;           // XCDs the hardware deals workgroups over (8 on MI355X), 1 = no remap
    int sched;          // TileSchedule
    int splits;         // pieces per tile (split schedule)
    int kt_per_split;   // k-steps (of the tile's BK) per piece (split schedule)
    float* ws;          // split partial slots, splits * tiles * BM * BN floats
    uint32_t* counters; // one per tile, zero between launches
};

// Tile configurations compiled into the library.
enum TileConfig : int {
    kTile256x256w8 = 0,  // 256 x 256 tile, 8 waves of 128 x 64, all in step (kept for comparison)
    kTile128x128w4 = 1,  // 128 x 128 tile, 4 waves of 64 x 64
    kTile256x256pp = 2,  // 256 x 256 tile, 8 waves in two groups alternating MFMA and memory phases
    kTileConfigCount
};

struct TileShape {
    int bm, bn, bk, threads;
};
TileShape tile_shape(int cfg);
// glu: the SwiGLU form, C = silu(A B[:, :N]) * (A B[:, N:2N]) with B K x 2N (TileArgs.N is the
// output width N; tiles_n counts BN-wide tiles over the 2N weight columns)
hipError_t launch_tile_gemm(int cfg, const TileArgs& a, int grid, bool glu, hipStream_t s);
hipError_t configure_tile_kernels();

}  // namespace glk
