// Host-visible launch interfaces of the library's kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stream_k.h"

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

// ---- general fallback (any alignment / leading dimension) ----------------------------------
hipError_t launch_generic_gemm(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M,
                               int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                               bool glu, hipStream_t s);

// ---- skinny-M weight-streaming GEMM ---------------------------------------------------------
struct SkinnyArgs {
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* C;
    int M, N, K;
    int lda, ldb, ldc;
    int strips;          // column strips of B (the launch's strip width, 128 or 256 columns, each)
    int ks;              // 64-row stages per strip, ceil(K / 64)
    int grid;            // workgroups; logical workgroup w takes range w of `split`
    UnitSplit split;     // grid balanced ranges of the strip-major list of U = strips * ks
                         // (strip, stage) units, U < 2^31
    int nxcd;            // XCDs the hardware deals workgroups over; logical ids are contiguous per
                         // XCD, so the pieces of a strip meet in one XCD (1 = no remap)
    float* ws;           // 2 * grid * skinny_slot_floats(mtiles) floats
    uint32_t* counters;  // one per strip, zero between launches
};
constexpr int kSkinnyStripMin = 128;  // narrowest strip (columns)
constexpr int kSkinnyStage = 64;    // k rows per streamed unit
// strip: 128 or 256 columns; glu: the SwiGLU form (strips cover the 2N weight columns, a strip
// makes strip / 2 outputs; SkinnyArgs.N is the output width N)
hipError_t launch_skinny_gemm(int mtiles, int strip, bool glu, const SkinnyArgs& a, hipStream_t s);
hipError_t configure_skinny_kernels();
int skinny_slot_floats(int mtiles, int strip);  // workspace floats per piece

// ---- block-scaled (MX) decode product ------------------------------------------------------
// C = deq(Aq) * deq(W)^T: Aq MXFP8 (E4M3, M x K row-major, ldaq bytes per row; scales M x K/32,
// ldas bytes per row), W MXFP4 in the packed layout (codes Wp, scales Sp; see gemm_mx.hip).
struct MxArgs {
    const uint8_t* Aq;
    const uint8_t* As;
    const uint8_t* Wp;
    const uint8_t* Sp;
    uint16_t* C;
    int M, N, K;
    int ldaq, ldas, ldc;
    int tiles;           // N / 16 column tiles
    int ks, kq;          // K / 128 k-steps; ceil(ks / 4) scale groups
    int pieces;          // K pieces per group of TN column tiles (one workgroup each)
    int nxcd;            // XCDs the hardware deals workgroups over (1 = no remap)
    float* ws;           // pieces > 1: groups * pieces * 4 * mtiles * 256 floats
    uint32_t* counters;  // one per group, zero between launches
    // the fused form (bf16 activations converted in the kernel, M <= 2): A16 (M x K bf16, lda16
    // elements per row), LDS row stride kpb bytes and reduction offset red_off (mx_fused_layout)
    const uint16_t* A16;
    int lda16;
    int kpb, red_off;
};
// tn: column tiles per workgroup, 3 or 4 (the plan's strip / 16)
int mx_fused_layout(int piece_ks, int tn, MxArgs& a);  // LDS bytes of the fused form, or -1
hipError_t launch_mx_decode_fused(int tn, const MxArgs& a, int grid, int lds_bytes, hipStream_t s);
int mx_decode_lds_bytes(int mtiles, int tn);
hipError_t configure_mx_kernels();
hipError_t launch_mx_decode(int mtiles, int tn, const MxArgs& a, int grid, hipStream_t s);
// bf16 rows -> MX codes and scales: fp4 = false, E4M3 row-major (Q: ldq bytes per row, S: lds);
// fp4 = true, E2M1 in the packed weight layout (rows % 16 == 0, cols % 128 == 0; ldq, lds unused)
hipError_t launch_mx_quant(bool fp4, const uint16_t* X, int rows, int cols, int ldx, uint8_t* Q, int ldq,
                           uint8_t* S, int lds, hipStream_t s);

// ---- decode product on a packed bf16 weight ---------------------------------------------------
// C = A * B with B (K x N) in the packed layout of gemm_packed.hip (K % 32 == 0, N % 16 == 0).
struct PkArgs {
    const uint16_t* A;
    const uint16_t* Bp;
    uint16_t* C;
    int M, N, K;
    int lda, ldc;
    int tiles;           // N / 16 column tiles
    int ks;              // K / 32 k-steps
    int pieces;          // K pieces per group of pk_decode_tiles_per_group(M) tiles (one workgroup each)
    int nxcd;            // XCDs the hardware deals workgroups over (1 = no remap)
    float* ws;           // pieces > 1: groups * pieces * tiles_per_group * mtiles * 256 floats
    uint32_t* counters;  // one per group, zero between launches
};
int pk_decode_tiles_per_group(int64_t M);
int pk_decode_lds_bytes(int mtiles, int tpg);
hipError_t configure_pk_kernels();
// tpg: pk_decode_tiles_per_group(M)
hipError_t launch_pk_decode(int mtiles, int tpg, const PkArgs& a, int grid, hipStream_t s);
hipError_t launch_pk_pack(const uint16_t* B, int K, int N, int ldb, uint16_t* P, hipStream_t s);

// ---- misc ------------------------------------------------------------------------------------
hipError_t launch_zero_c(uint16_t* C, int64_t M, int64_t N, int64_t ldc, hipStream_t s);
hipError_t launch_fill(void* dst, int64_t bytes, uint32_t value, hipStream_t s);
hipError_t launch_peak_mfma(int64_t iters, int blocks, float* sink, uint64_t* cycles,
                            hipStream_t s);
hipError_t launch_peak_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
hipError_t launch_peak_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_peak_empty(hipStream_t s);
hipError_t launch_peak_clock(int64_t iters, int blocks, uint64_t* out, hipStream_t s);
hipError_t launch_peak_xcc(int blocks, uint32_t* out, hipStream_t s);

}  // namespace glk
