// Launch interface of the packed-bf16-weight decode kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glk {

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

}  // namespace glk
