// Launch interface of the block-scaled (MX) decode kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glk {

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

}  // namespace glk
