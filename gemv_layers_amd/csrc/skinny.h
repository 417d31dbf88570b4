// Launch interface of the skinny-M weight-streaming kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stream_k.h"

namespace glk {

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

}  // namespace glk
