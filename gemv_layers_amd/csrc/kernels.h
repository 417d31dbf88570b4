// Host-visible launch interfaces of the library's kernels (internal header): each kernel
// family's own header, the general fallback and the measurement kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx.h"
#include "packed.h"
#include "skinny.h"
#include "tile.h"

namespace glk {

// ---- general fallback (any alignment / leading dimension) ----------------------------------
hipError_t launch_generic_gemm(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M,
                               int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                               bool glu, hipStream_t s);

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
