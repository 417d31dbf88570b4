// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer descriptor word 3 for the gfx9 family (32-bit data format, no swizzle).
constexpr int kBufWord3 = 0x00020000;
// num_records of every descriptor; an offset at or above it reads zeros and drops stores, which
// is how out-of-range tile elements are zero-filled without branches.
constexpr uint32_t kBufRecords = 0x7FFFFFF0u;
constexpr uint32_t kBufInvalid = 0x7FFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)kBufRecords,
                                             kBufWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// float32 pair -> two bf16 (round to nearest even; gfx950 v_cvt_pk_bf16_f32), low half = lo.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Transpose of an 8 x 8 block of 16-bit values held as 8 rows of 4 dwords (row r, dword q holds
// columns 2q (low half) and 2q+1 (high half)). Output column c as 4 dwords, dword p holding rows
// 2p (low half) and 2p+1 (high half).
__device__ __forceinline__ void transpose8x8_b16(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t x = in[2 * p][q], y = in[2 * p + 1][q];
            // even column 2q: low halves of rows 2p, 2p+1; odd column 2q+1: high halves
            out[2 * q][p] = __builtin_amdgcn_perm(y, x, 0x05040100u);
            out[2 * q + 1][p] = __builtin_amdgcn_perm(y, x, 0x07060302u);
        }
    }
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Map a hardware workgroup id onto a logical id so that each XCD's share of the grid (the
// hardware hands consecutive ids to the XCDs round robin) is one contiguous range of logical
// ids. Bijective on [0, total) for any total.
__device__ __forceinline__ int xcd_remap(int bid, int total, int nxcd) {
    if (nxcd <= 1) return bid;
    const int x = bid % nxcd, l = bid / nxcd;
    const int q = total / nxcd, r = total % nxcd;
    return x * q + (x < r ? x : r) + l;
}

}  // namespace glk
