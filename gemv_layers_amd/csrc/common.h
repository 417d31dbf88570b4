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

// `off` when `valid`, else an out-of-range offset; branch-free so that no control flow (and no
// conservative wait at a merge point) ends up between a wave's outstanding loads.
__device__ __forceinline__ uint32_t sel_off(bool valid, uint32_t off) {
    const uint32_t m = 0u - (uint32_t)valid;
    return (off & m) | (kBufInvalid & ~m);
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

// Cache policy for workspace traffic shared between workgroups on different XCDs: device scope
// (sc1), so stores are written through to the device coherence point and loads do not hit
// stale lines in another XCD's L2. Publishing a partial is then: device-scope stores, wait for
// them to complete, workgroup barrier, one device-scope counter increment. No cache-wide
// write-back or invalidate is needed.
constexpr int kAuxDevice = 16;
// Non-temporal (streaming) stores: data written once and not read back by this kernel.
constexpr int kAuxNonTemporal = 2;

__device__ __forceinline__ void buf_store16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kAuxDevice);
}

__device__ __forceinline__ u32x4 buf_load16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxDevice);
}

// Wait for this wave's outstanding vector-memory operations down to N (gfx9 s_waitcnt encoding,
// other counters unconstrained). Direct-to-LDS loads count here until their data is in LDS.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait for this wave's outstanding LDS operations.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }

// Workgroup barrier for LDS rings fed by direct-to-LDS loads. Unlike __syncthreads() it carries
// no memory fence, so it does not drain the loads still in flight for later stages; each wave
// first waits (wait_vmcnt) for exactly the loads the next stage needs and for its own LDS reads.
// The empty asm statements stop the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    wait_lgkmcnt0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ uint32_t counter_arrive(uint32_t* c) {
    return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void counter_reset(uint32_t* c) {
    __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ u32x4 f4_bits(f32x4 v) { return __builtin_bit_cast(u32x4, v); }
__device__ __forceinline__ f32x4 bits_f4(u32x4 v) { return __builtin_bit_cast(f32x4, v); }

// ---- direct-to-LDS loads --------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// Raw buffer descriptor words (base, stride 0, `bytes` records, raw word 3) for inline asm.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, kBufWord3};
}

// Each lane copies 16 bytes from descriptor + voff into LDS at lds_base + 16 * lane, without
// passing through registers. Issued from inline asm so that the compiler does not treat every
// later LDS read as possibly depending on it (it would wait for all loads in flight before each
// read); callers order it explicitly with wait_vmcnt<>() and a barrier. Offsets at or beyond the
// descriptor's range deliver zeros.
// (m0 is reserved, so clang warns that listing it as clobbered does not make it save m0; nothing
// in these kernels keeps a value in m0 across the statement.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_base, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// float32 pair -> two bf16 (round to nearest even; gfx950 v_cvt_pk_bf16_f32), low half = lo.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// SwiGLU of one gate/up accumulator pair: silu(g) * u, silu(x) = x / (1 + e^-x), in float32 with
// the library exponential and IEEE division. Large g gives g * u; below about -88 the exponential
// overflows and the result is -0 * u, the float32 limit of the exact value.
__device__ __forceinline__ float swiglu1(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__device__ __forceinline__ f32x4 swiglu4(f32x4 g, f32x4 u) {
    return f32x4{swiglu1(g[0], u[0]), swiglu1(g[1], u[1]), swiglu1(g[2], u[2]), swiglu1(g[3], u[3])};
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

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
