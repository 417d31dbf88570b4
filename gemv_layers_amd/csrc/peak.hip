// Roof measurements for this card (spark-kernels post, "how things are measured": a loop of
// register-resident matrix instructions for the compute peak, read with the clock counter during
// the loop, and a device-to-device copy for the memory roof; "the decode kernel": a kernel that
// only reads with 16-byte loads, and an empty launch; "Kernel development on sm_120", section 1:
// back-to-back matrix instructions on register-resident operands with several independent
// accumulator chains).

#include "common.h"
#include "kernels.h"

namespace glk {

// 8 independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave; operands stay in
// registers. Each instruction is 2 * 32 * 32 * 16 = 32768 flops.
__global__ void __launch_bounds__(256) peak_mfma_kernel(int64_t iters, float* sink, uint64_t* cycles) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 0.0078125f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.5f - 0.0078125f * (float)((lane * 3 + e) & 7));
    }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x16{};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = mfma32(a, b, acc[c]);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        cycles[2 * (size_t)blockIdx.x] = t1 - t0;
        cycles[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

// The matrix cores' rate on operands read from memory: v_mfma_f32_16x16x32_bf16 in the register
// layout of the large-tile kernel's wave tile (128 float accumulators per lane in 4 x 8 16 x 16
// blocks, 8 waves per workgroup, 2 per SIMD), 32 instructions per iteration on 8 A and 4 B
// operand registers loaded once from `ops`. Under the board's power limit the clock depends on
// how many operand bits toggle: random operands give the ceiling for products of random data,
// where the register-only loop above, with near-constant operands, gives the ceiling at the
// clock limit. Each instruction is 2 * 16 * 16 * 32 = 16384 flops.
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
peak_mfma_data_kernel(const u32x4* __restrict__ ops, int64_t iters, float* sink, uint64_t* cycles) {
    const int t = threadIdx.x;
    bf16x8 a[8], b[4];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = __builtin_bit_cast(bf16x8, ops[(q * 512 + t) & 2047]);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = __builtin_bit_cast(bf16x8, ops[2048 + ((q * 512 + t) & 1023)]);
    wait_all_memory();  // operands in registers before the timed loop
    __syncthreads();
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(b[i], a[j], acc[i][j]);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    sink[(size_t)blockIdx.x * 512 + t] = s;
    if (t == 0) {
        cycles[2 * (size_t)blockIdx.x] = t1 - t0;
        cycles[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

hipError_t launch_peak_mfma_data(const void* ops, int64_t iters, int blocks, float* sink, uint64_t* cycles,
                                 hipStream_t s) {
    peak_mfma_data_kernel<<<blocks, 512, 0, s>>>(static_cast<const u32x4*>(ops), iters, sink, cycles);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256) peak_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    int64_t i = ((int64_t)blockIdx.x * 256 * 4) + threadIdx.x;
    // 4 independent 16-byte loads in flight per thread per iteration
    for (; i + 3 * 256 < n16; i += stride) {
        const u32x4 v0 = __builtin_nontemporal_load(src + i);
        const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
        const u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
        const u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
        __builtin_nontemporal_store(v0, dst + i);
        __builtin_nontemporal_store(v1, dst + i + 256);
        __builtin_nontemporal_store(v2, dst + i + 512);
        __builtin_nontemporal_store(v3, dst + i + 768);
    }
    for (int u = 0; u < 4; ++u) {
        const int64_t j = i + u * 256;
        if (j < n16) dst[j] = src[j];
    }
}

__global__ void __launch_bounds__(256) peak_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                        uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    int64_t i = ((int64_t)blockIdx.x * 256 * 4) + threadIdx.x;
    uint32_t x = 0;
    for (; i + 3 * 256 < n16; i += stride) {
        const u32x4 v0 = __builtin_nontemporal_load(src + i);
        const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
        const u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
        const u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
        x ^= v0[0] ^ v1[1] ^ v2[2] ^ v3[3];
    }
    for (int u = 0; u < 4; ++u) {
        const int64_t j = i + u * 256;
        if (j < n16) x ^= src[j][0];
    }
    // one word per workgroup keeps the loads alive
    __shared__ uint32_t red[256];
    red[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int k = 0; k < 256; ++k) t ^= red[k];
        sink[blockIdx.x & 0xFFFF] = t;
    }
}

__global__ void peak_empty_kernel() {}

// Shader-clock probe: wave 0 of each workgroup reads the core-clock counter (s_memtime) and the
// 100 MHz constant counter (s_memrealtime) around a dependent FMA chain. Power management moves
// the clock over milliseconds, so a probe enqueued right behind a stream of kernels reads the
// clock the card held under that load.
__global__ void __launch_bounds__(64) peak_clock_kernel(int64_t iters, uint64_t* out) {
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    float x = (float)threadIdx.x;
    for (int64_t i = 0; i < iters; ++i) x = __builtin_fmaf(x, 0.999f, 0.5f);
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * (size_t)blockIdx.x] = t1 - t0;
        out[2 * (size_t)blockIdx.x + 1] = (x == -1.0f) ? 0 : r1 - r0;  // x kept alive
    }
}

// Placement probe: each workgroup records the XCD (accelerator complex die) it runs on, from the
// XCC_ID hardware register (its low 4 bits). The tile and strip orders assume that the dispatcher
// deals consecutive workgroups to the XCDs round robin; this probe lets a test check it.
__global__ void __launch_bounds__(64) peak_xcc_kernel(uint32_t* out) {
    uint32_t x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    if (threadIdx.x == 0) out[blockIdx.x] = x & 15u;
}

hipError_t launch_peak_xcc(int blocks, uint32_t* out, hipStream_t s) {
    peak_xcc_kernel<<<blocks, 64, 0, s>>>(out);
    return hipGetLastError();
}

hipError_t launch_peak_mfma(int64_t iters, int blocks, float* sink, uint64_t* cycles, hipStream_t s) {
    peak_mfma_kernel<<<blocks, 256, 0, s>>>(iters, sink, cycles);
    return hipGetLastError();
}

static int stream_blocks(int64_t n16) {
    int64_t b = (n16 + 1023) / 1024;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (int)b;
}

hipError_t launch_peak_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    peak_copy_kernel<<<stream_blocks(n16), 256, 0, s>>>(static_cast<const u32x4*>(src),
                                                       static_cast<u32x4*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_peak_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    peak_read_kernel<<<stream_blocks(n16), 256, 0, s>>>(static_cast<const u32x4*>(src), n16, sink);
    return hipGetLastError();
}

hipError_t launch_peak_clock(int64_t iters, int blocks, uint64_t* out, hipStream_t s) {
    peak_clock_kernel<<<blocks, 64, 0, s>>>(iters, out);
    return hipGetLastError();
}

hipError_t launch_peak_empty(hipStream_t s) {
    peak_empty_kernel<<<1, 64, 0, s>>>();
    return hipGetLastError();
}

}  // namespace glk
