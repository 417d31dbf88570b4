// General bf16 GEMM for operands the fast kernels do not take (unaligned pointers, leading
// dimensions or N, K not multiples of 8, extents beyond the fast kernels' 32-bit offsets).
// Same contract: bf16 in, float32 accumulation, bf16 out (round to nearest even). Element-wise
// bounds-checked loads through LDS; each thread accumulates a 4 x 4 block with float32 FMAs.
// The SwiGLU form (GLU = true) keeps a second accumulator block for the up half of B (columns
// N .. 2N-1) and writes silu(gate) * up.
// Also the zero-fill for K == 0 and a plain 32-bit fill used to poison outputs and evict caches.

#include "common.h"
#include "kernels.h"

namespace glk {

__device__ __forceinline__ float load_bf16(const uint16_t* p) {
    return __builtin_bit_cast(float, (uint32_t)(*p) << 16);
}

template <bool GLU>
__global__ void __launch_bounds__(256) generic_gemm_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ B,
                                                           uint16_t* __restrict__ C, int64_t M,
                                                           int64_t N, int64_t K, int64_t lda,
                                                           int64_t ldb, int64_t ldc) {
    constexpr int T = 64, KS = 16;
    __shared__ float sa[KS][T + 1];
    __shared__ float sb[KS][T + 1];
    __shared__ float su[GLU ? KS : 1][T + 1];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * T, n0 = (int64_t)blockIdx.x * T;
    float acc[4][4] = {};
    float accu[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += KS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            const int kk = e & (KS - 1), mm = e >> 4;
            const int64_t m = m0 + mm, k = k0 + kk;
            sa[kk][mm] = (m < M && k < K) ? load_bf16(A + m * lda + k) : 0.f;
            const int kb = e >> 6, nn = e & 63;
            const int64_t kr = k0 + kb, n = n0 + nn;
            sb[kb][nn] = (kr < K && n < N) ? load_bf16(B + kr * ldb + n) : 0.f;
            if constexpr (GLU) su[kb][nn] = (kr < K && n < N) ? load_bf16(B + kr * ldb + N + n) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sa[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sb[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
            if constexpr (GLU) {
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = su[kk][tx * 4 + j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) accu[i][j] = __builtin_fmaf(a[i], b[j], accu[i][j]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            const float h = GLU ? swiglu1(acc[i][j], accu[i][j]) : acc[i][j];
            if (n < N) C[m * ldc + n] = __builtin_bit_cast(uint16_t, (__bf16)h);
        }
    }
}

__global__ void __launch_bounds__(256) zero_c_kernel(uint16_t* C, int64_t M, int64_t N, int64_t ldc) {
    const int64_t total = M * N;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t m = e / N, n = e - m * N;
        C[m * ldc + n] = 0;
    }
}

__global__ void __launch_bounds__(256) fill_kernel(uint32_t* dst, int64_t words, uint32_t v) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t vec = words / 4;
    u32x4* d4 = reinterpret_cast<u32x4*>(dst);
    const u32x4 vv = {v, v, v, v};
    for (int64_t i = e; i < vec; i += stride) d4[i] = vv;
    for (int64_t i = vec * 4 + e; i < words; i += stride) dst[i] = v;
}

hipError_t launch_generic_gemm(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M,
                               int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                               bool glu, hipStream_t s) {
    const int64_t gx = (N + 63) / 64, gy = (M + 63) / 64;
    if (gx > 0x7FFFFFFF || gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    if (glu)
        generic_gemm_kernel<true><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    else
        generic_gemm_kernel<false><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    return hipGetLastError();
}

hipError_t launch_zero_c(uint16_t* C, int64_t M, int64_t N, int64_t ldc, hipStream_t s) {
    const int64_t total = M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    zero_c_kernel<<<(unsigned)blocks, 256, 0, s>>>(C, M, N, ldc);
    return hipGetLastError();
}

hipError_t launch_fill(void* dst, int64_t bytes, uint32_t value, hipStream_t s) {
    const int64_t words = bytes / 4;
    int64_t blocks = (words / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    fill_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint32_t*>(dst), words, value);
    return hipGetLastError();
}

}  // namespace glk
