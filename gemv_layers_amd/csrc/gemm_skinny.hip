// Skinny-M bf16 GEMM for gfx950 (1 <= M <= 64): C = A * B where B (K x N) is streamed from HBM
// exactly once for all M rows, float32 accumulation, bf16 output.
//
// Design ("The kernels that were there", "The GEMV": load-bound, so parallelise over output
// columns, coalesced 128-bit weight loads, fp32 accumulation, every weight loaded once for all
// rows; spark-kernels post, "the decode kernel": a tile of 16/32/64 rows picked from M, one
// workgroup per column strip of B, and K split only as far as needed to fill the card, the last
// slice leaving the workspace as it found it so a call stays one launch):
//
// * A workgroup owns a strip of 128 columns and one K slice; its 4 waves take the slice's
//   32-row k-blocks in turn. Each lane loads an 8 x 8 bf16 block of B (8 rows x 16 bytes, the 16
//   lanes of a row group covering 256 contiguous bytes of a row), two k-blocks ahead of use.
// * The block is transposed in registers so that column c of the block is the first operand of
//   v_mfma_f32_16x16x32_bf16 (row i of that operand = column 8*i + c of the strip); the second
//   operand is 16 rows of A, loaded from L2 as 16 bytes per lane. M is padded to 16 per tile with
//   zeros (the matrix cores are idle in a memory-bound kernel, so the padding costs no time).
// * The 4 waves' float32 partials are added in LDS in wave order. With more than one K slice,
//   each slice writes its strip partial to a workspace slot and bumps a per-strip counter; the
//   last arriver adds the slices in K order, writes bf16 and resets the counter to zero.

#include "common.h"
#include "kernels.h"

namespace glk {

template <int MT>
__global__ void __launch_bounds__(256) skinny_gemm_kernel(SkinnyArgs p) {
    constexpr int NR = 32 * MT;           // accumulator floats per lane: [c][mt][r]
    constexpr int PER_WAVE = NR / 4;      // floats per lane each wave finishes after the LDS sum
    extern __shared__ float red[];        // [4 waves][NR][64 lanes]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int strip = (int)blockIdx.x % p.strips;  // neighbouring workgroups read the same rows
    const int split = (int)blockIdx.x / p.strips;
    const int n0 = strip * kSkinnyStrip;
    const int kblocks = (p.K + kSkinnyKBlock - 1) / kSkinnyKBlock;
    const int kb0 = split * p.kb_per_split;
    const int kb1 = min(kblocks, kb0 + p.kb_per_split);

    const int g = lane >> 4;    // row group: k rows 8g .. 8g+7 of a k-block
    const int c16 = lane & 15;  // column octet: strip columns 8*c16 .. +7
    const bool col_ok = (n0 + 8 * c16) < p.N;
    const uint32_t b_lane = (uint32_t)(8 * g * p.ldb + 8 * c16) * 2u;
    const uint32_t ldb_bytes = (uint32_t)p.ldb * 2u;
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.A);
    uint32_t a_lane[MT];
    bool a_ok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + c16;
        a_ok[mt] = m < p.M;
        a_lane[mt] = (uint32_t)(m * p.lda + 8 * g) * 2u;
    }

    f32x4 acc[8][MT];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[c][mt] = f32x4{};

    auto load = [&](u32x4 (&b)[8], u32x4 (&a)[MT], int kb) {
        const bool kb_ok = kb < kb1;
        const int k0 = kb * kSkinnyKBlock;
        const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(p.B + (size_t)k0 * p.ldb + n0);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const bool ok = kb_ok && col_ok && (k0 + 8 * g + r) < p.K;
            b[r] = buf_load16(b_rsrc, ok ? b_lane + (uint32_t)r * ldb_bytes : kBufInvalid);
        }
        const bool ak = kb_ok && (k0 + 8 * g) < p.K;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            a[mt] = buf_load16(a_rsrc, (ak && a_ok[mt]) ? a_lane[mt] + (uint32_t)k0 * 2u : kBufInvalid);
    };

    auto compute = [&](const u32x4 (&b)[8], const u32x4 (&a)[MT]) {
        u32x4 t[8];
        transpose8x8_b16(b, t);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const bf16x8 x = __builtin_bit_cast(bf16x8, t[c]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[c][mt] = mfma16(x, __builtin_bit_cast(bf16x8, a[mt]), acc[c][mt]);
        }
    };

    {
        u32x4 b0[8], b1[8], a0[MT], a1[MT];
        int kb = kb0 + wave;
        load(b0, a0, kb);
        load(b1, a1, kb + 4);
        while (kb < kb1) {
            compute(b0, a0);
            load(b0, a0, kb + 8);
            if (kb + 4 >= kb1) break;
            compute(b1, a1);
            load(b1, a1, kb + 12);
            kb += 8;
        }
    }

    // ---- add the 4 waves' partials in wave order -------------------------------------------
    float* mine = red + (size_t)wave * NR * 64;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mine[((c * MT + mt) * 4 + r) * 64 + lane] = acc[c][mt][r];
    __syncthreads();
    // wave w finishes register indices [w * PER_WAVE, (w + 1) * PER_WAVE)
    float part[PER_WAVE];
#pragma unroll
    for (int t = 0; t < PER_WAVE; ++t) {
        const int ri = wave * PER_WAVE + t;
        float s = red[(0 * NR + ri) * 64 + lane];
        s += red[(1 * NR + ri) * 64 + lane];
        s += red[(2 * NR + ri) * 64 + lane];
        s += red[(3 * NR + ri) * 64 + lane];
        part[t] = s;
    }

    // ---- K slices meet in the workspace ------------------------------------------------------
    const int nsplit = min(p.splits, (kblocks + p.kb_per_split - 1) / p.kb_per_split);
    if (nsplit > 1) {
        __shared__ uint32_t last_flag;
        float* strip_ws = p.ws + (size_t)strip * p.splits * NR * 64;
        float* slot = strip_ws + (size_t)split * NR * 64;
#pragma unroll
        for (int t = 0; t < PER_WAVE; ++t) slot[(wave * PER_WAVE + t) * 64 + lane] = part[t];
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const uint32_t prev = atomicAdd(&p.counters[strip], 1u);
            last_flag = (prev == (uint32_t)(nsplit - 1)) ? 1u : 0u;
        }
        __syncthreads();
        if (!last_flag) return;
        __threadfence();
        if (tid == 0) p.counters[strip] = 0u;
#pragma unroll
        for (int t = 0; t < PER_WAVE; ++t) {
            const int ri = wave * PER_WAVE + t;
            float s = 0.f;
            for (int q = 0; q < nsplit; ++q)
                s += (q == split) ? part[t] : strip_ws[((size_t)q * NR + ri) * 64 + lane];
            part[t] = s;
        }
    }

    // ---- bf16 store ----------------------------------------------------------------------------
    // register index ri = (c * MT + mt) * 4 + r holds row m = 16 mt + (lane & 15) and strip
    // column 8 * (4 * (lane >> 4) + r) + c.
#pragma unroll
    for (int t = 0; t < PER_WAVE; ++t) {
        const int ri = wave * PER_WAVE + t;
        const int r = ri & 3, mt = (ri >> 2) % MT, c = (ri >> 2) / MT;
        const int m = 16 * mt + c16;
        const int n = n0 + 8 * (4 * g + r) + c;
        if (m < p.M && n < p.N) {
            const __bf16 h = (__bf16)part[t];
            p.C[(size_t)m * p.ldc + n] = __builtin_bit_cast(uint16_t, h);
        }
    }
}

hipError_t configure_skinny_kernels() {
    // the wave sum uses up to 128 KB of dynamic LDS (4 waves x 32 floats x 4 tiles x 64 lanes)
    const int max_lds = 4 * 32 * 4 * 64 * (int)sizeof(float);
    hipError_t e = hipSuccess;
    e = e != hipSuccess ? e : hipFuncSetAttribute((const void*)skinny_gemm_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    e = e != hipSuccess ? e : hipFuncSetAttribute((const void*)skinny_gemm_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    e = e != hipSuccess ? e : hipFuncSetAttribute((const void*)skinny_gemm_kernel<3>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    e = e != hipSuccess ? e : hipFuncSetAttribute((const void*)skinny_gemm_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    return e;
}

hipError_t launch_skinny_gemm(int mtiles, const SkinnyArgs& a, hipStream_t s) {
    const int grid = a.strips * a.splits;
    const size_t lds = (size_t)4 * 32 * mtiles * 64 * sizeof(float);
    switch (mtiles) {
        case 1: skinny_gemm_kernel<1><<<grid, 256, lds, s>>>(a); break;
        case 2: skinny_gemm_kernel<2><<<grid, 256, lds, s>>>(a); break;
        case 3: skinny_gemm_kernel<3><<<grid, 256, lds, s>>>(a); break;
        case 4: skinny_gemm_kernel<4><<<grid, 256, lds, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace glk
