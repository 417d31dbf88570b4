// Block-scaled (MX) decode product for gfx950, and the conversions that feed it.
//
// C (M x N, bf16) = deq(Aq) * deq(W)^T with the activations Aq (M x K) in MXFP8 and the weights W
// (N x K, the nn.Linear layout) in MXFP4: E4M3 and E2M1 element codes, one E8M0 scale 2^(e - 127)
// per 32 consecutive k (OCP Microscaling Formats v1.0). The weights are the bytes that bound
// decode; in MXFP4 they take 0.53 bytes per element instead of 2 (spark-kernels post, "the
// decode kernel": the decode GEMM is a weight stream; the "Benchmarks" page of gemm3 measures
// block-scaled GEMMs on pre-quantized operands, "Implementations").
//
// * mx_quant_kernel: four lanes per 32-element block of a bf16 row. The shared exponent is
//   floor(log2(max |v|)) - emax of the element format (exact, from the bf16 exponent bits), clamped
//   to [-127, 127]; each element is v * 2^-exponent (exact) rounded to the element format,
//   nearest with ties to even, saturating at its largest magnitude; an all-zero block gets scale
//   byte 0. Activations (E4M3) are written row-major with their scales; weights (E2M1) are written
//   straight into the packed layout the product reads.
// * Packed weights: column tile t (16 rows n of W) and k-step s (128 k) form one 1 KB block at
//   byte 1024 (t KS + s), KS = K / 128, in which lane l's 16 bytes are the 32 codes of row
//   16 t + l % 16, k = 128 s + 32 (l / 16) + j, two per byte, even j low: exactly the operand a
//   lane hands to v_mfma_scale_f32_16x16x128_f8f6f4, so one 1 KB load per wave needs no shuffle.
//   The scales of four k-steps of a tile share 256 bytes, lane l owning byte 4 l + s % 4.
// * mx_decode_kernel: a workgroup takes TN = 3 or 4 column tiles and one of S pieces of their k-steps;
//   its 4 waves take contiguous quarters of the piece and run independently: no LDS and no
//   barrier in the loop. Each wave keeps D = 2 k-steps of weights, activations and scales in flight
//   in registers (the loads of step s + D go out as step s is consumed), and issues one scaled
//   MFMA per tile and 16-row tile of M per k-step, with the weights as the first operand (so a
//   lane's accumulator holds 4 consecutive columns of one row of C).
// * Operand layouts of v_mfma_scale_f32_16x16x128_f8f6f4 (measured with impulse inputs): lane l
//   (group g = l / 16) holds row or column l % 16. An FP4 operand holds k = 32 g .. 32 g + 31 in
//   its 16 bytes, even k in the low nibble; an FP8 operand holds k = 16 g .. 16 g + 15 in bytes
//   0 .. 15 and k = 64 + 16 g .. 64 + 16 g + 15 in bytes 16 .. 31. The scale byte a lane of group g
//   supplies applies to k-block g (k = 32 g .. 32 g + 31) of its row or column, whichever lanes
//   hold that block's elements. The activations are loaded to match. The waves' sums meet in LDS
//   (added in wave order); with S > 1 the pieces' float32 partials meet at device scope and the
//   last arriver adds them in K order and writes bf16, returning its counter to zero.

#include "common.h"
#include "mx.h"

namespace glk {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---- element conversion ------------------------------------------------------------------------

// x (a bf16 value divided by its block scale, exact in float32) to an element code with EB
// exponent bits, MB mantissa bits and bias BIAS: nearest, ties to even, saturating at VMAX;
// the sign bit is x's (so -0 and negatives that round to zero keep it).
template <int EB, int MB, int BIAS>
__device__ __forceinline__ uint32_t mx_encode(float x, float vmax) {
    const uint32_t sign = __builtin_bit_cast(uint32_t, x) >> 31;
    const float a = fabsf(x);
    float mag = vmax;
    if (!(a >= vmax)) {
        int e = __builtin_amdgcn_frexp_expf(a) - 1;  // floor(log2 a) for a > 0
        e = e < 1 - BIAS ? 1 - BIAS : e;              // subnormals share the smallest quantum
        const float n = __builtin_rintf(ldexpf(a, MB - e));
        mag = fminf(ldexpf(n, e - MB), vmax);
    }
    uint32_t code = 0;
    if (mag != 0.0f) {
        const int e2 = __builtin_amdgcn_frexp_expf(mag) - 1;
        if (e2 < 1 - BIAS)
            code = (uint32_t)ldexpf(mag, MB - (1 - BIAS));
        else
            code = ((uint32_t)(e2 + BIAS) << MB) | ((uint32_t)ldexpf(mag, MB - e2) - (1u << MB));
    }
    return (sign << (EB + MB)) | code;
}

// floor(log2 |v|) of a nonzero bf16 magnitude (16-bit pattern without sign)
__device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
    const int e = (int)(mag >> 7);
    if (e > 0) return e - 127;
    return (31 - __builtin_clz(mag & 0x7Fu)) - 133;  // subnormal: m * 2^-133
}

// Eight elements (one lane's quarter of a 32-element block) to codes; the four lanes of a block
// are consecutive lanes of one wave and reduce the block maximum by shuffles, so all four must
// run this together. Returns the block's scale byte.
template <bool FP4>
__device__ __forceinline__ uint8_t mx_quant8(const u32x4& v, uint32_t (&codes)[8]) {
    constexpr int EMAX = FP4 ? 2 : 8;
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = v[j] & 0x7FFFu, hi = (v[j] >> 16) & 0x7FFFu;
        amax = lo > amax ? lo : amax;
        amax = hi > amax ? hi : amax;
    }
#pragma unroll
    for (int d = 1; d < 4; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)amax, d, 4);
        amax = o > amax ? o : amax;
    }
    int se = -127;
    if (amax != 0) {
        se = bf16_floor_log2(amax) - EMAX;
        se = se < -127 ? -127 : (se > 127 ? 127 : se);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = ldexpf(bf16_lo(v[j]), -se), hi = ldexpf(bf16_hi(v[j]), -se);
        if (FP4) {
            codes[2 * j] = mx_encode<2, 1, 1>(lo, 6.0f);
            codes[2 * j + 1] = mx_encode<2, 1, 1>(hi, 6.0f);
        } else {
            codes[2 * j] = mx_encode<4, 3, 7>(lo, 448.0f);
            codes[2 * j + 1] = mx_encode<4, 3, 7>(hi, 448.0f);
        }
    }
    return (uint8_t)(se + 127);
}

// four consecutive lanes per (row, 32-element block), 8 elements each; the block maximum is
// reduced across the four lanes. FP4 = false: E4M3 codes row-major into Q (ldq bytes per row) and
// scales into S (lds bytes per row). FP4 = true: E2M1 codes and scales into the packed weight
// layout (rows = N, a multiple of 16; cols = K, a multiple of 128); blocks past K (up to the next
// multiple of four k-steps) get the zero scale bytes of the missing k-steps.
template <bool FP4>
__global__ void __launch_bounds__(256) mx_quant_kernel(const uint16_t* __restrict__ X, int rows,
                                                       int cols, int ldx, uint8_t* __restrict__ Q,
                                                       int ldq, uint8_t* __restrict__ S, int lds,
                                                       int blocks_per_row) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= (int64_t)rows * blocks_per_row * 4) return;  // whole groups of four lanes
    const int64_t blk = id >> 2;
    const int qtr = (int)(id & 3);
    const int r = (int)(blk / blocks_per_row), b = (int)(blk - (int64_t)r * blocks_per_row);
    const int ks = cols / 128, kq = (ks + 3) / 4;
    // packed position of (row, block): tile t, lane, k-step s
    const int t = r >> 4, s = b >> 2, lane = 16 * (b & 3) + (r & 15);
    if (b * 32 >= cols) {  // FP4 only: a k-step past K inside the last group of four
        if (qtr == 0) S[(size_t)256 * ((size_t)t * kq + (s >> 2)) + 4 * lane + (s & 3)] = 0;
        return;
    }
    const u32x4 v = *reinterpret_cast<const u32x4*>(X + (size_t)r * ldx + 32 * b + 8 * qtr);
    uint32_t codes[8];
    const uint8_t scale = mx_quant8<FP4>(v, codes);
    if (FP4) {
        uint32_t word = 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) word |= codes[n] << (4 * n);
        *reinterpret_cast<uint32_t*>(Q + (size_t)1024 * ((size_t)t * ks + s) + 16 * lane + 4 * qtr) = word;
        if (qtr == 0) S[(size_t)256 * ((size_t)t * kq + (s >> 2)) + 4 * lane + (s & 3)] = scale;
    } else {
        const u32x2 out = {codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24),
                           codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24)};
        *reinterpret_cast<u32x2*>(Q + (size_t)r * ldq + 32 * b + 8 * qtr) = out;
        if (qtr == 0) S[(size_t)r * lds + b] = scale;
    }
}

// ---- the product ---------------------------------------------------------------------------------

// k-steps in flight per wave (measured: 2 beat 3, 4 and 6 on every decode shape)
constexpr int kMxD = 2;
constexpr int kMxFusedLdsMax = 160 * 1024;  // the fused form's activation rows + reduction

// TN column tiles (16 columns each) per workgroup: 3 or 4, chosen by the planner
template <int MT, int TN>
struct MxStage {
    u32x4 w[TN];          // weight codes, lane's 16 bytes of each tile's block
    uint32_t ws[TN];      // weight scale byte
    u32x4 a[MT][2];       // activation codes of each 16-row tile: k 16 g .. +15 and 64 + 16 g .. +15
    uint32_t as[MT];      // activation scale byte
};

// FUSED (M <= 2, MT = 1): the workgroup converts the bf16 activations of its K piece to MXFP8 in
// LDS itself (while its first weight loads are in flight) and reads the activation operands from
// there: the product from bf16 activations in one launch, with the same bits as the two-launch path.
template <int MT, bool FUSED, int TN>
__global__ void __launch_bounds__(256) mx_decode_kernel(MxArgs p) {
    constexpr int D = kMxD;
    static_assert(!FUSED || MT == 1, "the fused conversion serves one 16-row tile");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // logical workgroup: nxcd > 1 keeps a group's pieces on one XCD; the planner passes 1 (the
    // hardware's round-robin order, measured faster)
    const int wg = xcd_remap((int)blockIdx.x, (int)gridDim.x, p.nxcd);
    const int group = wg / p.pieces, piece = wg - group * p.pieces;
    // k-steps of the piece, then of this wave (contiguous quarters)
    const int pb = (int)(((int64_t)p.ks * piece) / p.pieces);
    const int pe = (int)(((int64_t)p.ks * (piece + 1)) / p.pieces);
    const int wb = pb + ((pe - pb) * wave) / 4, we = pb + ((pe - pb) * (wave + 1)) / 4;

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.Wp), rws = make_rsrc(p.Sp);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.Aq), ras = make_rsrc(p.As);
    const int g16 = lane >> 4, i16 = lane & 15;
    bool tile_ok[TN];
    uint32_t w_base[TN], ws_base[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int tile = group * TN + t;
        tile_ok[t] = tile < p.tiles;
        w_base[t] = (uint32_t)tile * (uint32_t)p.ks * 1024u + 16u * lane;
        ws_base[t] = (uint32_t)tile * (uint32_t)p.kq * 256u + 4u * lane;
    }
    bool row_ok[MT];
    uint32_t a_base[MT], as_base[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + i16;
        row_ok[mt] = m < p.M;
        a_base[mt] = (uint32_t)m * (uint32_t)p.ldaq + 16u * g16;
        as_base[mt] = (uint32_t)m * (uint32_t)p.ldas + g16;
    }
    // every call issues the same loads, out-of-range ones at an invalid offset (they read zeros:
    // code 0 with scale byte 0 adds nothing)
    auto load = [&](MxStage<MT, TN>& st, int s) {
        const bool sok = s < we;
        if constexpr (FUSED) {  // activations come from LDS at compute time
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                const bool ok = sok && tile_ok[t];
                st.w[t] = buf_load16(rw, sel_off(ok, w_base[t] + (uint32_t)s * 1024u));
                st.ws[t] = __builtin_amdgcn_raw_buffer_load_b8(
                    rws, sel_off(ok, ws_base[t] + (uint32_t)(s >> 2) * 256u + (uint32_t)(s & 3)), 0, 0);
            }
            return;
        }
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const bool ok = sok && tile_ok[t];
            st.w[t] = buf_load16(rw, sel_off(ok, w_base[t] + (uint32_t)s * 1024u));
            st.ws[t] = __builtin_amdgcn_raw_buffer_load_b8(
                rws, sel_off(ok, ws_base[t] + (uint32_t)(s >> 2) * 256u + (uint32_t)(s & 3)), 0, 0);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const bool ok = sok && row_ok[mt];
            const uint32_t off = a_base[mt] + (uint32_t)s * 128u;
            st.a[mt][0] = buf_load16(ra, sel_off(ok, off));
            st.a[mt][1] = buf_load16(ra, sel_off(ok, off + 64u));
            st.as[mt] = __builtin_amdgcn_raw_buffer_load_b8(ras, sel_off(ok, as_base[mt] + 4u * (uint32_t)s), 0, 0);
        }
    };

    f32x4 acc[TN][MT];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{};

    // fused: activation codes [row][k - 128 pb] at lds, scales [row][block - 4 pb] at lds + 2 kpb
    const uint8_t* aq_lds = reinterpret_cast<const uint8_t*>(lds);
    const uint8_t* as_lds = aq_lds + 2 * p.kpb;
    auto compute = [&](MxStage<MT, TN>& st, int s) {
        if constexpr (FUSED) {
            const int m = i16, ls = s - pb;
            u32x4 x0 = u32x4{0u, 0u, 0u, 0u}, x1 = x0;
            uint32_t sc = 0;
            if (m < p.M && s < we) {
                x0 = *reinterpret_cast<const u32x4*>(aq_lds + m * p.kpb + 128 * ls + 16 * g16);
                x1 = *reinterpret_cast<const u32x4*>(aq_lds + m * p.kpb + 128 * ls + 64 + 16 * g16);
                sc = as_lds[m * (p.kpb / 32) + 4 * ls + g16];
            }
            st.a[0][0] = x0;
            st.a[0][1] = x1;
            st.as[0] = sc;
        }
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const i32x8 wv = {(int)st.w[t][0], (int)st.w[t][1], (int)st.w[t][2], (int)st.w[t][3], 0, 0, 0, 0};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const i32x8 av = {(int)st.a[mt][0][0], (int)st.a[mt][0][1], (int)st.a[mt][0][2], (int)st.a[mt][0][3],
                                  (int)st.a[mt][1][0], (int)st.a[mt][1][1], (int)st.a[mt][1][2], (int)st.a[mt][1][3]};
                // first operand: weights, E2M1 (format 4); second: activations, E4M3 (format 0)
                acc[t][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    wv, av, acc[t][mt], 4, 0, 0, (int)st.ws[t], 0, (int)st.as[mt]);
            }
        }
    };

    MxStage<MT, TN> st[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load(st[j], wb + j);
    if constexpr (FUSED) {
        // convert rows 0 .. M-1 of A over the piece's k-steps [pb, pe) into LDS: four lanes per
        // 32-element block (consecutive tasks of one wave), 8 elements each
        const int nb = (pe - pb) * 4;  // blocks per row in the piece
        const int total = p.M * nb * 4;
        for (int task = tid; task < total; task += 256) {
            const int m = task / (nb * 4), rem = task - m * (nb * 4);
            const int b = rem >> 2, q = rem & 3;
            const u32x4 v = *reinterpret_cast<const u32x4*>(p.A16 + (size_t)m * p.lda16 + 128 * pb + 32 * b + 8 * q);
            uint32_t codes[8];
            const uint8_t scale = mx_quant8<false>(v, codes);
            uint8_t* qd = reinterpret_cast<uint8_t*>(lds) + m * p.kpb + 32 * b + 8 * q;
            *reinterpret_cast<u32x2*>(qd) = u32x2{codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24),
                                                  codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24)};
            if (q == 0) reinterpret_cast<uint8_t*>(lds)[2 * p.kpb + m * (p.kpb / 32) + b] = scale;
        }
        __syncthreads();
    }
    for (int s0 = wb; s0 < we; s0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            compute(st[j], s0 + j);
            load(st[j], s0 + D + j);
        }
    }

    // ---- the waves' sums: LDS [wave][t][mt][lane], added in wave order ----------------------
    f32x4* red = reinterpret_cast<f32x4*>(lds + (FUSED ? p.red_off : 0));
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[((wave * TN + t) * MT + mt) * 64 + lane] = acc[t][mt];
    __syncthreads();
    // wave w finishes the (t, mt) pairs j = w, w + 4, ...
    constexpr int NJ = TN * MT;
    f32x4 sum[(NJ + 3) / 4];
#pragma unroll
    for (int q = 0; q < (NJ + 3) / 4; ++q) {
        const int j = 4 * q + wave;
        f32x4 x = f32x4{};
        if (j < NJ) {
#pragma unroll
            for (int w = 0; w < 4; ++w) x += red[(w * NJ + j) * 64 + lane];
        }
        sum[q] = x;
    }
    auto store_c = [&](int j, const f32x4& v) {
        const int t = j / MT, mt = j - (j / MT) * MT;
        const int m = 16 * mt + i16, tile = group * TN + t;
        if (m < p.M && tile < p.tiles) {
            const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2*>(p.C + (size_t)m * p.ldc + 16 * tile + 4 * g16) = o;
        }
    };
    if (p.pieces == 1) {
#pragma unroll
        for (int q = 0; q < (NJ + 3) / 4; ++q)
            if (4 * q + wave < NJ) store_c(4 * q + wave, sum[q]);
        return;
    }
    // ---- pieces meet at device scope; the last arriver adds them in K order ---------------------
    // slot of (group, piece): NJ x 64 lanes x 16 bytes
    const __amdgpu_buffer_rsrc_t rws_ws = make_rsrc(p.ws);
    const uint32_t slot = (uint32_t)NJ * 1024u;
    const uint32_t mine = ((uint32_t)group * (uint32_t)p.pieces + (uint32_t)piece) * slot;
#pragma unroll
    for (int q = 0; q < (NJ + 3) / 4; ++q) {
        const int j = 4 * q + wave;
        const bool ok = j < NJ && 16 * (j % MT) + i16 < p.M;
        buf_store16_dev(rws_ws, sel_off(ok, mine + (uint32_t)j * 1024u + 16u * lane), f4_bits(sum[q]));
    }
    wait_all_memory();
    __syncthreads();
    volatile uint32_t& last_flag = *reinterpret_cast<volatile uint32_t*>(lds + (FUSED ? p.red_off : 0));
    if (tid == 0)
        last_flag = (counter_arrive(&p.counters[group]) == (uint32_t)(p.pieces - 1)) ? 1u : 0u;
    __syncthreads();
    if (!last_flag) return;
    if (tid == 0) counter_reset(&p.counters[group]);
    const uint32_t first = (uint32_t)group * (uint32_t)p.pieces * slot;
#pragma unroll
    for (int q = 0; q < (NJ + 3) / 4; ++q) {
        const int j = 4 * q + wave;
        if (j >= NJ) continue;
        const bool ok = 16 * (j % MT) + i16 < p.M;
        // in K order, four pieces' loads in flight before their adds
        f32x4 x = f32x4{};
        for (int b0 = 0; b0 < p.pieces; b0 += 4) {
            f32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pc = b0 + u;
                const bool ld = ok && pc < p.pieces && pc != piece;
                v[u] = bits_f4(buf_load16_dev(rws_ws, sel_off(ld, first + (uint32_t)pc * slot + (uint32_t)j * 1024u + 16u * lane)));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (b0 + u < p.pieces) x += (b0 + u == piece) ? sum[q] : v[u];
        }
        store_c(j, x);
    }
}

template <int MT, bool FUSED, int TN>
static hipError_t mx_configure_one() {
    return hipFuncSetAttribute((const void*)mx_decode_kernel<MT, FUSED, TN>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               FUSED ? kMxFusedLdsMax : mx_decode_lds_bytes(MT, TN));
}

int mx_decode_lds_bytes(int mtiles, int tn) { return 4 * tn * mtiles * 1024; }

template <int TN>
static hipError_t mx_configure_tn() {
    hipError_t e = mx_configure_one<1, false, TN>();
    if (e == hipSuccess) e = mx_configure_one<2, false, TN>();
    if (e == hipSuccess) e = mx_configure_one<3, false, TN>();
    if (e == hipSuccess) e = mx_configure_one<4, false, TN>();
    if (e == hipSuccess) e = mx_configure_one<1, true, TN>();
    return e;
}

hipError_t configure_mx_kernels() {
    hipError_t e = mx_configure_tn<3>();
    if (e == hipSuccess) e = mx_configure_tn<4>();
    return e;
}

template <int TN>
static hipError_t launch_mx_tn(int mtiles, const MxArgs& a, int grid, hipStream_t s) {
    const size_t lds = (size_t)mx_decode_lds_bytes(mtiles, TN);
    switch (mtiles) {
        case 1: mx_decode_kernel<1, false, TN><<<grid, 256, lds, s>>>(a); break;
        case 2: mx_decode_kernel<2, false, TN><<<grid, 256, lds, s>>>(a); break;
        case 3: mx_decode_kernel<3, false, TN><<<grid, 256, lds, s>>>(a); break;
        case 4: mx_decode_kernel<4, false, TN><<<grid, 256, lds, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mx_decode(int mtiles, int tn, const MxArgs& a, int grid, hipStream_t s) {
    if (tn == 3) return launch_mx_tn<3>(mtiles, a, grid, s);
    if (tn == 4) return launch_mx_tn<4>(mtiles, a, grid, s);
    return hipErrorInvalidValue;
}

// LDS of the fused form for pieces of at most `piece_ks` k-steps, or -1 if it does not fit; sets
// the args' activation row stride and reduction offset
int mx_fused_layout(int piece_ks, int tn, MxArgs& a) {
    const int kpb = piece_ks * 128;
    const int red_off = (2 * kpb + 2 * (kpb / 32) + 15) / 16 * 16;
    const int bytes = red_off + mx_decode_lds_bytes(1, tn);
    if (bytes > kMxFusedLdsMax) return -1;
    a.kpb = kpb;
    a.red_off = red_off;
    return bytes;
}

hipError_t launch_mx_decode_fused(int tn, const MxArgs& a, int grid, int lds_bytes, hipStream_t s) {
    if (tn == 3)
        mx_decode_kernel<1, true, 3><<<grid, 256, (size_t)lds_bytes, s>>>(a);
    else if (tn == 4)
        mx_decode_kernel<1, true, 4><<<grid, 256, (size_t)lds_bytes, s>>>(a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mx_quant(bool fp4, const uint16_t* X, int rows, int cols, int ldx, uint8_t* Q, int ldq,
                           uint8_t* S, int lds, hipStream_t s) {
    // FP4 (packed weights): blocks up to the next multiple of four k-steps, for the zero scales
    const int bpr = fp4 ? ((cols / 128 + 3) / 4) * 16 : cols / 32;
    const int64_t threads = (int64_t)rows * bpr * 4;
    if (threads == 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (fp4)
        mx_quant_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(X, rows, cols, ldx, Q, ldq, S, lds, bpr);
    else
        mx_quant_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(X, rows, cols, ldx, Q, ldq, S, lds, bpr);
    return hipGetLastError();
}

}  // namespace glk
