// Decode product (1 <= M <= 64) on a packed bf16 weight, for gfx950: C = A * B with B (K x N)
// stored once in the order the matrix instructions consume it, float32 accumulation, bf16 out.
//
// The decode product is a stream of weight bytes read once for all M rows (spark-kernels post,
// "the decode kernel"; "The kernels that were there", "The GEMV"). A weight that does not change
// between calls can be stored in operand order, which removes the LDS staging and transposes the
// row-major skinny kernel needs:
//
// * Packed layout: column tile t (columns 16 t .. 16 t + 15) and k-step s (rows 32 s .. 32 s + 31)
//   form one 1 KB block at byte 1024 (t KS + s), KS = K / 32; lane l's 16 bytes are the 8 elements
//   B[32 s + 8 (l / 16) + j][16 t + l % 16], j = 0 .. 7: the first operand of
//   v_mfma_f32_16x16x32_bf16 for that lane, so one 1 KB load per wave is one operand.
// * pk_decode_kernel<MT, TN, D>: a workgroup takes TN column tiles and one of S pieces of the
//   k-steps; its 4 waves take contiguous quarters of the piece and run independently (no LDS, no
//   barrier in the loop), each keeping D k-steps of weight and activation loads in flight in
//   registers. For M <= 4 one tile per workgroup and 8 k-steps in flight (the activation loads
//   are nearly free there), above that 4 tiles sharing each activation load and 4 k-steps. The
//   activations are read straight from A (row-major, L2-resident): lane l reads row l % 16 of each
//   16-row tile, k = 32 s + 8 (l / 16) .. + 7. The waves' sums meet in LDS in wave order; with
//   S > 1 the pieces' float32 partials meet at device scope and the last arriver adds them in K
//   order and returns its counter to zero (as the skinny kernel does).

#include "common.h"
#include "packed.h"

namespace glk {

// one thread per (tile, k-step, lane): 8 strided elements of B into the lane's 16 bytes
__global__ void __launch_bounds__(256) pk_pack_kernel(const uint16_t* __restrict__ B, int K, int N, int ldb,
                                                      uint16_t* __restrict__ P) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int ks = K / 32;
    if (id >= (int64_t)(N / 16) * ks * 64) return;
    const int lane = (int)(id & 63);
    const int64_t ts = id >> 6;
    const int t = (int)(ts / ks), s = (int)(ts - (int64_t)t * ks);
    const int n = 16 * t + (lane & 15), k0 = 32 * s + 8 * (lane >> 4);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)B[(size_t)(k0 + 2 * j) * ldb + n] | ((uint32_t)B[(size_t)(k0 + 2 * j + 1) * ldb + n] << 16);
    *reinterpret_cast<u32x4*>(P + (size_t)512 * ts + 8 * lane) = u32x4{w[0], w[1], w[2], w[3]};
}

template <int MT, int TN>
struct PkStage {
    u32x4 w[TN];  // weight operand of each tile
    u32x4 a[MT];  // activation operand of each 16-row tile
};

template <int MT, int TN, int D>
__global__ void __launch_bounds__(256) pk_decode_kernel(PkArgs p) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wg = xcd_remap((int)blockIdx.x, (int)gridDim.x, p.nxcd);  // pieces of a group: one XCD
    const int group = wg / p.pieces, piece = wg - group * p.pieces;
    const int pb = (int)(((int64_t)p.ks * piece) / p.pieces);
    const int pe = (int)(((int64_t)p.ks * (piece + 1)) / p.pieces);
    const int wb = pb + ((pe - pb) * wave) / 4, we = pb + ((pe - pb) * (wave + 1)) / 4;

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.Bp), ra = make_rsrc(p.A);
    const int g16 = lane >> 4, i16 = lane & 15;
    bool tile_ok[TN];
    uint32_t w_base[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int tile = group * TN + t;
        tile_ok[t] = tile < p.tiles;
        w_base[t] = (uint32_t)tile * (uint32_t)p.ks * 1024u + 16u * lane;
    }
    bool row_ok[MT];
    uint32_t a_base[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + i16;
        row_ok[mt] = m < p.M;
        a_base[mt] = (uint32_t)m * (uint32_t)p.lda * 2u + 16u * g16;
    }
    // every call issues the same loads; out-of-range ones read zeros at an invalid offset
    auto load = [&](PkStage<MT, TN>& st, int s) {
        const bool sok = s < we;
#pragma unroll
        for (int t = 0; t < TN; ++t)
            st.w[t] = buf_load16(rw, sel_off(sok && tile_ok[t], w_base[t] + (uint32_t)s * 1024u));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            st.a[mt] = buf_load16(ra, sel_off(sok && row_ok[mt], a_base[mt] + (uint32_t)s * 64u));
    };

    f32x4 acc[TN][MT];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{};
    auto compute = [&](const PkStage<MT, TN>& st) {
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[t][mt] = mfma16(__builtin_bit_cast(bf16x8, st.w[t]), __builtin_bit_cast(bf16x8, st.a[mt]),
                                    acc[t][mt]);
    };

    PkStage<MT, TN> st[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load(st[j], wb + j);
    for (int s0 = wb; s0 < we; s0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            compute(st[j]);
            load(st[j], s0 + D + j);
        }
    }

    // ---- the waves' sums: LDS [wave][t][mt][lane], added in wave order ----------------------
    f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[((wave * TN + t) * MT + mt) * 64 + lane] = acc[t][mt];
    __syncthreads();
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
    const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws);
    const uint32_t slot = (uint32_t)NJ * 1024u;
    const uint32_t mine = ((uint32_t)group * (uint32_t)p.pieces + (uint32_t)piece) * slot;
#pragma unroll
    for (int q = 0; q < (NJ + 3) / 4; ++q) {
        const int j = 4 * q + wave;
        const bool ok = j < NJ && 16 * (j % MT) + i16 < p.M;
        buf_store16_dev(rws, sel_off(ok, mine + (uint32_t)j * 1024u + 16u * lane), f4_bits(sum[q]));
    }
    wait_all_memory();
    __syncthreads();
    volatile uint32_t& last_flag = *reinterpret_cast<volatile uint32_t*>(lds);
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
                v[u] = bits_f4(buf_load16_dev(rws, sel_off(ld, first + (uint32_t)pc * slot + (uint32_t)j * 1024u + 16u * lane)));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (b0 + u < p.pieces) x += (b0 + u == piece) ? sum[q] : v[u];
        }
        store_c(j, x);
    }
}

// tiles per workgroup for M rows (measured: one tile and 8 k-steps in flight up to M = 4, four
// tiles and 4 k-steps above)
int pk_decode_tiles_per_group(int64_t M) { return M <= 4 ? 1 : 4; }
int pk_decode_lds_bytes(int mtiles, int tpg) { return 4 * tpg * mtiles * 1024; }

template <int MT, int TN, int D>
static hipError_t pk_configure_one() {
    return hipFuncSetAttribute((const void*)pk_decode_kernel<MT, TN, D>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, pk_decode_lds_bytes(MT, TN));
}

hipError_t configure_pk_kernels() {
    hipError_t e = pk_configure_one<1, 1, 8>();
    if (e == hipSuccess) e = pk_configure_one<1, 4, 4>();
    if (e == hipSuccess) e = pk_configure_one<2, 4, 4>();
    if (e == hipSuccess) e = pk_configure_one<3, 4, 4>();
    if (e == hipSuccess) e = pk_configure_one<4, 4, 4>();
    return e;
}

hipError_t launch_pk_decode(int mtiles, int tpg, const PkArgs& a, int grid, hipStream_t s) {
    if (tpg == 1) {
        if (mtiles != 1) return hipErrorInvalidValue;
        pk_decode_kernel<1, 1, 8><<<grid, 256, (size_t)pk_decode_lds_bytes(1, 1), s>>>(a);
        return hipGetLastError();
    }
    if (tpg != 4) return hipErrorInvalidValue;
    const size_t lds = (size_t)pk_decode_lds_bytes(mtiles, 4);
    switch (mtiles) {
        case 1: pk_decode_kernel<1, 4, 4><<<grid, 256, lds, s>>>(a); break;
        case 2: pk_decode_kernel<2, 4, 4><<<grid, 256, lds, s>>>(a); break;
        case 3: pk_decode_kernel<3, 4, 4><<<grid, 256, lds, s>>>(a); break;
        case 4: pk_decode_kernel<4, 4, 4><<<grid, 256, lds, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pk_pack(const uint16_t* B, int K, int N, int ldb, uint16_t* P, hipStream_t s) {
    const int64_t threads = (int64_t)(N / 16) * (K / 32) * 64;
    if (threads == 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    pk_pack_kernel<<<(unsigned)blocks, 256, 0, s>>>(B, K, N, ldb, P);
    return hipGetLastError();
}

}  // namespace glk
