// Large-tile bf16 GEMM for gfx950: C = A * B, float32 accumulation on MFMA, bf16 output.
//
// Design (spark-kernels post, "the bf16 gemm": tiles staged HBM -> shared memory, more than one
// stage in flight, an XOR-swizzled shared tile instead of padding, the epilogue written from the
// accumulator registers; "stream-k proper": grouped tile order for cache reuse and a split-tile
// fixup summed in K order so every run gives the same bits):
//
// * One workgroup per (tile, K piece). Workgroup ids are first remapped so that each XCD's
//   round-robin share of the grid is a contiguous run of tiles, then walked in grouped order
//   (group_m tile rows at a time), so the tiles resident on one XCD share A rows and B columns
//   in that XCD's L2.
// * K advances in steps of 64. Each step's A tile (BM x 64) and B tile (64 x BN) are fetched
//   with 16-byte buffer loads into registers one step ahead of use, then written to one of two
//   LDS stages. Out-of-range rows, columns and k are fetched as zeros by pointing their offset
//   past the descriptor's range, so ragged edges need no branches.
// * Both operands sit in LDS K-contiguous ([row][k] for A, [col][k] for B), 128 bytes per row
//   split into eight 16-byte chunks stored at chunk ^ (row & 7). B arrives N-contiguous, so each
//   thread fetches an 8 x 8 block of B and transposes it in registers (v_perm) before its LDS
//   write; the MFMA operand of B then becomes one 16-byte LDS read per lane, like A's.
// * v_mfma_f32_32x32x16_bf16 with B as the first operand and A as the second, so each lane's
//   accumulator holds 4 consecutive columns of one row of C: the epilogue converts pairs with
//   v_cvt_pk_bf16_f32 (round to nearest even) and stores 8 bytes per lane.
// * Split pieces store float32 partials to a workspace slot, publish with a release fence and
//   an arrival counter; the last arriver adds all pieces of the tile in K order, writes bf16 and
//   returns the counter to zero for the next launch (no memset, no spin-waiting).

#include "common.h"
#include "kernels.h"

namespace glk {

template <int BM, int BN, int WM, int WN>
struct TileTraits {
    static constexpr int BK = 64;
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM;
    static constexpr int WTN = BN / WN;
    static constexpr int TM = WTM / 32;
    static constexpr int TN = WTN / 32;
    static constexpr int A_CH = BM * BK / 8 / NT;          // 16-byte A chunks per thread
    static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);   // 8x8 B blocks per stage
    static constexpr int B_BL = B_BLOCKS >= NT ? B_BLOCKS / NT : 1;  // per active thread
    static constexpr bool B_ALL = B_BLOCKS >= NT;          // every thread stages B
    static constexpr int STAGE = (BM + BN) * BK;           // bf16 elements per LDS stage
    static_assert(A_CH >= 1 && A_CH * NT * 8 == BM * BK, "A staging must divide evenly");
    static_assert(B_ALL ? (B_BL * NT == B_BLOCKS) : (NT % B_BLOCKS == 0), "B staging must divide evenly");
    static_assert(TM >= 1 && TN >= 1, "wave tile must hold whole 32x32 MFMA tiles");
};

template <int BM, int BN, int WM, int WN>
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                               amdgpu_waves_per_eu(1, 1)))
tile_gemm_kernel(TileArgs p) {
    using T = TileTraits<BM, BN, WM, WN>;
    constexpr int BK = T::BK, NT = T::NT, TM = T::TM, TN = T::TN;
    constexpr int A_CH = T::A_CH, B_BL = T::B_BL;
    constexpr bool B_ALL = T::B_ALL;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- which tile and K range ------------------------------------------------------------
    const int ntiles = p.tiles_m * p.tiles_n;
    const int nunits = (p.sched == kSchedSplitK) ? ntiles * p.splits : ntiles;
    const int unit = xcd_remap((int)blockIdx.x, nunits, p.nxcd);
    int tile = unit, piece = 0;
    if (p.sched == kSchedSplitK) {
        tile = unit / p.splits;
        piece = unit % p.splits;
    }
    const int per_group = p.group_m * p.tiles_n;
    const int g = tile / per_group;
    const int first_m = g * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int in_g = tile - g * per_group;
    const int tm = first_m + in_g % gm;
    const int tn = in_g / gm;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt_total = (p.K + BK - 1) / BK;
    int kt_begin = 0, kt_end = kt_total;
    if (p.sched == kSchedSplitK) {
        kt_begin = piece * p.kt_per_split;
        kt_end = min(kt_total, kt_begin + p.kt_per_split);
    }

    // ---- per-thread load coordinates ---------------------------------------------------------
    // A: chunk i covers row a_m[i] of the tile, k-chunk a_kc (same for all i).
    const int a_kc = tid & 7;
    uint32_t a_off[A_CH];
    bool a_row_ok[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int m = i * (NT / 8) + (tid >> 3);
        a_off[i] = (uint32_t)(m * p.lda + a_kc * 8) * 2u;
        a_row_ok[i] = (m0 + m) < p.M;
    }
    // B: block j covers k rows 8*b_kb .. +7 and columns 8*b_nb[j] .. +7 of the tile.
    const int b_kb = tid & 7;
    uint32_t b_off[B_BL];
    bool b_col_ok[B_BL];
#pragma unroll
    for (int j = 0; j < B_BL; ++j) {
        const int nb = j * (NT / 8) + (tid >> 3);
        b_off[j] = (uint32_t)(8 * b_kb * p.ldb + 8 * nb) * 2u;
        b_col_ok[j] = (n0 + 8 * nb) < p.N;
    }
    const uint32_t ldb_bytes = (uint32_t)p.ldb * 2u;
    const bool b_active = B_ALL || tid < T::B_BLOCKS;  // threads that stage B

    u32x4 ra[A_CH];
    u32x4 rb[B_BL][8];

    auto load_stage = [&](int kt) {
        const int k0 = kt * BK;
        const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(p.A + (size_t)m0 * p.lda + k0);
        const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(p.B + (size_t)k0 * p.ldb + n0);
        const bool a_k_ok = (k0 + a_kc * 8) < p.K;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            ra[i] = buf_load16(ra_rsrc, (a_row_ok[i] && a_k_ok) ? a_off[i] : kBufInvalid);
        if (!b_active) return;
#pragma unroll
        for (int j = 0; j < B_BL; ++j) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const bool ok = b_col_ok[j] && (k0 + 8 * b_kb + r) < p.K;
                rb[j][r] = buf_load16(rb_rsrc, ok ? b_off[j] + (uint32_t)r * ldb_bytes : kBufInvalid);
            }
        }
    };

    auto store_stage = [&](int stage) {
        uint16_t* sa = lds + stage * T::STAGE;
        uint16_t* sb = sa + BM * BK;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int m = i * (NT / 8) + (tid >> 3);
            *reinterpret_cast<u32x4*>(sa + m * BK + ((a_kc ^ (m & 7)) * 8)) = ra[i];
        }
        if (!b_active) return;
#pragma unroll
        for (int j = 0; j < B_BL; ++j) {
            const int nb = j * (NT / 8) + (tid >> 3);
            u32x4 tcol[8];
            transpose8x8_b16(rb[j], tcol);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int n = 8 * nb + c;
                *reinterpret_cast<u32x4*>(sb + n * BK + ((b_kb ^ c) * 8)) = tcol[c];
            }
        }
    };

    f32x16 acc[TN][TM];
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) acc[ni][mi] = f32x16{};

    // fragment read coordinates: lane reads row (lane & 31) of a 32-row block, k-chunk
    // 2*kk + (lane >> 5); the swizzle term is (row & 7) == (lane & 7).
    const int fr_row = lane & 31;
    const int fr_half = lane >> 5;
    const int fr_sw = lane & 7;

    if (kt_begin < kt_end) {
        load_stage(kt_begin);
        store_stage(0);
        __syncthreads();
        for (int kt = kt_begin; kt < kt_end; ++kt) {
            const int cur = (kt - kt_begin) & 1;
            const bool more = (kt + 1) < kt_end;
            if (more) load_stage(kt + 1);
            const uint16_t* sa = lds + cur * T::STAGE;
            const uint16_t* sb = sa + BM * BK;
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int kc = 2 * kk + fr_half;
                bf16x8 af[TM], bfr[TN];
#pragma unroll
                for (int mi = 0; mi < TM; ++mi) {
                    const int m = wm * T::WTM + mi * 32 + fr_row;
                    af[mi] = *reinterpret_cast<const bf16x8*>(sa + m * BK + ((kc ^ fr_sw) * 8));
                }
#pragma unroll
                for (int ni = 0; ni < TN; ++ni) {
                    const int n = wn * T::WTN + ni * 32 + fr_row;
                    bfr[ni] = *reinterpret_cast<const bf16x8*>(sb + n * BK + ((kc ^ fr_sw) * 8));
                }
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int mi = 0; mi < TM; ++mi) acc[ni][mi] = mfma32(bfr[ni], af[mi], acc[ni][mi]);
            }
            if (more) store_stage(cur ^ 1);
            __syncthreads();
        }
    }

    // ---- split fixup ---------------------------------------------------------------------------
    // Lane layout of acc[ni][mi][r]: row m = wm*WTM + mi*32 + (lane & 31),
    // column n = wn*WTN + ni*32 + 8*(r >> 2) + 4*(lane >> 5) + (r & 3).
    if (p.sched == kSchedSplitK && p.splits > 1) {
        const int npieces = min(p.splits, (kt_total + p.kt_per_split - 1) / p.kt_per_split);
        if (npieces > 1) {
            __shared__ uint32_t last_flag;
            // slot layout (floats, fragment order): [wave][ni][mi][r/4][lane][4]
            const __amdgpu_buffer_rsrc_t ws = make_rsrc(p.ws + (size_t)tile * p.splits * (BM * BN));
            const uint32_t slot_bytes = (uint32_t)(BM * BN) * 4u;
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t off = (uint32_t)(((((wave * TN + ni) * TM + mi) * 4 + q) * 256 + lane * 4) * 4);
                        f32x4 v = {acc[ni][mi][4 * q], acc[ni][mi][4 * q + 1], acc[ni][mi][4 * q + 2],
                                   acc[ni][mi][4 * q + 3]};
                        buf_store16_dev(ws, (uint32_t)piece * slot_bytes + off, f4_bits(v));
                    }
            wait_all_memory();
            __syncthreads();
            if (tid == 0)
                last_flag = (counter_arrive(&p.counters[tile]) == (uint32_t)(npieces - 1)) ? 1u : 0u;
            __syncthreads();
            if (!last_flag) return;
            if (tid == 0) counter_reset(&p.counters[tile]);
            // sum the pieces in K order: piece 0 first
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t off = (uint32_t)(((((wave * TN + ni) * TM + mi) * 4 + q) * 256 + lane * 4) * 4);
                        f32x4 s = {0.f, 0.f, 0.f, 0.f};
                        for (int pc = 0; pc < npieces; ++pc) {
                            f32x4 v;
                            if (pc == piece)
                                v = f32x4{acc[ni][mi][4 * q], acc[ni][mi][4 * q + 1], acc[ni][mi][4 * q + 2],
                                          acc[ni][mi][4 * q + 3]};
                            else
                                v = bits_f4(buf_load16_dev(ws, (uint32_t)pc * slot_bytes + off));
                            s += v;
                        }
                        acc[ni][mi][4 * q] = s[0];
                        acc[ni][mi][4 * q + 1] = s[1];
                        acc[ni][mi][4 * q + 2] = s[2];
                        acc[ni][mi][4 * q + 3] = s[3];
                    }
        }
    }

    // ---- epilogue: bf16 (round to nearest even), 8-byte stores -------------------------------
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + (size_t)m0 * p.ldc + n0);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
        const int m = wm * T::WTM + mi * 32 + fr_row;
        const bool m_ok = (m0 + m) < p.M;
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = wn * T::WTN + ni * 32 + 8 * q + 4 * fr_half;
                const bool ok = m_ok && (n0 + n) < p.N;
                u32x2 v = {pack_bf16x2(acc[ni][mi][4 * q], acc[ni][mi][4 * q + 1]),
                           pack_bf16x2(acc[ni][mi][4 * q + 2], acc[ni][mi][4 * q + 3])};
                buf_store8(rc, ok ? (uint32_t)(m * p.ldc + n) * 2u : kBufInvalid, v);
            }
        }
    }
}

TileShape tile_shape(int cfg) {
    switch (cfg) {
        case kTile256x256w4: return {256, 256, 64, 256};
        case kTile256x256w8: return {256, 256, 64, 512};
        case kTile128x128w4: return {128, 128, 64, 256};
        default: return {0, 0, 0, 0};
    }
}

hipError_t launch_tile_gemm(int cfg, const TileArgs& a, int grid, hipStream_t s) {
    const TileShape t = tile_shape(cfg);
    switch (cfg) {
        case kTile256x256w4:
            tile_gemm_kernel<256, 256, 2, 2><<<grid, t.threads, 0, s>>>(a);
            break;
        case kTile256x256w8:
            tile_gemm_kernel<256, 256, 2, 4><<<grid, t.threads, 0, s>>>(a);
            break;
        case kTile128x128w4:
            tile_gemm_kernel<128, 128, 2, 2><<<grid, t.threads, 0, s>>>(a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace glk
