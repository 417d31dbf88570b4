// Large-tile bf16 GEMM for gfx950: C = A * B, float32 accumulation on MFMA, bf16 output.
//
// Design (spark-kernels post, "the bf16 gemm": tiles staged HBM -> shared memory with several
// stages in flight, an XOR-swizzled shared tile instead of padding, the epilogue written from the
// accumulator registers; "the copies were the problem": take the copies out of the compute
// waves' instruction stream and avoid a full barrier's cost per k step; "stream-k proper":
// grouped tile order for cache reuse and a split-tile fixup summed in K order so every run gives
// the same bits):
//
// * One workgroup per (tile, K piece). Workgroup ids are first remapped so that each XCD's
//   round-robin share of the grid is a contiguous run of tiles, then walked in grouped order
//   (group_m tile rows at a time), so the tiles resident on one XCD share A rows and B columns
//   in that XCD's L2.
// * K advances in steps of BK = 32. A and B are copied HBM -> LDS by direct-to-LDS buffer loads
//   (1 KB per wave instruction, no registers) into two rings: B in 3 stages of 32 x BN, A in 3
//   stages of BM x 64 so that every A row the loads touch is one whole 128-byte
//   line (32-k stages would fetch half lines, which costs the address unit about a third more per
//   byte). Each step every wave issues the same loads: half an A stage and one B stage, several
//   steps ahead of use; one barrier per step, with no memory fence, so later loads stay in flight.
// * MFMA operands are double-buffered in registers: while the matrix cores run step i from one
//   register set, the LDS reads for step i + 1 fill the other, so the MFMA stream never waits on
//   an LDS read; each barrier therefore guards the data of the step after the next.
// * A sits in LDS K-contiguous (128-byte rows, 16-byte chunks stored at chunk ^ ((row >> 1) & 7))
//   and is read with ds_read_b128. B stays row-major (N-contiguous, 32-byte column groups stored
//   at group ^ s(k), s(k) = (k & 3) | ((k >> 1) & 4)); its MFMA operand, 8 consecutive k for one
//   column, comes from ds_read_b64_tr_b16, which transposes 4 x 16 blocks on the way out of LDS.
// * v_mfma_f32_16x16x32_bf16 (a whole 32-k step per instruction, 32 per wave per step) with B as
//   the first operand and A as the second, so each lane's accumulator holds 4 consecutive columns
//   of one row of C: the epilogue converts pairs with v_cvt_pk_bf16_f32 (round to nearest even)
//   and stores 8 bytes per lane. Against v_mfma_f32_32x32x16_bf16 (same flops per cycle, same
//   LDS reads and registers) it measured 1-4% faster: shorter instructions leave the compiler
//   finer interleaving.
// * Split pieces store float32 partials to a workspace slot with device-scope stores, then bump
//   an arrival counter; the last arriver adds all pieces of the tile in K order, writes bf16 and
//   returns the counter to zero for the next launch (no memset, no spin-waiting).
// * The SwiGLU form (GLU = true) computes h = silu(A Wg) * (A Wu) with Wg and Wu the two halves
//   of one K x 2N weight. A BN-wide tile then covers BN / 2 outputs: each wave's WTN columns in
//   LDS are WTN / 2 gate columns followed by the same WTN / 2 up columns, chosen per lane in the
//   B loads, so gate tile ni and up tile ni + TN / 2 of a lane hold the same outputs and the
//   epilogue combines them in registers (spark-kernels post, "the memory-bound kernels": SwiGLU
//   in one kernel instead of two, here fused into the product that makes its inputs).

#include <type_traits>

#include "common.h"
#include "tile.h"

namespace glk {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int BM, int BN, int WM, int WN, int SB_ = 3>
struct TileTraits {
    static constexpr int BK = 32;                           // k per step (B stage, MFMA step)
    static constexpr int AK = 64;                           // k per A stage: 128-byte rows
    // A ring SA stages of BM x 64, B ring SB stages of 32 x BN (144 KB for the 256 x 256 tile,
    // 72 KB for 128 x 128). A 3-stage B ring measured faster than 4 stages, with the same bits:
    // about 10% on every 128 x 128 grid and 0.5-1% with 256 x 256 tiles; 2 stages lost 25-30%
    static constexpr int SA = 3;
    static constexpr int SB = SB_;
    static constexpr int DB = SB;                           // steps B is issued ahead
    static constexpr int DA = DB + 1;                       // A half stages issued ahead
    static constexpr int NW = WM * WN;
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WM;
    static constexpr int WTN = BN / WN;
    static constexpr int TM = WTM / 16;                     // 16-row MFMA tiles per wave
    static constexpr int TN = WTN / 16;                     // 16-column MFMA tiles per wave
    static constexpr int A_BYTES = BM * AK * 2;             // one A stage, 128-byte rows
    static constexpr int B_BYTES = BK * BN * 2;             // one B stage, 2*BN-byte rows
    static constexpr int A_INSTR = A_BYTES / 1024;          // 1 KB direct-to-LDS instructions
    static constexpr int B_INSTR = B_BYTES / 1024;
    static constexpr int A_PER_WAVE = A_INSTR / NW;         // per wave per A stage
    static constexpr int A_HALF = A_PER_WAVE / 2;           // ... issued over two steps
    static constexpr int B_PER_WAVE = B_INSTR / NW;
    static constexpr int LOADS = A_HALF + B_PER_WAVE;       // per wave per step
    static constexpr int B_CHUNKS = BN / 8;                 // 16-byte chunks per B row
    static constexpr int B_ROWS_PER_INSTR = 1024 / (2 * BN);
    static constexpr int B_RING = SA * A_BYTES;             // B ring offset
    static constexpr int LDS_BYTES = SA * A_BYTES + SB * B_BYTES;
    // The planner splits K only for tiles smaller than 256 x 256 (a grid of 256-wide tiles too
    // small to fill the card falls back to smaller tiles first), so only those carry the split
    // fixup, whose registers would otherwise crowd the main loop of the big tiles.
    static constexpr bool SPLIT = BM * BN < 256 * 256;
    static_assert(A_PER_WAVE * NW == A_INSTR && B_PER_WAVE * NW == B_INSTR, "loads split evenly");
    static_assert(BN >= 128, "B swizzle needs at least 8 column groups per row");
    static_assert(TM >= 1 && TN >= 1, "wave tile must hold whole 16x16 MFMA tiles");
    static_assert(A_HALF * 2 == A_PER_WAVE, "A stage loads split over two steps");
    static_assert(LDS_BYTES <= ((BM * BN >= 256 * 256) ? 160 * 1024 : 80 * 1024), "LDS");
    static_assert(DB <= SB && DA <= 2 * SA - 1, "ring slots reused only after their last read");
    static_assert(LOADS * (DB + 2) + A_HALF <= 63, "vmcnt range");
};

// A: physical 16-byte chunk of logical chunk c (0..7) in row m. Sixteen consecutive rows (the
// lanes one LDS cycle serves a ds_read_b128 for) then cover all 64 banks for any fixed c: the
// two rows of a 256-byte bank line differ in m & 1, the eight lines in (m >> 1) & 7.
__device__ __forceinline__ int a_swz(int c, int m) { return c ^ ((m >> 1) & 7); }
// B: physical 32-byte column group of logical group u in k row k. One transposed fragment read
// touches rows k = 8 G + r + 4 h (lane group G = 0..3, r = 0..3, h fixed) of one logical group;
// XOR-ing in k's bits 0, 1 and 3 puts those 16 row pieces on 8 distinct 32-byte bank groups,
// two each, where k & 7 gave 4 (the four G collided). Measured: 3.5 instead of 4.0 LDS cycles
// per read.
__device__ __forceinline__ int b_swz(int u, int k) { return u ^ ((k & 3) | ((k >> 1) & 4)); }

template <int BM, int BN, int WM, int WN, bool GLU>
// (two waves per SIMD: at most 256 registers per lane, so two 128 x 128 workgroups fit on a CU
// together, and one 256 x 256 workgroup's eight waves fit at all)
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                               amdgpu_waves_per_eu(2, 2)))
tile_gemm_kernel(TileArgs p) {
    using T = TileTraits<BM, BN, WM, WN>;
    static_assert(!GLU || (T::TN % 2 == 0), "SwiGLU pairs gate and up tiles within a wave");
    constexpr int BK = T::BK, TM = T::TM, TN = T::TN;
    extern __shared__ __attribute__((aligned(1024))) char lds[];

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
    // n0: first output column of the tile (a SwiGLU tile's BN columns make BN / 2 outputs)
    const int m0 = tm * BM, n0 = tn * (GLU ? BN / 2 : BN);
    const int kt_total = (p.K + BK - 1) / BK;
    int kt_begin = 0, kt_end = kt_total;
    if (p.sched == kSchedSplitK) {
        kt_begin = piece * p.kt_per_split;
        kt_end = min(kt_total, kt_begin + p.kt_per_split);
    }
    const int nsteps = max(kt_end - kt_begin, 0);

    // ---- direct-to-LDS load addressing ---------------------------------------------------------
    // A instruction i of this wave (per A stage): tile rows 8 (wave * A_PER_WAVE + i) .. +7; lane
    // l lands at byte 16 l = row + l/8, physical chunk l%8, and fetches the logical chunk stored
    // there. Instructions 0 .. A_HALF-1 go out in the first step of the stage's issue, the rest in
    // the second.
    uint32_t a_off[T::A_PER_WAVE];
    int a_kchunk[T::A_PER_WAVE];
    bool a_row_ok[T::A_PER_WAVE];
#pragma unroll
    for (int i = 0; i < T::A_PER_WAVE; ++i) {
        const int row = 8 * (wave * T::A_PER_WAVE + i) + (lane >> 3);
        a_kchunk[i] = a_swz(lane & 7, row);  // the swizzle is an involution
        a_row_ok[i] = m0 + row < p.M;
        a_off[i] = (uint32_t)(row * p.lda + 8 * a_kchunk[i]) * 2u;
    }
    // B instruction i: k rows R0 .. R0 + B_ROWS_PER_INSTR - 1; lane l -> row R0 + l / B_CHUNKS,
    // physical chunk l % B_CHUNKS (group pc/2, half pc%2), holding logical group b_swz(pc/2, k).
    uint32_t b_off[T::B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < T::B_PER_WAVE; ++i) {
        const int k = (wave * T::B_PER_WAVE + i) * T::B_ROWS_PER_INSTR + lane / T::B_CHUNKS;
        const int pc = lane % T::B_CHUNKS;
        const int col = 16 * b_swz(pc >> 1, k) + 8 * (pc & 1);
        if constexpr (GLU) {  // LDS column -> output column `out` of the gate or the up half
            const int r = col % T::WTN;
            const int out = (col / T::WTN) * (T::WTN / 2) + r % (T::WTN / 2);
            const int src = (r < T::WTN / 2 ? 0 : p.N) + out;
            b_off[i] = sel_off(n0 + out < p.N, (uint32_t)(k * p.ldb + src) * 2u);
        } else {
            b_off[i] = sel_off(n0 + col < p.N, (uint32_t)(k * p.ldb + col) * 2u);
        }
    }

    // half h of A stage s (k 64 s .. 64 s + 63 of this workgroup's range) into A slot s % SA
    auto issue_a_half = [&](int s, int h) {
        const uint32_t st_lds = lds_addr(lds + (s % T::SA) * T::A_BYTES);
        const int k0 = kt_begin * BK + s * T::AK;
        const int kend = kt_end * BK < p.K ? kt_end * BK : p.K;
        const int krows = max(0, min(T::AK, kend - k0));  // uniform
        const i32x4 ar = rsrc_words(p.A + (size_t)m0 * p.lda + k0, kBufRecords);
#pragma unroll
        for (int u = 0; u < T::A_HALF; ++u) {
            const int t = h * T::A_HALF + u;
            const bool ok = a_row_ok[t] && 8 * a_kchunk[t] < krows;
            dma16(ar, st_lds + (wave * T::A_PER_WAVE + t) * 1024, sel_off(ok, a_off[t]));
        }
    };
    // the B stage of step i into B slot i % SB
    auto issue_b = [&](int i) {
        const uint32_t st_lds = lds_addr(lds + T::B_RING + (i % T::SB) * T::B_BYTES);
        const int k0 = (kt_begin + i) * BK;
        const int krows = (i < nsteps) ? min(BK, p.K - k0) : 0;  // uniform
        const i32x4 br = rsrc_words(p.B + (size_t)k0 * p.ldb + n0, (uint32_t)krows * (uint32_t)p.ldb * 2u);
#pragma unroll
        for (int t = 0; t < T::B_PER_WAVE; ++t)
            dma16(br, st_lds + (wave * T::B_PER_WAVE + t) * 1024, b_off[t]);
    };
    // the loads of loop iteration I: A half stage I + DA, then the B stage of step I + DB
    auto issue_iter = [&](int I) {
        issue_a_half((I + T::DA) >> 1, (I + T::DA) & 1);
        issue_b(I + T::DB);
    };

    f32x4 acc[TN][TM];
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) acc[ni][mi] = f32x4{};

    // fragment addressing (v_mfma_f32_16x16x32_bf16, B first): 16-lane group G = lane / 16 holds
    // k 8G .. 8G + 7 of the step's 32.
    // A (second operand, 32 k x 16 m): lane l reads row 16 mi + (l & 15), the step's logical chunk
    // 4 (i & 1) + G of the 64-k A stage.
    // B (first operand, 16 n x 32 k): inside group G, lane j addresses k row 8G + j / 4 (+ 4 for
    // the second read) and columns 4 (j % 4) .. +3 of the 16-column tile; the transposed read
    // hands lane j column j of each 4 x 16 block.
    const int fa_row = lane & 15, fG = lane >> 4, fj = lane & 15;
    const int fb_k = 8 * fG + (fj >> 2);
    const int fb_n = 4 * (fj & 3);

    struct Frags {
        bf16x8 a[TM];
        bf16x8 b[TN];
    };

    auto read_frags = [&](int i, Frags& f) {
        const char* sa = lds + ((i >> 1) % T::SA) * T::A_BYTES;
        const char* sb = lds + T::B_RING + (i % T::SB) * T::B_BYTES;
        const int ch = 4 * (i & 1) + fG;  // logical 16-byte chunk of the 64-k A row
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) {
            const int m = wm * T::WTM + mi * 16 + fa_row;
            f.a[mi] = *reinterpret_cast<const bf16x8*>(sa + m * 128 + 16 * a_swz(ch, m));
        }
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int n = wn * T::WTN + ni * 16 + fb_n;
            i16x4 v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = fb_k + 4 * h;
                const char* addr = sb + k * (2 * BN) + 32 * b_swz(n >> 4, k) + 2 * (n & 15);
                v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)addr);
            }
            const i16x8 x = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
            f.b[ni] = __builtin_bit_cast(bf16x8, x);
        }
    };

    auto mfma_frags = [&](const Frags& f) {
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int mi = 0; mi < TM; ++mi) acc[ni][mi] = mfma16(f.b[ni], f.a[mi], acc[ni][mi]);
    };

    // ---- main loop ------------------------------------------------------------------------
    // Iteration I issues A half stage I + DA and the B stage of step I + DB, reads the fragments
    // of step I + 1 and runs the MFMAs of step I (fragments read during iteration I - 1). Every
    // iteration's loads are the same LOADS instructions per wave, so "the loads of iteration X
    // have landed" is one vmcnt threshold: step I + 1's B stage was issued in iteration
    // I + 1 - DB and the second half of its A stage no later, so iteration I waits for all but
    // the last DB - 2 iterations' loads. A B slot is refilled DB steps after the step that last
    // read it, an A slot 2 SA - DA half stages after; both reads ended before that iteration's
    // barrier.
    Frags f0, f1;
    issue_a_half(0, 0);  // the prologue issues as iterations -DB .. -1 would, plus half stage 0
#pragma unroll
    for (int I = -T::DB; I < 0; ++I) issue_iter(I);
    wait_vmcnt<T::LOADS * (T::DB - 1)>();  // iteration -DB's loads (step 0's B, A stage 0) landed
    lds_barrier();
    read_frags(0, f0);
    // (reading the next fragments past the last step is harmless: that slot holds zeros or
    // stale data that no MFMA consumes)
#define GLK_TILE_STEP(I, CUR, NEXT)                                                           \
    do {                                                                                      \
        wait_vmcnt<T::LOADS * (T::DB - 2)>(); /* this wave's loads for step I + 1 landed */   \
        lds_barrier(); /* every wave's have; all are done reading the slots refilled next */  \
        issue_iter(I);                                                                        \
        read_frags((I) + 1, NEXT);                                                            \
        mfma_frags(CUR);                                                                      \
    } while (0)
    int i = 0;
    for (; i + 1 < nsteps; i += 2) {
        GLK_TILE_STEP(i, f0, f1);
        GLK_TILE_STEP(i + 1, f1, f0);
    }
    if (i < nsteps) GLK_TILE_STEP(i, f0, f1);
#undef GLK_TILE_STEP
    wait_vmcnt<0>();
    lds_barrier();  // the ring is idle from here on; its first word serves the fixup below

    // ---- split fixup ---------------------------------------------------------------------------
    // Lane layout of acc[ni][mi][r]: row m = wm*WTM + mi*16 + (lane & 15),
    // column n = wn*WTN + ni*16 + 4*(lane >> 4) + r.
    if (T::SPLIT && p.sched == kSchedSplitK && p.splits > 1) {
        const int npieces = min(p.splits, (kt_total + p.kt_per_split - 1) / p.kt_per_split);
        if (npieces > 1) {
            volatile uint32_t& last_flag = *reinterpret_cast<volatile uint32_t*>(lds);
            // slot layout (floats, fragment order): [wave][ni][mi][lane][4]
            const __amdgpu_buffer_rsrc_t ws = make_rsrc(p.ws + (size_t)tile * p.splits * (BM * BN));
            const uint32_t slot_bytes = (uint32_t)(BM * BN) * 4u;
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int mi = 0; mi < TM; ++mi) {
                    const uint32_t off = (uint32_t)((((wave * TN + ni) * TM + mi) * 64 + lane) * 16);
                    buf_store16_dev(ws, (uint32_t)piece * slot_bytes + off, f4_bits(acc[ni][mi]));
                }
            wait_all_memory();
            __syncthreads();
            if (tid == 0)
                last_flag = (counter_arrive(&p.counters[tile]) == (uint32_t)(npieces - 1)) ? 1u : 0u;
            __syncthreads();
            if (!last_flag) return;
            if (tid == 0) counter_reset(&p.counters[tile]);
            // sum the pieces in K order, piece 0 first, with all of a piece's loads in flight
            // before its adds (one memory latency per piece, not one per fragment)
            f32x4 sum[TN][TM];
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int mi = 0; mi < TM; ++mi) sum[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int pc = 0; pc < npieces; ++pc) {
                if (pc == piece) {
#pragma unroll
                    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                        for (int mi = 0; mi < TM; ++mi) sum[ni][mi] += acc[ni][mi];
                    continue;
                }
                f32x4 v[TN][TM];
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int mi = 0; mi < TM; ++mi) {
                        const uint32_t off = (uint32_t)((((wave * TN + ni) * TM + mi) * 64 + lane) * 16);
                        v[ni][mi] = bits_f4(buf_load16_dev(ws, (uint32_t)pc * slot_bytes + off));
                    }
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int mi = 0; mi < TM; ++mi) sum[ni][mi] += v[ni][mi];
            }
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int mi = 0; mi < TM; ++mi) acc[ni][mi] = sum[ni][mi];
        }
    }

    // ---- epilogue: bf16 (round to nearest even), 8-byte stores -------------------------------
    // (SwiGLU: gate tile ni and up tile ni + TN / 2 hold the same outputs)
    constexpr int TNO = GLU ? TN / 2 : TN;
    constexpr int WTNO = GLU ? T::WTN / 2 : T::WTN;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + (size_t)m0 * p.ldc + n0);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
        const int m = wm * T::WTM + mi * 16 + fa_row;
        const bool m_ok = (m0 + m) < p.M;
#pragma unroll
        for (int ni = 0; ni < TNO; ++ni) {
            const int n = wn * WTNO + ni * 16 + 4 * fG;
            const bool ok = m_ok && (n0 + n) < p.N;
            f32x4 h;
            if constexpr (GLU) {
                h = swiglu4(acc[ni][mi], acc[ni + TNO][mi]);
            } else {
                h = acc[ni][mi];
            }
            u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
            buf_store8(rc, ok ? (uint32_t)(m * p.ldc + n) * 2u : kBufInvalid, v);
        }
    }
}

// ---- 256 x 256 tile, two wave groups alternating MFMA and memory phases ----------------------
// The same tile, staging, swizzles, fragment layout and epilogue as tile_gemm_kernel<256, 256, 2,
// 4>, with a different schedule for the eight waves. The waves form two groups of four, one wave
// of each group per SIMD (group 0: waves 0-3, rows 0-127 of the tile; group 1: waves 4-7, rows
// 128-255). Every 32-k step a wave runs two phases, separated by workgroup barriers:
//   memory phase:  its MFMA operands for the step, LDS -> registers, and its share of the
//                  direct-to-LDS loads of a later stage; then it waits for both;
//   compute phase: the step's 32 MFMAs back to back, on operands already in registers.
// Group 1 starts one barrier later, so while one group's four waves keep the four SIMDs' matrix
// cores busy, the other group's waves fetch, and the roles swap at every barrier. (spark-kernels
// post, "the copies were the problem, not the power": keep copies and their waits out of the
// matrix instructions' stream; here the copies move to the other wave of each SIMD, not to a
// dedicated producer, because gfx950 gives every wave of a workgroup the same register budget.)
//
// Barriers after the prologue's are numbered b1, b2, ...; group 0 runs the memory phase of step
// s before b(2s+1) and its compute phase before b(2s+2); group 1 (with its extra first barrier)
// one barrier later. The last LDS read of step s's data is group 1's, before b(2s+2); so B stage
// s + SB - 1, which reuses step s - 1's slot, and A half stage s + 4, which reuses a slot last read
// before b(2s), may be issued in step s's memory phases. Each wave waits at the end of its memory
// phase of step s for its loads of step s + 1 (issued by iteration s + 1 - DB and earlier), before
// the barrier after which group 0 reads them.
template <int SB, bool GLU>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
tile_pp_kernel(TileArgs p) {
    constexpr int BM = 256, BN = 256, WM = 2, WN = 4;
    using T = TileTraits<BM, BN, WM, WN, SB>;
    static_assert(T::TN % 2 == 0, "SwiGLU pairs gate and up tiles within a wave");
    static_assert(T::LDS_BYTES <= 160 * 1024, "LDS");
    constexpr int BK = T::BK, TM = T::TM, TN = T::TN;
    constexpr int DB = SB - 1;  // B stages issued ahead
    constexpr int DA = 4;       // A half stages issued ahead
    constexpr int LOADS = T::LOADS;
    extern __shared__ __attribute__((aligned(1024))) char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int wm = grp, wn = wave & 3;

    // ---- which tile (data-parallel only) -------------------------------------------------------
    const int ntiles = p.tiles_m * p.tiles_n;
    const int tile = xcd_remap((int)blockIdx.x, ntiles, p.nxcd);
    const int per_group = p.group_m * p.tiles_n;
    const int g = tile / per_group;
    const int first_m = g * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int in_g = tile - g * per_group;
    const int tm = first_m + in_g % gm;
    const int tn = in_g / gm;
    const int m0 = tm * BM, n0 = tn * (GLU ? BN / 2 : BN);
    const int nsteps = (p.K + BK - 1) / BK;

    // ---- direct-to-LDS load addressing (as in tile_gemm_kernel) ------------------------------
    uint32_t a_off[T::A_PER_WAVE];
    int a_kchunk[T::A_PER_WAVE];
    bool a_row_ok[T::A_PER_WAVE];
#pragma unroll
    for (int i = 0; i < T::A_PER_WAVE; ++i) {
        const int row = 8 * (wave * T::A_PER_WAVE + i) + (lane >> 3);
        a_kchunk[i] = a_swz(lane & 7, row);
        a_row_ok[i] = m0 + row < p.M;
        a_off[i] = (uint32_t)(row * p.lda + 8 * a_kchunk[i]) * 2u;
    }
    uint32_t b_off[T::B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < T::B_PER_WAVE; ++i) {
        const int k = (wave * T::B_PER_WAVE + i) * T::B_ROWS_PER_INSTR + lane / T::B_CHUNKS;
        const int pc = lane % T::B_CHUNKS;
        const int col = 16 * b_swz(pc >> 1, k) + 8 * (pc & 1);
        if constexpr (GLU) {
            const int r = col % T::WTN;
            const int out = (col / T::WTN) * (T::WTN / 2) + r % (T::WTN / 2);
            const int src = (r < T::WTN / 2 ? 0 : p.N) + out;
            b_off[i] = sel_off(n0 + out < p.N, (uint32_t)(k * p.ldb + src) * 2u);
        } else {
            b_off[i] = sel_off(n0 + col < p.N, (uint32_t)(k * p.ldb + col) * 2u);
        }
    }
    // half H (a compile-time 0 or 1) of A stage st
    auto issue_a_half = [&](int st, auto hc) {
        constexpr int H = decltype(hc)::value;
        const uint32_t st_lds = lds_addr(lds + (st % T::SA) * T::A_BYTES);
        const int k0 = st * T::AK;
        const int krows = max(0, min(T::AK, p.K - k0));  // uniform
        const i32x4 ar = rsrc_words(p.A + (size_t)m0 * p.lda + k0, kBufRecords);
#pragma unroll
        for (int u = 0; u < T::A_HALF; ++u) {
            const int t = H * T::A_HALF + u;
            const bool ok = a_row_ok[t] & (8 * a_kchunk[t] < krows);
            dma16(ar, st_lds + (wave * T::A_PER_WAVE + t) * 1024, sel_off(ok, a_off[t]));
        }
    };
    auto issue_b = [&](int i) {
        const uint32_t st_lds = lds_addr(lds + T::B_RING + (i % SB) * T::B_BYTES);
        const int k0 = i * BK;
        const int krows = (i < nsteps) ? min(BK, p.K - k0) : 0;  // uniform
        const i32x4 br = rsrc_words(p.B + (size_t)k0 * p.ldb + n0, (uint32_t)krows * (uint32_t)p.ldb * 2u);
#pragma unroll
        for (int t = 0; t < T::B_PER_WAVE; ++t)
            dma16(br, st_lds + (wave * T::B_PER_WAVE + t) * 1024, b_off[t]);
    };

    f32x4 acc[TN][TM];
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) acc[ni][mi] = f32x4{};

    const int fa_row = lane & 15, fG = lane >> 4, fj = lane & 15;
    const int fb_k = 8 * fG + (fj >> 2);
    const int fb_n = 4 * (fj & 3);
    bf16x8 fa[TM], fb[TN];
    auto read_frags = [&](int i) {
        const char* sa = lds + ((i >> 1) % T::SA) * T::A_BYTES;
        const char* sb = lds + T::B_RING + (i % SB) * T::B_BYTES;
        const int ch = 4 * (i & 1) + fG;
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) {
            const int m = wm * T::WTM + mi * 16 + fa_row;
            fa[mi] = *reinterpret_cast<const bf16x8*>(sa + m * 128 + 16 * a_swz(ch, m));
        }
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int n = wn * T::WTN + ni * 16 + fb_n;
            i16x4 v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = fb_k + 4 * h;
                const char* addr = sb + k * (2 * BN) + 32 * b_swz(n >> 4, k) + 2 * (n & 15);
                v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)addr);
            }
            const i16x8 x = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
            fb[ni] = __builtin_bit_cast(bf16x8, x);
        }
    };
    auto phase_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: the loads iterations -DA .. -1 would issue; step 0's data landed ----------
    // (iteration I issues A half stage I + DA, then B stage I + DB; in the loop the wait for step
    // s + 1's data then allows exactly the last DB - 1 iterations' loads in flight)
    static_assert(DA == 4 && DB >= 2 && DB <= 3, "load order and counts");
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    issue_a_half(0, H0{});   // iteration -4
    issue_a_half(0, H1{});   // iteration -3
    if (DB >= 3) issue_b(0);
    issue_a_half(1, H0{});   // iteration -2
    issue_b(DB - 2);
    issue_a_half(1, H1{});   // iteration -1
    issue_b(DB - 1);
    wait_vmcnt<LOADS * (DB - 1)>();
    lds_barrier();
    if (grp == 1) phase_barrier();
    // step s issues A half stage s + DA (half (s + DA) & 1 = s & 1) and B stage s + DB
    auto step = [&](int s, auto hc) {
        // memory phase
        read_frags(s);
        issue_a_half((s + DA) >> 1, hc);
        issue_b(s + DB);
        wait_vmcnt<LOADS * (DB - 1)>();  // this wave's loads for step s + 1 landed
        wait_lgkmcnt0();                 // and its operands for step s are in registers
        phase_barrier();
        // compute phase
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int mi = 0; mi < TM; ++mi) acc[ni][mi] = mfma16(fb[ni], fa[mi], acc[ni][mi]);
        phase_barrier();
    };
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
        step(s, H0{});
        step(s + 1, H1{});
    }
    if (s < nsteps) step(s, H0{});
    if (grp == 0) phase_barrier();
    wait_vmcnt<0>();  // every direct-to-LDS write of this wave (prefetches past K included) landed
    lds_barrier();    // ... and of every wave: the ring is free for the output

    // ---- epilogue: bf16 (round to nearest even) through LDS, whole 128-byte rows ------------
    // Lane l holds rows 16 mi + (l & 15), columns 16 ni + 4 (l >> 4) .. + 3 of the wave's tile,
    // 8 bytes per (mi, ni) once rounded. Each wave writes its WTM x WTNO bf16 block to its own
    // LDS area (rows of RB bytes, 16-byte chunk c of row r stored at c ^ (r & 7)), then reads it
    // back 16 bytes per lane, RB / 16 lanes per row, and writes C in whole row segments: one
    // 16-byte store per lane instead of two 8-byte ones, every row segment written by one
    // instruction (measured: the 8-byte stores took 6.5 us of a 103 us 4096^3 product; this
    // epilogue takes about 4 us, and 101 us for the whole product).
    // (SwiGLU: gate tile ni and up tile ni + TN / 2 hold the same outputs)
    constexpr int TNO = GLU ? TN / 2 : TN;
    constexpr int WTNO = GLU ? T::WTN / 2 : T::WTN;
    constexpr int RB = WTNO * 2;                 // bytes per output row of the wave's block
    constexpr int CPR = RB / 16;                 // 16-byte chunks per row (8 or 4)
    constexpr int ROWS_PER_ST = 64 / CPR;        // rows per 16-byte store instruction
    static_assert(T::WTM * RB * 8 <= T::LDS_BYTES, "output blocks fit the ring");
    char* ob = lds + wave * (T::WTM * RB);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
        const int r = mi * 16 + fa_row;
#pragma unroll
        for (int ni = 0; ni < TNO; ++ni) {
            f32x4 h;
            if constexpr (GLU) {
                h = swiglu4(acc[ni][mi], acc[ni + TNO][mi]);
            } else {
                h = acc[ni][mi];
            }
            const u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
            const int byte = ni * 32 + fG * 8;         // within the row
            const int c = (byte >> 4) ^ (r & (CPR - 1) & 7);
            *reinterpret_cast<u32x2*>(ob + r * RB + c * 16 + (byte & 15)) = v;
        }
    }
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + (size_t)m0 * p.ldc + n0);
    const int lr = lane / CPR, lc = lane % CPR;  // row within a store, logical chunk
    const int gn = wn * WTNO + lc * 8;           // output column of the chunk, within the tile
#pragma unroll
    for (int st = 0; st < T::WTM / ROWS_PER_ST; ++st) {
        const int r = st * ROWS_PER_ST + lr;
        const u32x4 v = *reinterpret_cast<const u32x4*>(ob + r * RB + (lc ^ (r & (CPR - 1) & 7)) * 16);
        const int m = wm * T::WTM + r;
        const bool ok = (m0 + m) < p.M && (n0 + gn) < p.N;
        // non-temporal: C is written once and is far larger than the L2s (measured 1.2-1.4%
        // faster on multi-wave grids, neutral at 4096^3)
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, ok ? (uint32_t)(m * p.ldc + gn) * 2u : kBufInvalid, 0, kAuxNonTemporal);
    }
}


TileShape tile_shape(int cfg) {
    switch (cfg) {
        case kTile256x256w8: return {256, 256, 32, 512};
        case kTile128x128w4: return {128, 128, 32, 256};
        case kTile256x256pp: return {256, 256, 32, 512};
        default: return {0, 0, 0, 0};
    }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_cfg(const TileArgs& a, int grid, bool glu, hipStream_t s) {
    using T = TileTraits<BM, BN, WM, WN>;
    if (!T::SPLIT && a.sched == kSchedSplitK && a.splits > 1) return hipErrorInvalidValue;
    if (glu)
        tile_gemm_kernel<BM, BN, WM, WN, true><<<grid, T::NT, T::LDS_BYTES, s>>>(a);
    else
        tile_gemm_kernel<BM, BN, WM, WN, false><<<grid, T::NT, T::LDS_BYTES, s>>>(a);
    return hipGetLastError();
}

template <int SB>
static hipError_t launch_pp(const TileArgs& a, int grid, bool glu, hipStream_t s) {
    using T = TileTraits<256, 256, 2, 4, SB>;
    if (a.sched != kSchedDataParallel) return hipErrorInvalidValue;
    if (glu)
        tile_pp_kernel<SB, true><<<grid, T::NT, T::LDS_BYTES, s>>>(a);
    else
        tile_pp_kernel<SB, false><<<grid, T::NT, T::LDS_BYTES, s>>>(a);
    return hipGetLastError();
}

template <int SB>
static hipError_t configure_pp() {
    const int bytes = TileTraits<256, 256, 2, 4, SB>::LDS_BYTES;
    hipError_t e = hipFuncSetAttribute((const void*)tile_pp_kernel<SB, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)tile_pp_kernel<SB, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return e;
}

template <int BM, int BN, int WM, int WN>
static hipError_t configure_cfg() {
    hipError_t e = hipFuncSetAttribute((const void*)tile_gemm_kernel<BM, BN, WM, WN, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       TileTraits<BM, BN, WM, WN>::LDS_BYTES);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)tile_gemm_kernel<BM, BN, WM, WN, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                TileTraits<BM, BN, WM, WN>::LDS_BYTES);
    return e;
}

hipError_t configure_tile_kernels() {
    hipError_t e = configure_cfg<256, 256, 2, 4>();
    if (e == hipSuccess) e = configure_cfg<128, 128, 2, 2>();
    if (e == hipSuccess) e = configure_pp<4>();
    return e;
}

hipError_t launch_tile_gemm(int cfg, const TileArgs& a, int grid, bool glu, hipStream_t s) {
    switch (cfg) {
        case kTile256x256w8: return launch_cfg<256, 256, 2, 4>(a, grid, glu, s);
        case kTile128x128w4: return launch_cfg<128, 128, 2, 2>(a, grid, glu, s);
        case kTile256x256pp: return launch_pp<4>(a, grid, glu, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace glk
