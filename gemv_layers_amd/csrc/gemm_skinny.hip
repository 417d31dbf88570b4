// Skinny-M bf16 GEMM for gfx950 (1 <= M <= 64): C = A * B where B (K x N) is streamed from HBM
// exactly once for all M rows, float32 accumulation, bf16 output.
//
// Design ("The kernels that were there", "The GEMV": load-bound, so parallelise over output
// columns, coalesced 128-bit weight loads, fp32 accumulation, every weight loaded once for all
// rows; spark-kernels post, "the decode kernel": a tile of 16/32/64 rows picked from M, one
// workgroup per column strip of B, and K split only as far as needed to fill the card, the last
// slice leaving the workspace as it found it so a call stays one launch; enough bytes in flight
// per workgroup to reach the memory floor):
//
// * The work is a strip-major list of units (one 64-row stage of one strip of SW = 128 or 256
//   columns). At most one workgroup per CU takes a balanced, contiguous range of units (the
//   Stream-K decomposition of the spark-kernels post, "stream-k proper"), so no partial last wave
//   of workgroups exists; only the first and the last strip a range touches can be partial, and
//   when the grid is a whole number of pieces per strip every range is one piece of one strip. Ranges are dealt so that each
//   XCD holds consecutive ones, so the pieces of a strip mostly run on one XCD and an XCD that
//   starts late delays only its own strips. The units stream through
//   an LDS ring of STAGES stages: each is fetched with direct-to-LDS buffer loads (16 bytes per
//   lane, 1 KB per wave instruction, no registers involved), STAGES - 1 stages ahead of use, and
//   carries the matching 64 columns of A (M rows) so every wave reads A from LDS.
// * B sits in LDS row-major (k rows of 2 SW bytes). The MFMA operand wants 8 consecutive k per
//   lane for one column, which ds_read_b64_tr_b16 produces directly from row-major data: within
//   each 16-lane group, lanes 4r .. 4r+3 address row r of a 4 x 16 block and lane j receives
//   column j. The 32-byte column groups of each row are XOR-swizzled with the row so the rows a
//   wave reads together fall in different banks.
// * Each of the 4 waves owns SW / 4 columns (SW / 64 16-column MFMA tiles) for all M rows, using
//   v_mfma_f32_16x16x32_bf16 with B as the first operand: each lane's accumulator then holds 4
//   consecutive columns of one row of C, stored as one 8-byte bf16 write. M is padded to 16 per
//   tile with zero rows (A rows past M are fetched as zeros); the matrix cores are otherwise idle
//   in this memory-bound kernel, so the padding costs nothing.
// * A strip whose units all fall in one workgroup is written straight to C. Otherwise each piece
//   writes its float32 partial to the workgroup's slot and bumps a per-strip counter; the last
//   arriver loads every piece (all loads issued before any add), adds them in K order, writes
//   bf16 and returns the counter to zero. Partials travel at device scope (written through to the
//   device coherence point), whichever XCDs the pieces ran on.
// * The SwiGLU form (GLU = true) computes h = silu(A Wg) * (A Wu), Wg and Wu the two halves of one
//   K x 2N weight: a strip of SW columns in LDS covers SW / 2 outputs, each wave's first TN / 2
//   tiles being gate columns and its last TN / 2 the same up columns (chosen per lane in the B
//   loads), so the epilogue pairs tile t with tile t + TN / 2 in registers. Partials and their
//   reduction are unchanged; the activation is applied where bf16 is written.

#include "common.h"
#include "skinny.h"

namespace glk {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kSkRows = kSkinnyStage;                  // k rows per LDS stage

// MT 16-row tiles of M; SW columns per strip
template <int MT, int SW>
struct SkinnyTraits {
    static constexpr int TN = SW / 64;                     // 16-column tiles per wave
    static constexpr int ROW_BYTES = SW * 2;               // B bytes per k row of a strip
    static constexpr int B_BYTES = kSkRows * ROW_BYTES;    // B bytes per stage (16 or 32 KB)
    static constexpr int B_INSTR = B_BYTES / 1024;         // 1 KB load instructions for B per stage
    static constexpr int B_PER_WAVE = B_INSTR / 4;
    static constexpr int ROWS_PER_INSTR = 1024 / ROW_BYTES;
    static constexpr int CHUNKS = ROW_BYTES / 16;          // 16-byte chunks per B row
    static constexpr int A_BYTES = 16 * MT * kSkRows * 2;  // A rows (M padded to 16 MT) x 64 k
    static constexpr int STAGE_BYTES = B_BYTES + A_BYTES;
    // ring: 4 stages in every configuration. 128-column strips: 72, 80, 88 and 96 KB for one to
    // four 16-row tiles of M (budgets of 80 KB up to two tiles, 96 KB above; measured with
    // settled clocks against the earlier 128 KB, same bits: dec_down_M1 22.3 -> 20.4 us,
    // dec_down_M16 22.7 -> 21.0, dec_up_M64 29.3 -> 28.4). 256-column strips: 136 and 144 KB
    // (all of LDS less the padding sink and the static flag; their stages are twice as big)
    static constexpr int STAGES = (SW == 128 ? (MT <= 2 ? 81920 : 98304) : 163840 - 2048) / STAGE_BYTES;
    static constexpr int DUMMY = STAGES * STAGE_BYTES;     // 1 KB sink for padding loads
    static constexpr int LDS_BYTES = DUMMY + 1024;
    // LDS the launch asks for: more than half of a CU's 160 KB, so no two workgroups ever share a
    // CU (the grids are sized to one workgroup per CU, and a second one would halve both's share
    // of the CU's load path)
    static constexpr int LAUNCH_LDS = LDS_BYTES > 81920 ? LDS_BYTES : 81920 + 1024;
    static constexpr int A_INSTR = A_BYTES / 1024;         // 1 KB load instructions for A per stage
    static constexpr int A_PER_WAVE = (A_INSTR + 3) / 4;
    static constexpr int LOADS = B_PER_WAVE + A_PER_WAVE;  // load instructions per wave per stage
    static constexpr int SLOT_FLOATS = 4 * TN * MT * 64 * 4; // one piece: 4 waves x TN tiles x M
    static_assert(SW == 128 || SW == 256, "strip width");
    static_assert(B_PER_WAVE * ROWS_PER_INSTR == 16, "each wave loads 16 B rows of a stage");
    static_assert(STAGES >= 3, "need at least three stages");
    static_assert(LAUNCH_LDS > 163840 / 2 && LAUNCH_LDS <= 163840, "one workgroup per CU");
    static_assert(LOADS * (STAGES - 2) <= 63, "vmcnt range");
};

// Physical 32-byte column group of logical group u in row r (8 or 16 groups of 16 columns per
// row; rows are whole 256-byte bank lines, or two of them): the 4 rows a 16-lane group reads, and
// the groups 8 rows apart, land on different banks.
__device__ __forceinline__ int b_swz(int u, int r) { return u ^ ((r & 3) | (((r >> 3) & 1) << 2)); }

template <int MT, int SW, bool GLU>
__global__ void __launch_bounds__(256) skinny_gemm_kernel(SkinnyArgs p) {
    using T = SkinnyTraits<MT, SW>;
    constexpr int TN = T::TN;
    constexpr int SO = GLU ? SW / 2 : SW;    // output columns per strip
    constexpr int TNO = GLU ? TN / 2 : TN;   // output tiles per wave
    constexpr int STAGES = T::STAGES;
    extern __shared__ __attribute__((aligned(1024))) char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // ---- this workgroup's units: [u_begin, u_begin + nunits) of the strip-major list ----------
    const int w = xcd_remap((int)blockIdx.x, p.grid, p.nxcd);  // logical id: contiguous per XCD
    const int u_begin = range_begin(p.split, w);
    const int nunits = range_begin(p.split, w + 1) - u_begin;
    const int first_strip = (int)((uint32_t)u_begin / (uint32_t)p.ks);

    // ---- load addressing ---------------------------------------------------------------------
    // B: wave w fetches rows 16w .. 16w+15 of a stage, 4 rows per instruction; lane l lands at
    // byte 16 l of the instruction's 1 KB = row 4i + l/16 (of the wave's 16), physical 16-byte
    // chunk l%16, and fetches the logical chunk the swizzle keeps there (the swizzle is an
    // involution on the group index). Column validity is checked per unit (the strip varies).
    // (SwiGLU: LDS column 16 u + c of tile t = u % TN of wave u / TN is output column
    // 16 (TNO (u / TN) + t % TNO) + c of the strip, from the gate half for t < TNO, else the up
    // half N columns further on)
    uint32_t b_off[T::B_PER_WAVE];
    int b_col[T::B_PER_WAVE];  // output column within the strip, for the range check
#pragma unroll
    for (int i = 0; i < T::B_PER_WAVE; ++i) {
        const int r = 16 * wave + T::ROWS_PER_INSTR * i + lane / T::CHUNKS;
        const int pc = lane % T::CHUNKS;
        const int u = b_swz(pc >> 1, r);
        if constexpr (GLU) {
            const int t = u % TN;
            b_col[i] = 16 * (TNO * (u / TN) + t % TNO) + 8 * (pc & 1);
            b_off[i] = (uint32_t)(r * p.ldb + (t < TNO ? 0 : p.N) + b_col[i]) * 2u;
        } else {
            b_col[i] = 16 * u + 8 * (pc & 1);
            b_off[i] = (uint32_t)(r * p.ldb + b_col[i]) * 2u;
        }
    }
    // A: instruction j (= wave + 4t) covers A rows 8j .. 8j+7 of the padded M x 64 block;
    // lane l -> row 8j + l/8, physical chunk l%8 holding logical chunk (l%8) ^ (row & 7).
    uint32_t a_off[T::A_PER_WAVE];
    int a_chunk[T::A_PER_WAVE];
#pragma unroll
    for (int t = 0; t < T::A_PER_WAVE; ++t) {
        const int j = wave + 4 * t;
        const int row = 8 * j + (lane >> 3);
        a_chunk[t] = (lane & 7) ^ (row & 7);
        a_off[t] = sel_off(j < T::A_INSTR && row < p.M, (uint32_t)(row * p.lda + 8 * a_chunk[t]) * 2u);
    }
    const uint32_t dummy_lds = lds_addr(lds + T::DUMMY);

    // issue the loads of the workgroup's i-th unit into ring slot i % STAGES (units past the
    // range read nothing: a zero-length descriptor). Units are issued in order, so the (strip,
    // stage) position advances by one each call instead of being divided out of the index.
    int iss_strip = first_strip;
    int iss_stage = u_begin - first_strip * p.ks;
    auto issue_unit = [&](int i) {
        char* st = lds + (i % STAGES) * T::STAGE_BYTES;
        const int strip = __builtin_amdgcn_readfirstlane(iss_strip);  // wave-uniform
        const int k0 = __builtin_amdgcn_readfirstlane(iss_stage) * kSkRows;
        if (++iss_stage == p.ks) {
            iss_stage = 0;
            ++iss_strip;
        }
        const int n0 = strip * SO;
        const int rows = (i < nunits) ? min(kSkRows, p.K - k0) : 0;  // uniform
        const i32x4 b_rsrc = rsrc_words(p.B + (size_t)k0 * p.ldb + n0, (uint32_t)rows * (uint32_t)p.ldb * 2u);
        const uint32_t st_lds = lds_addr(st);
#pragma unroll
        for (int t = 0; t < T::B_PER_WAVE; ++t)
            dma16(b_rsrc, st_lds + (16 * wave + T::ROWS_PER_INSTR * t) * T::ROW_BYTES, sel_off(n0 + b_col[t] < p.N, b_off[t]));
        // A columns k0 .. k0 + rows; K % 8 == 0, so a 16-byte chunk is wholly in or out. A wave
        // without a real A instruction this round (the count need not divide by 4) still issues
        // one, into a spare kilobyte, so every wave issues the same number of loads per unit and
        // one vmcnt threshold fits all waves.
        const i32x4 a_rsrc = rsrc_words(p.A + k0, kBufRecords);
#pragma unroll
        for (int t = 0; t < T::A_PER_WAVE; ++t) {
            const int j = wave + 4 * t;
            const bool real = j < T::A_INSTR;
            const uint32_t off = sel_off(real && 8 * a_chunk[t] < rows, a_off[t]);
            dma16(a_rsrc, real ? st_lds + T::B_BYTES + j * 1024 : dummy_lds, off);
        }
    };

    f32x4 acc[TN][MT];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{};

    // fragment addressing: 16-lane group G = lane / 16 holds k rows 8G .. 8G+7 of a 32-row block;
    // inside the group, lane j addresses row (j / 4) of the 4-row transpose block and the 4
    // columns 4 (j % 4) .. +3 of the 16-column tile.
    const int fG = lane >> 4, fj = lane & 15;
    const int tr_row = 8 * fG + (fj >> 2);
    const int tr_colb = 8 * (fj & 3);
    const int a_frow = lane & 15;

    auto compute_unit = [&](int i) {
        const char* st = lds + (i % STAGES) * T::STAGE_BYTES;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {               // two 32-row blocks per stage
            bf16x8 bx[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                const int u = TN * wave + t;           // the wave's 16-column tile (logical group)
                i16x4 v[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 32 * kb + tr_row + 4 * h;
                    const char* addr = st + r * T::ROW_BYTES + b_swz(u, r) * 32 + tr_colb;
                    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)addr);
                }
                typedef short i16x8 __attribute__((ext_vector_type(8)));
                const i16x8 x = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
                bx[t] = __builtin_bit_cast(bf16x8, x);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = 16 * mt + a_frow;
                const int chunk = (4 * kb + fG) ^ (row & 7);
                const bf16x8 ay = *reinterpret_cast<const bf16x8*>(st + T::B_BYTES + row * 128 + chunk * 16);
#pragma unroll
                for (int t = 0; t < TN; ++t) acc[t][mt] = mfma16(bx[t], ay, acc[t][mt]);
            }
        }
    };

    // lane holds rows m = 16 mt + (lane & 15), columns 4 (lane >> 4) + 0..3 of each 16-column tile
    // (SwiGLU: tile t holds the gate and tile t + TNO the up values of the same outputs)
    auto store_c = [&](int strip) {
        const int n0 = strip * SO;
#pragma unroll
        for (int t = 0; t < TNO; ++t) {
            const int n = n0 + 16 * (TNO * wave + t) + 4 * (lane >> 4);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = 16 * mt + (lane & 15);
                if (m < p.M && n < p.N) {
                    f32x4 h;
                    if constexpr (GLU) {
                        h = swiglu4(acc[t][mt], acc[t + TNO][mt]);
                    } else {
                        h = acc[t][mt];
                    }
                    u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
                    *reinterpret_cast<u32x2*>(p.C + (size_t)m * p.ldc + n) = v;
                }
            }
        }
    };

    // workspace slot of workgroup w's piece of `strip`: 0 for the strip its range starts in, else 1
    const __amdgpu_buffer_rsrc_t ws = make_rsrc(p.ws);
    auto slot_off = [&](int wg, int seg, int t, int mt) {
        return (uint32_t)((((((wg * 2 + seg) * 4 + wave) * TN + t) * MT + mt) * 64 + lane) * 16);
    };
    // pieces of `strip` belong to logical workgroups wf .. wl (in K order)
    auto pieces_of = [&](int strip, int& wf, int& wl) {
        wf = range_of(p.split, strip * p.ks);
        wl = range_of(p.split, (strip + 1) * p.ks - 1);
    };
    // Only lanes holding a row below M move data: the padding rows' lanes get an out-of-range
    // offset, so a piece costs M rows of traffic rather than 16 MT.
    const int part_row = lane & 15;
    auto store_partial = [&](int strip) {  // device scope; not waited for here
        const int seg = (strip == first_strip) ? 0 : 1;
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                buf_store16_dev(ws, sel_off(16 * mt + part_row < p.M, slot_off(w, seg, t, mt)), f4_bits(acc[t][mt]));
    };
    // once every wave's partial stores of `strip` have completed: count this piece in; true for
    // the piece that completes the strip
    __shared__ uint32_t last_flag;
    auto arrive = [&](int strip) -> bool {
        int wf, wl;
        pieces_of(strip, wf, wl);
        lds_barrier();
        if (tid == 0) last_flag = (counter_arrive(&p.counters[strip]) == (uint32_t)(wl - wf)) ? 1u : 0u;
        lds_barrier();
        return last_flag != 0;
    };
    // the last arriver: every piece, added in K order (all loads of a batch issued before any
    // add), written as bf16; the counter goes back to zero for the next launch. With own_in_acc
    // this workgroup's own piece is still in acc (the strip its range ends in) and is not read
    // back: the stored copy holds the same bits.
    auto reduce = [&](int strip, bool own_in_acc) {
        int wf, wl;
        pieces_of(strip, wf, wl);
        if (tid == 0) counter_reset(&p.counters[strip]);
        // a piece's slot: pieces after the first start their range inside the strip (slot 0);
        // the first piece's range starts there too only if it starts at the strip's first unit
        const int seg_first = (range_begin(p.split, wf) == strip * p.ks) ? 0 : 1;
        constexpr int PB = (32 / (TN * MT)) > 0 ? 32 / (TN * MT) : 1;
        f32x4 sum[TN][MT];
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sum[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int b0 = wf; b0 <= wl; b0 += PB) {
            f32x4 v[PB][TN][MT];
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                const int wg = b0 + q;
                const int sq = (wg == wf) ? seg_first : 0;
                const bool own = own_in_acc && wg == w;
#pragma unroll
                for (int t = 0; t < TN; ++t)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const uint32_t off = sel_off(!own && wg <= wl && 16 * mt + part_row < p.M, slot_off(wg, sq, t, mt));
                        v[q][t][mt] = bits_f4(buf_load16_dev(ws, off));
                    }
            }
            // pieces past wl read as zeros (out-of-range offsets), so adding them changes nothing;
            // the own piece (read as zeros above) comes from the registers, at its place in K order
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                const bool own = own_in_acc && b0 + q == w;
#pragma unroll
                for (int t = 0; t < TN; ++t)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) sum[t][mt] += own ? acc[t][mt] : v[q][t][mt];
            }
        }
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[t][mt] = sum[t][mt];
        store_c(strip);
    };

    // ---- the ring: STAGES - 1 units in flight while one is consumed --------------------------
    // A strip that ends inside the range (the first one the range touches, when it is shared)
    // leaves its partial stored but unannounced: waiting for the store at once would also wait
    // for every load of the ring behind it. Vector-memory operations complete in issue order, so
    // by the time the loads of unit i + STAGES (issued after the store) have landed, the store has
    // too, and the arrival is counted then. (Reading the arrival's result then waits for the loads
    // wave 0 has in flight; reading it only after the range measured slower.) Reductions wait
    // for the range's end.
    int pend = -1, pend_at = 0;  // stored, not yet counted
    int fin = -1;                // stored at the range's last unit
    int red0 = -1, red1 = -1;    // strips this workgroup completes
    int cur_strip = first_strip;  // (strip, stage) of unit i
    int cur_stage = iss_stage;
    // kept rolled: unrolled, the compiler computes every prologue unit's addresses before the
    // first load goes out
#pragma unroll 1
    for (int i = 0; i < STAGES - 1; ++i) issue_unit(i);
    for (int i = 0; i < nunits; ++i) {
        wait_vmcnt<T::LOADS * (STAGES - 2)>();  // this wave's loads for unit i have landed
        lds_barrier();    // ... and every wave's; every wave is also done reading unit i - 1
        if (pend >= 0 && i >= pend_at) {
            if (arrive(pend)) red0 = pend;
            pend = -1;
        }
        issue_unit(i + STAGES - 1);             // refills the slot unit i - 1 used
        compute_unit(i);
        const int strip = cur_strip;
        const bool strip_end = ++cur_stage == p.ks;
        if (strip_end) {
            cur_stage = 0;
            ++cur_strip;
        }
        if (i == nunits - 1 || strip_end) {  // last unit of a strip in this range
            if (strip * p.ks >= u_begin && (strip + 1) * p.ks <= u_begin + nunits) {  // all ours
                store_c(strip);
            } else {
                store_partial(strip);
                if (i == nunits - 1) {
                    fin = strip;
                } else {
                    pend = strip;
                    pend_at = i + STAGES;
                }
            }
            if (i < nunits - 1) {  // (after the range's last unit acc keeps the piece for reduce)
#pragma unroll
                for (int t = 0; t < TN; ++t)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{};
            }
        }
    }
    wait_vmcnt<0>();  // every load and partial store of this wave has completed
    if (pend >= 0 && arrive(pend)) red0 = pend;
    if (fin >= 0 && arrive(fin)) red1 = fin;
    if (red1 >= 0) reduce(red1, true);  // first, while acc still holds this range's last piece
    if (red0 >= 0) reduce(red0, false);
}

template <int MT, int SW>
static hipError_t configure_one() {
    hipError_t e = hipFuncSetAttribute((const void*)skinny_gemm_kernel<MT, SW, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SkinnyTraits<MT, SW>::LAUNCH_LDS);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)skinny_gemm_kernel<MT, SW, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, SkinnyTraits<MT, SW>::LAUNCH_LDS);
    return e;
}
hipError_t configure_skinny_kernels() {
    const hipError_t es[] = {configure_one<1, 128>(), configure_one<2, 128>(), configure_one<3, 128>(),
                             configure_one<4, 128>(), configure_one<1, 256>(), configure_one<2, 256>(),
                             configure_one<3, 256>(), configure_one<4, 256>()};
    for (hipError_t e : es)
        if (e != hipSuccess) return e;
    return hipSuccess;
}
template <int SW>
static int slot_floats(int mtiles) {
    switch (mtiles) {
        case 1: return SkinnyTraits<1, SW>::SLOT_FLOATS;
        case 2: return SkinnyTraits<2, SW>::SLOT_FLOATS;
        case 3: return SkinnyTraits<3, SW>::SLOT_FLOATS;
        default: return SkinnyTraits<4, SW>::SLOT_FLOATS;
    }
}
int skinny_slot_floats(int mtiles, int strip) { return strip == 256 ? slot_floats<256>(mtiles) : slot_floats<128>(mtiles); }
template <int SW, bool GLU>
static hipError_t launch_sw(int mtiles, const SkinnyArgs& a, hipStream_t s) {
    const int grid = a.grid;
    switch (mtiles) {
        case 1: skinny_gemm_kernel<1, SW, GLU><<<grid, 256, SkinnyTraits<1, SW>::LAUNCH_LDS, s>>>(a); break;
        case 2: skinny_gemm_kernel<2, SW, GLU><<<grid, 256, SkinnyTraits<2, SW>::LAUNCH_LDS, s>>>(a); break;
        case 3: skinny_gemm_kernel<3, SW, GLU><<<grid, 256, SkinnyTraits<3, SW>::LAUNCH_LDS, s>>>(a); break;
        case 4: skinny_gemm_kernel<4, SW, GLU><<<grid, 256, SkinnyTraits<4, SW>::LAUNCH_LDS, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
hipError_t launch_skinny_gemm(int mtiles, int strip, bool glu, const SkinnyArgs& a, hipStream_t s) {
    if (glu) return strip == 256 ? launch_sw<256, true>(mtiles, a, s) : launch_sw<128, true>(mtiles, a, s);
    return strip == 256 ? launch_sw<256, false>(mtiles, a, s) : launch_sw<128, false>(mtiles, a, s);
}

}  // namespace glk
