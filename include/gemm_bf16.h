/*
 * gemm_bf16.h: C ABI of the MI355X (gfx950) bf16 matrix-multiply library.
 *
 * The library computes C = A * B with bf16 inputs, float32 accumulation and bf16 output
 * (rounded to nearest, ties to even). This is the product the spark-kernels post builds up in
 * "the bf16 gemm" (a 4096^3 GEMM in bf16 with fp32 accumulation, then the Llama-7B MLP shapes
 * and decode shapes) and that "The kernels that were there" specialises in "The GEMV" for
 * M = 1 or 2 (fp32 accumulate, bf16 store).
 *
 * Layout (all row-major, element type bf16 = 16-bit bfloat16 bit patterns):
 *   A  M x K, element (i, k) at A[i * lda + k], lda >= K
 *   B  K x N, element (k, j) at B[k * ldb + j], ldb >= N
 *   C  M x N, element (i, j) at C[i * ldc + j], ldc >= N, fully overwritten (no alpha/beta)
 * A, B and C are device pointers owned by the caller; the library never allocates, frees or
 * retains them. C must not overlap A or B.
 *
 * Every function is extern "C", returns an int status (gemm_status_t) and never throws.
 * Argument errors are detected on the host before any HIP call, so they are reported even on
 * a machine without a GPU. Compute calls only enqueue work on the caller's stream (never the
 * null stream unless the caller passes it) and return without synchronising; this is what lets
 * a caller capture them into a graph ("The kernels that were there", "The bench that lied":
 * the launch has to go to the stream being captured).
 */
#ifndef GEMM_BF16_H
#define GEMM_BF16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *gemm_stream_t; /* the same type as hipStream_t */

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,     /* bad dimension, leading dimension, null pointer */
    GEMM_ERR_UNSUPPORTED = 2,     /* e.g. M > 64 on the skinny entry point */
    GEMM_ERR_NOT_INITIALIZED = 3, /* compute call before gemm_init on this device */
    GEMM_ERR_HIP = 4              /* a HIP runtime call or kernel launch failed */
} gemm_status_t;

/*
 * gemm_init: prepare the library for HIP device `device`: queries the device's compute-unit
 * count and XCD count for the planner ("Kernel development on sm_120", section 1: query every
 * hardware number rather than hard-coding it) and sets the kernels' LDS limits. Allocates no
 * workspace: each stream gets its own region on its first call that needs one (see gemm_bf16).
 * Call it outside graph capture, before the first compute call on that device. Calling it again
 * for an initialised device is a no-op. Returns GEMM_ERR_INVALID_ARG for a negative device
 * number and GEMM_ERR_HIP when the device cannot be used.
 */
int gemm_init(int device);

/*
 * gemm_bf16: C = A * B (bf16 in, float32 accumulate, bf16 out, round to nearest even).
 * Dispatch: M <= 64 runs the skinny weight-streaming kernel (the decode shapes of the
 * spark-kernels post, "the decode kernel"); larger M runs the large-tile MFMA kernel with a tile
 * and schedule chosen per call from the shape and the device's compute-unit count ("1024 cubed
 * and the decode shapes": the launch picks the tile per call). Operands whose pointers are not
 * 16-byte aligned, or whose N, K, lda, ldb, ldc are not multiples of 8, take a general kernel
 * with the same result contract. When the large tiles would leave a last wave at most half full,
 * the product is cut into a rectangle of whole waves and the strip left over, each planned on its
 * own and launched in turn on `stream` (two kernels, no host work between them): "Kernel
 * development on sm_120", section 4, wave quantization of the last wave.
 * M == 0 or N == 0: nothing is launched. K == 0: C is set to zero (the empty sum).
 * Errors: GEMM_ERR_INVALID_ARG for negative sizes, lda < K, ldb < N, ldc < N, or a null
 * pointer with a non-empty extent; GEMM_ERR_NOT_INITIALIZED before gemm_init; GEMM_ERR_HIP if a
 * launch fails. The call is deterministic: the same inputs give the same bits on every run.
 * Workspace: split layouts sum float32 partials in K order through slots and arrival counters
 * that the kernel itself returns to zero, so a call needs no memset (spark-kernels post,
 * "stream-k proper": nothing cleared between launches; "the decode kernel": the last slice
 * resets the workspace, so no clearing launch is needed). The slots and counters live in a
 * region per (device, stream), made on the stream's first call that needs one (hipMalloc, plus a
 * clear on a library-private stream that is waited for, so that even a first call inside a graph
 * capture records only the product's kernels). Calls on different streams therefore never share
 * partials and may run concurrently; calls on one stream run in order. A captured graph keeps
 * using the region of the stream it was captured on, so it must not be replayed concurrently
 * with calls on that stream. At most 64 streams per device get a region; a call on a further
 * stream that needs one returns GEMM_ERR_UNSUPPORTED.
 */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const void *A, int64_t lda,
              const void *B, int64_t ldb,
              void *C, int64_t ldc,
              gemm_stream_t stream);

/*
 * gemm_bf16_noalloc: gemm_bf16 for callers that cannot allocate device memory (code under graph
 * capture that must not make a workspace, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, plan, kernels and bits as gemm_bf16, but the split partials and arrival counters
 * live in a fixed library array of 32 MiB of float32 slots plus 16384 counters per GPU, held from
 * the library's load until the process ends, instead of the stream's workspace region; the call
 * never allocates or frees. gemm_init must have run on the device. A plan whose partials or
 * counters exceed that array returns GEMM_ERR_UNSUPPORTED (on 256 CUs none does: the largest
 * split plan needs exactly 8 Mi floats, 512 pieces of a 128 x 128 tile, and the fast kernels
 * take at most 2^20 columns, 8192 strips). Every call on one GPU shares the one array:
 * calls that overlap in time on that GPU, on any streams, race and must be serialised by the
 * caller. Counters return to zero at the end of every call.
 */
int gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda,
                      const void *B, int64_t ldb,
                      void *C, int64_t ldc,
                      gemm_stream_t stream);

/*
 * gemm_bf16_skinny: the same product, forced onto the skinny kernel: every byte of B is read
 * once for all M rows ("The kernels that were there", "The GEMV": the M = 2 kernel loads each
 * weight once for both rows; spark-kernels "the decode kernel"). Requires 1 <= M <= 64
 * (GEMM_ERR_UNSUPPORTED otherwise); same layout, errors and semantics as gemm_bf16.
 */
int gemm_bf16_skinny(int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda,
                     const void *B, int64_t ldb,
                     void *C, int64_t ldc,
                     gemm_stream_t stream);

/*
 * gemm_bf16_tiled: the same product, forced onto the large-tile MFMA kernel family (any M >= 1),
 * for comparisons and tests. Same layout, errors and semantics as gemm_bf16.
 */
int gemm_bf16_tiled(int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda,
                    const void *B, int64_t ldb,
                    void *C, int64_t ldc,
                    gemm_stream_t stream);

/*
 * gemm_bf16_swiglu: the gate and up projections of a Llama MLP and their SwiGLU in one call:
 *   C = silu(A * Wg) .* (A * Wu),   silu(x) = x / (1 + e^-x),   .* element by element,
 * where Wg and Wu are the two halves of one K x 2N weight B: columns 0 .. N-1 are Wg and
 * columns N .. 2N-1 are Wu (gate and up concatenated along the output dimension). SwiGLU is
 * silu of the gate times the up projection (spark-kernels post, "the memory-bound kernels",
 * where it is one kernel instead of PyTorch's two); here it runs in the epilogue of the product
 * that makes g and u, so g and u stay float32 accumulators and only C is rounded to bf16 (round
 * to nearest even), once.
 * Layout: A M x K (lda >= K), B K x 2N (ldb >= 2N), C M x N (ldc >= N), row-major bf16, device
 * pointers owned by the caller; C must not overlap A or B.
 * Dispatch as gemm_bf16: M <= 64 streams B once with the skinny kernel, larger M runs the
 * large-tile kernel; operands the fast kernels cannot take (alignment, N, K or leading
 * dimensions not multiples of 8) run a general kernel with the same contract.
 * M == 0 or N == 0: nothing is launched. K == 0: C is set to zero (silu(0) * 0).
 * Errors: GEMM_ERR_INVALID_ARG for negative sizes, lda < K, ldb < 2N, ldc < N, or a null pointer
 * with a non-empty extent; GEMM_ERR_NOT_INITIALIZED before gemm_init; GEMM_ERR_HIP if a launch
 * fails. Deterministic, enqueued on `stream` without synchronising (capturable), and using the
 * stream's workspace region like gemm_bf16.
 */
int gemm_bf16_swiglu(int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda,
                     const void *B, int64_t ldb,
                     void *C, int64_t ldc,
                     gemm_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Block-scaled (MX) decode: the decode product with weights in MXFP4 and activations in MXFP8,
 * on gfx950's scaled matrix instructions. Formats are those of the OCP Microscaling (MX)
 * specification v1.0: a block of 32 consecutive elements along K shares one E8M0 scale byte e
 * (value 2^(e - 127)); elements are E2M1 (FP4: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives) or E4M3
 * (FP8, largest 448). The weights are the bytes that bound decode (spark-kernels post, "the
 * decode kernel"); in MXFP4 they take 0.53 bytes per element instead of bf16's 2. The pages
 * measure block-scaled GEMMs on pre-quantized operands ("Benchmarks" page of gemm3,
 * "Implementations"); here the conversions are entry points of their own.
 * Conversion of a block (both formats): shared exponent floor(log2(max |v|)) - emax (emax 2 for
 * E2M1, 8 for E4M3), clamped to [-127, 127]; elements v / 2^exponent rounded to the element
 * format, nearest with ties to even, saturating at its largest magnitude; an all-zero block
 * gets scale byte 0. Deterministic, bit for bit.
 * ------------------------------------------------------------------------------------------ */

/*
 * gemm_mx_packed_sizes: host-only. Bytes of the packed MXFP4 weight codes (*wp_bytes) and scales
 * (*sp_bytes) of an N x K weight. Requires N % 16 == 0 and K % 128 == 0 (GEMM_ERR_INVALID_ARG
 * otherwise); GEMM_ERR_UNSUPPORTED when either exceeds 2^31 - 1 bytes.
 */
int gemm_mx_packed_sizes(int64_t N, int64_t K, int64_t *wp_bytes, int64_t *sp_bytes);

/*
 * gemm_mx_pack_weight: converts a bf16 weight W (N x K row-major, the nn.Linear layout: row n
 * holds the K inputs of output n; ldw >= K, ldw % 8 == 0, W 16-byte aligned) to MXFP4 in the
 * packed layout the decode product reads (Wp 16-byte aligned, Sp; sizes from
 * gemm_mx_packed_sizes; both device memory owned by the caller). Layout: column tile t (rows
 * 16 t .. 16 t + 15) and k-step s (k = 128 s .. 128 s + 127) are the 1024 bytes at
 * Wp + 1024 (t * K/128 + s); in them bytes 16 l .. 16 l + 15 (l = 0 .. 63) hold the codes of row
 * 16 t + l % 16 at k = 128 s + 32 (l / 16) + j, j = 0 .. 31, two per byte, even j in the low
 * nibble. The scale of that 32-element block is Sp[256 (t * ceil(K/512) + s / 4) + 4 l + s % 4];
 * scale bytes of k-steps past K / 128 are zero. Run once per weight, outside the decode loop.
 */
int gemm_mx_pack_weight(int64_t N, int64_t K, const void *W, int64_t ldw, void *Wp, void *Sp,
                        gemm_stream_t stream);

/*
 * gemm_mx_quantize_act: converts bf16 activations A (M x K, lda >= K, lda % 8 == 0, 16-byte
 * aligned) to MXFP8 (E4M3) codes Aq (M x K bytes row-major, ldaq >= K, ldaq % 16 == 0, 16-byte
 * aligned) and scales As (M x K/32 bytes, ldas >= K/32). K % 32 == 0.
 */
int gemm_mx_quantize_act(int64_t M, int64_t K, const void *A, int64_t lda, void *Aq, int64_t ldaq,
                         void *As, int64_t ldas, gemm_stream_t stream);

/*
 * gemm_mx_decode: C = deq(Aq) * deq(W)^T, float32 accumulation, bf16 output (round to nearest
 * even): C[m][n] = sum_k a[m][k] w[n][k] over the dequantised MXFP8 activations (layout of
 * gemm_mx_quantize_act) and MXFP4 weights (packed by gemm_mx_pack_weight). C is M x N bf16
 * (ldc >= N, ldc % 4 == 0, 8-byte aligned). Requires M <= 64, N % 16 == 0, K % 128 == 0
 * (GEMM_ERR_UNSUPPORTED otherwise). M == 0 or N == 0: nothing; K == 0: C = 0. One launch;
 * deterministic; uses the stream's workspace region like gemm_bf16.
 */
int gemm_mx_decode(int64_t M, int64_t N, int64_t K, const void *Aq, int64_t ldaq, const void *As,
                   int64_t ldas, const void *Wp, const void *Sp, void *C, int64_t ldc,
                   gemm_stream_t stream);

/*
 * gemm_mx_decode_bf16: gemm_mx_quantize_act into the library's workspace, then gemm_mx_decode
 * (two launches on `stream`; for M <= 2 one launch that converts inside the product): the decode
 * product from bf16 activations A (M x K, lda >= K, lda % 8 == 0, 16-byte aligned) and packed MXFP4
 * weights. The quantised activations go to the tail of the stream's workspace region. Same
 * requirements and results as the two calls.
 */
int gemm_mx_decode_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *Wp,
                        const void *Sp, void *C, int64_t ldc, gemm_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Decode on a packed bf16 weight: the decode product is a stream of weight bytes read once
 * (spark-kernels post, "the decode kernel"); a weight that does not change between calls can be
 * stored once in the order the matrix instructions consume it, so the product needs no staging
 * through LDS. Same arithmetic and results contract as gemm_bf16 (bf16 in, float32 accumulation,
 * bf16 out, round to nearest even).
 * ------------------------------------------------------------------------------------------ */

/*
 * gemm_pack_weight_bf16: writes the K x N bf16 weight B (row-major, ldb >= N, the layout of
 * gemm_bf16's B) into Bp (device memory of K * N * 2 bytes owned by the caller, 16-byte aligned)
 * in the packed layout: column tile t (columns 16 t .. 16 t + 15) and k-step s (rows 32 s .. 32 s +
 * 31) are the 1024 bytes at Bp + 1024 (t * K/32 + s); in them bytes 16 l .. 16 l + 15 (l = 0 .. 63)
 * hold B[32 s + 8 (l / 16) + j][16 t + l % 16], j = 0 .. 7. Requires K % 32 == 0 and N % 16 == 0
 * (GEMM_ERR_INVALID_ARG otherwise); GEMM_ERR_UNSUPPORTED beyond 2^31 - 1 bytes. Run once per weight.
 */
int gemm_pack_weight_bf16(int64_t K, int64_t N, const void *B, int64_t ldb, void *Bp,
                          gemm_stream_t stream);

/*
 * gemm_bf16_packed: C = A * B for 1 <= M <= 64 with B packed by gemm_pack_weight_bf16. A is M x K
 * bf16 (lda >= K, lda % 8 == 0, 16-byte aligned), C is M x N bf16 (ldc >= N, ldc % 4 == 0, 8-byte
 * aligned). Requires M <= 64, N % 16 == 0, K % 32 == 0 (GEMM_ERR_UNSUPPORTED otherwise).
 * M == 0 or N == 0: nothing; K == 0: C = 0. One launch; deterministic; uses the stream's
 * workspace region like gemm_bf16.
 */
int gemm_bf16_packed(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *Bp,
                     void *C, int64_t ldc, gemm_stream_t stream);

/* Flags of gemm_plan_describe. */
#define GEMM_PLAN_SKINNY 1 /* the plan of gemm_bf16_skinny */
#define GEMM_PLAN_SWIGLU 2 /* the plan of gemm_bf16_swiglu (with GEMM_PLAN_SKINNY: its skinny form) */
#define GEMM_PLAN_MX 4     /* the plan of gemm_mx_decode (alone) */
#define GEMM_PLAN_PACKED 8 /* the plan of gemm_bf16_packed (alone) */

/*
 * gemm_plan_describe: host-only. Writes, as a JSON object, the plan the library would use for an
 * M x N x K product on a device with `cus` compute units (tile, grid, schedule, split count,
 * wave count and wave efficiency = (tiles/slots)/ceil(tiles/slots), the quantity of "Kernel
 * development on sm_120", section 4, budget 4; "nxcd": 1 where workgroups keep the hardware's
 * round-robin XCD order, else the XCD count the tile order is remapped over; for a product cut
 * in two, "cut": the axis, the offset and the rest's own plan). `flags` is 0 for gemm_bf16, a combination of
 * GEMM_PLAN_SKINNY and GEMM_PLAN_SWIGLU, or GEMM_PLAN_MX or GEMM_PLAN_PACKED alone. Touches no HIP state. Returns
 * GEMM_ERR_INVALID_ARG for bad sizes, unknown flags or a buffer too small (buf is always
 * NUL-terminated when len > 0), GEMM_ERR_UNSUPPORTED for GEMM_PLAN_SKINNY with M outside 1 .. 64
 * or GEMM_PLAN_MX / GEMM_PLAN_PACKED outside their entry points' shapes.
 */
int gemm_plan_describe(int64_t M, int64_t N, int64_t K, int cus, int flags, char *buf, int len);

/*
 * gemm_wave_efficiency: host-only closed form of "Kernel development on sm_120", section 4,
 * budget 4: with `ctas` workgroups over `slots` concurrent slots,
 * (ctas / slots) / ceil(ctas / slots). Writes the efficiency and the wave count.
 */
int gemm_wave_efficiency(int64_t ctas, int64_t slots, double *efficiency, int64_t *waves);

/*
 * gemm_last_plan: the JSON plan (the same fields as gemm_plan_describe) of the last successful
 * compute call in this process, any device or stream, copied into buf (len bytes, always
 * NUL-terminated when len > 0). The plan is chosen per call from the shape and the device, so
 * this is how a benchmark or test reads which kernel, tile and split a call took (spark-kernels
 * post, "1024 cubed and the decode shapes": the launch picks the tile per call). Host-only; touches
 * no HIP state. GEMM_ERR_INVALID_ARG for a null buf, len <= 0, or a plan longer than len - 1
 * (buf then holds the truncated text).
 */
int gemm_last_plan(char *buf, int len);

/*
 * gemm_status_string: a static, human-readable name for a status code ("GEMM_ERR_UNKNOWN" for a
 * value outside gemm_status_t). Every entry point returns a status and never throws, so that a
 * benchmark or test reports a refused or failed call by name instead of timing it as if it had
 * run ("Kernel development on sm_120", section 6, "Benchmarking": the benchmark is audited as
 * carefully as the kernel, since several of that repository's bugs were benchmark bugs). Never
 * null; the caller must not free it.
 */
const char *gemm_status_string(int status);

/*
 * gemm_finalize: frees every stream's workspace region and the private stream of every
 * initialised device, and returns the devices to the uninitialised state (gemm_init may be called
 * again). The workspaces are the library's only allocations, the ones gemm_init's contract says
 * the library owns (spark-kernels post, "stream-k proper" and "the decode kernel": partial slots
 * and counters that persist between launches instead of being cleared per call). Call it outside
 * graph capture, after every stream that used the library has drained and after any graph that
 * holds its kernels has been destroyed. GEMM_ERR_HIP if a free fails (the rest are still freed).
 */
int gemm_finalize(void);

/* ------------------------------------------------------------------------------------------
 * Measurement kernels: the card's own roofs, measured rather than quoted (spark-kernels post,
 * "how things are measured": a loop of register-resident matrix instructions and a device copy;
 * "the decode kernel": a read-only kernel with 16-byte loads, an empty launch, single launch vs
 * back to back; "Kernel development on sm_120", section 1: measure peak DRAM bandwidth and peak
 * matmul rate, never derive them). All enqueue on `stream` and return immediately.
 * ------------------------------------------------------------------------------------------ */

/*
 * gemm_peak_mfma_launch: `blocks` workgroups of 256 threads each run `iters` iterations of
 * 8 independent v_mfma_f32_32x32x16_bf16 chains on register-resident operands per wave
 * (16 * 32^3 flops per instruction; flops = blocks * 4 waves * iters * 8 * 32768).
 * `sink` (device, >= blocks * 256 floats) receives a reduction of the accumulators so the work
 * cannot be removed; `cycles` (device, >= 2 * blocks uint64) receives, per block, the
 * s_memtime delta (shader clock cycles) and the s_memrealtime delta (100 MHz constant clock)
 * measured by wave 0 around its loop.
 */
int gemm_peak_mfma_launch(int64_t iters, int blocks, float *sink, uint64_t *cycles,
                          gemm_stream_t stream);

/*
 * gemm_peak_mfma_data_launch: the matrix-core rate on operands from memory. `blocks` workgroups
 * of 512 threads (8 waves, 2 per SIMD) each run `iters` iterations of 32 v_mfma_f32_16x16x32_bf16
 * per wave into 128 float accumulators per lane (the large-tile kernel's wave-tile layout), on
 * 8 A and 4 B operand registers per lane loaded once from `ops` (device, 16-byte aligned, at
 * least 3072 * 16 = 49152 bytes: lane t of the workgroup reads 16-byte words (q * 512 + t) % 2048
 * for A register q and 2048 + (q * 512 + t) % 1024 for B register q). flops = blocks * 8 waves *
 * iters * 32 * 16384. `sink` (device, >= blocks * 512 floats) and `cycles` (device, >= 2 *
 * blocks uint64) as for gemm_peak_mfma_launch. Random operands measure the ceiling the board's
 * power limit leaves for products of random data (the register-only loop's near-constant
 * operands toggle few bits and measure the clock-limited ceiling).
 */
int gemm_peak_mfma_data_launch(const void *ops, int64_t iters, int blocks, float *sink,
                               uint64_t *cycles, gemm_stream_t stream);

/* gemm_peak_copy_launch: dst[0 .. bytes) = src[0 .. bytes) with 16-byte loads and stores;
 * bytes must be a multiple of 16 and both pointers 16-byte aligned. HBM traffic = 2 * bytes. */
int gemm_peak_copy_launch(const void *src, void *dst, int64_t bytes, gemm_stream_t stream);

/* gemm_peak_read_launch: reads src[0 .. bytes) with 16-byte loads and writes one 32-bit value
 * per workgroup to sink (device, >= 65536 uint32) so the loads are kept. bytes % 16 == 0. */
int gemm_peak_read_launch(const void *src, int64_t bytes, uint32_t *sink, gemm_stream_t stream);

/* gemm_peak_empty_launch: one workgroup that does nothing (launch floor). */
int gemm_peak_empty_launch(gemm_stream_t stream);

/*
 * gemm_peak_clock_launch: `blocks` workgroups of one wave each run `iters` dependent fp32 FMAs;
 * `out` (device, >= 2 * blocks uint64) receives, per block, the s_memtime delta (shader clock
 * cycles) and the s_memrealtime delta (100 MHz constant clock) around the loop. Enqueued right
 * after other work on the same stream it reads the shader clock the card held under that work
 * (the clock changes over milliseconds, the probe lasts microseconds).
 */
int gemm_peak_clock_launch(int64_t iters, int blocks, uint64_t *out, gemm_stream_t stream);

/*
 * gemm_peak_xcc_launch: `blocks` workgroups of one wave each write, to out[b] (device, >= blocks
 * uint32), the index of the XCD (accelerator complex die) that workgroup b ran on. The planner's
 * tile and strip orders assume consecutive workgroups are dealt to the XCDs round robin, each
 * XCD with its own L2; this measures the assumption instead of quoting it ("Kernel development on
 * sm_120", section 1: query or measure every hardware number).
 */
int gemm_peak_xcc_launch(int blocks, uint32_t *out, gemm_stream_t stream);

/* gemm_fill_launch: writes the 32-bit `value` over dst[0 .. bytes) (bytes % 4 == 0); used to
 * evict the device's caches between timed calls and to poison outputs before checks. */
int gemm_fill_launch(void *dst, int64_t bytes, uint32_t value, gemm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_BF16_H */
