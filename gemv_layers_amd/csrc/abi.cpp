// The library's C ABI (declared in include/gemm_bf16.h): argument validation on the host before
// any HIP call, per-device state and workspace, planning and dispatch onto the caller's stream.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "gemm_bf16.h"
#include "kernels.h"
#include "plan.h"

namespace {

constexpr int kMaxDevices = 64;
// Workspace region, one per (device, stream): float32 partial slots for split tiles / K slices,
// and their arrival counters. On 256 CUs no plan needs more than 8 Mi floats of partials (32 MiB:
// 512 split pieces of a 128 x 128 tile, two per CU; the skinny kernel's two 16 x 64 x 128 slots
// per workgroup take 4 Mi).
constexpr int64_t kWsFloats = int64_t(8) << 20;   // 32 MiB
constexpr int64_t kWsCounters = int64_t(1) << 16;
// The last 16 MiB of a region hold the MXFP8 activations that gemm_mx_decode_bf16 quantises
// before its product; MX plans keep their partial slots below them.
constexpr int64_t kMxActBytes = int64_t(16) << 20;
constexpr int64_t kMxPartialFloats = kWsFloats - kMxActBytes / 4;
// Streams with a region of their own, per device. A further stream gets GEMM_ERR_UNSUPPORTED.
constexpr int kMaxStreams = 64;

// One stream's workspace. Its counters start at zero (cleared when the region is made) and every
// kernel that uses them returns them to zero, so the region is never cleared again.
struct Region {
    hipStream_t stream = nullptr;
    float* ws = nullptr;
    uint32_t* counters = nullptr;
};

// Workspace of gemm_bf16_noalloc, for callers that cannot allocate: a file-scope device array
// (each GPU the library runs on holds its own copy until the process ends), arrival counters
// first, then float32 partial slots. 8 Mi floats hold the largest split plan on 256 CUs.
constexpr int64_t kScratchCounters = int64_t(1) << 14;   // 64 KiB
constexpr int64_t kScratchFloats = int64_t(8) << 20;     // 32 MiB
static __device__ __align__(256) uint32_t scratch[kScratchCounters + kScratchFloats];

struct DeviceState {
    // set (release) by gemm_init once the rest of the state is written; compute calls read it
    // (acquire) without taking the lock
    std::atomic<bool> ready{false};
    glk::DeviceInfo info;
    std::mutex mu;             // guards the region table
    Region regions[kMaxStreams];
    int nregions = 0;
    hipStream_t clear_stream = nullptr;  // library-private: clears the counters of new regions
    // this device's copy of `scratch`, as a device address (from hipGetSymbolAddress: in host
    // code the array's own name is not a device address)
    uint32_t* scratch_ptr = nullptr;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];
std::atomic<int> g_ready_count{0};
std::string g_last_plan = "{}";

// The workspace region of `stream` on the device of `ds` (the current device), made on the
// stream's first call that needs one. Split partials and counters of concurrent calls on
// different streams then never meet; calls on one stream run in order and share its region.
// A region is made with hipMalloc in the relaxed capture mode, so that a first call inside a
// graph capture can still make it: the allocation is not a stream operation, and the counters
// are cleared on a library-private stream and waited for before the call enqueues anything, so
// the capture records no memset. A captured graph keeps using the region of the stream it was
// captured on.
int region_for(DeviceState& ds, hipStream_t stream, Region** out) {
    std::lock_guard<std::mutex> lk(ds.mu);
    for (int i = 0; i < ds.nregions; ++i) {
        if (ds.regions[i].stream == stream) {
            *out = &ds.regions[i];
            return GEMM_OK;
        }
    }
    if (ds.nregions == kMaxStreams) return GEMM_ERR_UNSUPPORTED;
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    if (hipThreadExchangeStreamCaptureMode(&mode) != hipSuccess) return GEMM_ERR_HIP;
    const size_t cbytes = kWsCounters * sizeof(uint32_t);
    void* mem = nullptr;
    int rc = GEMM_OK;
    if (hipMalloc(&mem, cbytes + kWsFloats * sizeof(float)) != hipSuccess) {
        mem = nullptr;
        rc = GEMM_ERR_HIP;
    }
    if (rc == GEMM_OK && (hipMemsetAsync(mem, 0, cbytes, ds.clear_stream) != hipSuccess ||
                          hipStreamSynchronize(ds.clear_stream) != hipSuccess))
        rc = GEMM_ERR_HIP;
    if (rc != GEMM_OK && mem) hipFree(mem);
    hipThreadExchangeStreamCaptureMode(&mode);
    if (rc != GEMM_OK) return rc;
    Region& r = ds.regions[ds.nregions];
    r.stream = stream;
    r.counters = static_cast<uint32_t*>(mem);
    r.ws = reinterpret_cast<float*>(static_cast<char*>(mem) + cbytes);
    ++ds.nregions;
    *out = &r;
    return GEMM_OK;
}

int copy_out(const std::string& s, char* buf, int len) {
    if (!buf || len <= 0) return GEMM_ERR_INVALID_ARG;
    const size_t n = s.size();
    if (n + 1 > (size_t)len) {
        memcpy(buf, s.data(), (size_t)len - 1);
        buf[len - 1] = '\0';
        return GEMM_ERR_INVALID_ARG;
    }
    memcpy(buf, s.c_str(), n + 1);
    return GEMM_OK;
}

// glu: B holds 2N columns (gate, then up)
int validate(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
             int64_t ldb, const void* C, int64_t ldc, bool glu) {
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
    if (glu && N > INT64_MAX / 2) return GEMM_ERR_INVALID_ARG;
    if (ldc < N || ldc < 0) return GEMM_ERR_INVALID_ARG;
    if (lda < K || ldb < (glu ? 2 * N : N)) return GEMM_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && C == nullptr) return GEMM_ERR_INVALID_ARG;
    if (M > 0 && K > 0 && A == nullptr) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && N > 0 && B == nullptr) return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

// one launch of the large-tile kernel family for plan `p` over an M x N output (N outputs, 2N weight
// columns in the SwiGLU form)
hipError_t launch_tile_plan(const glk::Plan& p, int64_t M, int64_t N, int64_t K, const uint16_t* a16,
                            int64_t lda, const uint16_t* b16, int64_t ldb, uint16_t* c16, int64_t ldc,
                            bool glu, const Region* rg, hipStream_t stream) {
    glk::TileArgs t;
    t.A = a16;
    t.B = b16;
    t.C = c16;
    t.M = (int)M;
    t.N = (int)N;
    t.K = (int)K;
    t.lda = (int)lda;
    t.ldb = (int)ldb;
    t.ldc = (int)ldc;
    t.tiles_m = (int)p.tiles_m;
    t.tiles_n = (int)p.tiles_n;
    t.group_m = p.group_m;
    t.nxcd = p.nxcd;
    t.sched = p.sched;
    t.splits = p.splits;
    t.kt_per_split = p.kt_per_split;
    t.ws = rg->ws;
    t.counters = rg->counters;
    return glk::launch_tile_gemm(p.tile_cfg, t, (int)p.grid, glu, stream);
}

// force: 0 dispatch on M, 1 skinny, 2 large-tile family; glu: the SwiGLU form; noalloc: split
// partials and counters in the device's scratch array instead of the stream's region
int run(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
        void* C, int64_t ldc, hipStream_t stream, int force, bool glu = false, bool noalloc = false) {
    int st = validate(M, N, K, A, lda, B, ldb, C, ldc, glu);
    if (st != GEMM_OK) return st;
    if (force == 1 && (M < 1 || M > 64)) return GEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GEMM_OK;
    if (g_ready_count == 0) return GEMM_ERR_NOT_INITIALIZED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_ERR_HIP;
    DeviceState& ds = g_dev[dev];
    if (!ds.ready.load(std::memory_order_acquire)) return GEMM_ERR_NOT_INITIALIZED;

    // (the SwiGLU form's up half starts N columns in: N % 8 == 0 keeps it 16-byte aligned)
    const bool fast = glk::fast_path_ok(M, glu ? 2 * N : N, K, A, lda, B, ldb, C, ldc) &&
                      glk::fast_path_ok(M, N, K, A, lda, B, ldb, C, ldc);
    const glk::Plan p = glk::make_plan(M, N, K, ds.info, fast, force, glu);
    // (no buffer that fits in device memory gets here; the launch takes a 32-bit grid)
    if (p.grid > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    Region* rg = nullptr;
    Region fixed;
    if (p.kernel == glk::kKernTile || p.kernel == glk::kKernSkinny) {
        if (noalloc) {
            // the plan is gemm_bf16's own (same bits); one whose partials or counters do not fit
            // the scratch array is refused rather than changed
            if (p.ws_floats > kScratchFloats || p.counters > kScratchCounters) return GEMM_ERR_UNSUPPORTED;
            fixed.counters = ds.scratch_ptr;
            fixed.ws = reinterpret_cast<float*>(ds.scratch_ptr + kScratchCounters);
            rg = &fixed;
        } else {
            st = region_for(ds, stream, &rg);
            if (st != GEMM_OK) return st;
        }
    }
    const uint16_t* a16 = static_cast<const uint16_t*>(A);
    const uint16_t* b16 = static_cast<const uint16_t*>(B);
    uint16_t* c16 = static_cast<uint16_t*>(C);
    hipError_t e = hipSuccess;
    switch (p.kernel) {
        case glk::kKernNone:
            break;
        case glk::kKernZero:
            e = glk::launch_zero_c(c16, M, N, ldc, stream);
            break;
        case glk::kKernGeneric:
            e = glk::launch_generic_gemm(a16, b16, c16, M, N, K, lda, ldb, ldc, glu, stream);
            break;
        case glk::kKernTile: {
            // a cut plan covers the first cut_at columns (axis 1) or rows (axis 2); the strip left
            // over runs next on the same stream with its own plan (only it may use the workspace)
            const int64_t Mm = p.cut_axis == 2 ? p.cut_at : M;
            const int64_t Nm = p.cut_axis == 1 ? p.cut_at : N;
            e = launch_tile_plan(p, Mm, Nm, K, a16, lda, b16, ldb, c16, ldc, glu, rg, stream);
            if (e == hipSuccess && p.cut_axis != 0) {
                const glk::Plan& r = p.rest[0];
                if (p.cut_axis == 1)
                    e = launch_tile_plan(r, M, N - p.cut_at, K, a16, lda, b16 + p.cut_at, ldb, c16 + p.cut_at,
                                         ldc, glu, rg, stream);
                else
                    e = launch_tile_plan(r, M - p.cut_at, N, K, a16 + p.cut_at * lda, lda, b16, ldb,
                                         c16 + p.cut_at * ldc, ldc, glu, rg, stream);
            }
            break;
        }
        case glk::kKernSkinny: {
            glk::SkinnyArgs s;
            s.A = a16;
            s.B = b16;
            s.C = c16;
            s.M = (int)M;
            s.N = (int)N;
            s.K = (int)K;
            s.lda = (int)lda;
            s.ldb = (int)ldb;
            s.ldc = (int)ldc;
            s.strips = p.strips;
            s.ks = p.ks;
            s.grid = (int)p.grid;
            s.split = glk::make_unit_split(p.strips * p.ks, (int)p.grid);
            s.nxcd = p.nxcd;
            s.ws = rg->ws;
            s.counters = rg->counters;
            e = glk::launch_skinny_gemm(p.mtiles, p.strip, glu, s, stream);
            break;
        }
        default:
            return GEMM_ERR_UNSUPPORTED;
    }
    if (e != hipSuccess) return GEMM_ERR_HIP;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        g_last_plan = glk::plan_json(p, M, N, K);
    }
    return GEMM_OK;
}

}  // namespace

// ---- block-scaled (MX) decode -------------------------------------------------------------------

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// the device state of the current device, or nullptr
DeviceState* current_state(int* status) {
    if (g_ready_count == 0) {
        *status = GEMM_ERR_NOT_INITIALIZED;
        return nullptr;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = GEMM_ERR_HIP;
        return nullptr;
    }
    if (!g_dev[dev].ready.load(std::memory_order_acquire)) {
        *status = GEMM_ERR_NOT_INITIALIZED;
        return nullptr;
    }
    return &g_dev[dev];
}

int mx_packed(int64_t N, int64_t K, int64_t* wbytes, int64_t* sbytes) {
    if (N < 0 || K < 0 || (N % 16) || (K % 128)) return GEMM_ERR_INVALID_ARG;
    const int64_t ks = K / 128, kq = (ks + 3) / 4;
    *wbytes = (N / 16) * ks * 1024;
    *sbytes = (N / 16) * kq * 256;
    if (*wbytes > INT32_MAX || *sbytes > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    return GEMM_OK;
}

int mx_quantize_act(int64_t M, int64_t K, const void* A, int64_t lda, void* Aq, int64_t ldaq, void* As,
                    int64_t ldas, hipStream_t stream) {
    if (M < 0 || K < 0 || (K % 32) || lda < K || ldaq < K || ldas < K / 32) return GEMM_ERR_INVALID_ARG;
    if (M > 0 && K > 0 && (!A || !Aq || !As)) return GEMM_ERR_INVALID_ARG;
    if (!aligned(A, 16) || !aligned(Aq, 16) || (lda % 8) || (ldaq % 16)) return GEMM_ERR_INVALID_ARG;
    if (M > INT32_MAX || lda > INT32_MAX || ldaq > INT32_MAX || ldas > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    if (M == 0 || K == 0) return GEMM_OK;
    int st = GEMM_OK;
    if (!current_state(&st)) return st;
    return glk::launch_mx_quant(false, static_cast<const uint16_t*>(A), (int)M, (int)K, (int)lda,
                                static_cast<uint8_t*>(Aq), (int)ldaq, static_cast<uint8_t*>(As), (int)ldas,
                                stream) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

// fused: A16 (bf16 activations, lda16) is converted inside the product (M <= 2), Aq/As unused
int mx_decode(int64_t M, int64_t N, int64_t K, const void* Aq, int64_t ldaq, const void* As, int64_t ldas,
              const void* Wp, const void* Sp, void* C, int64_t ldc, hipStream_t stream,
              const void* A16 = nullptr, int64_t lda16 = 0) {
    const bool fused = A16 != nullptr;
    if (M < 0 || N < 0 || K < 0 || ldaq < K || ldas < K / 32 || ldc < N) return GEMM_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && !C) return GEMM_ERR_INVALID_ARG;
    if (!fused && M > 0 && K > 0 && (!Aq || !As)) return GEMM_ERR_INVALID_ARG;
    if (N > 0 && K > 0 && (!Wp || !Sp)) return GEMM_ERR_INVALID_ARG;
    if (M > 64 || (N % 16) || (K % 128) || (fused && M > 2)) return GEMM_ERR_UNSUPPORTED;
    if ((!fused && (!aligned(Aq, 16) || (ldaq % 16))) || !aligned(Wp, 16) || !aligned(C, 8) || (ldc % 4))
        return GEMM_ERR_INVALID_ARG;
    if (fused && (!aligned(A16, 16) || (lda16 % 8) || lda16 < K || lda16 > INT32_MAX))
        return GEMM_ERR_INVALID_ARG;
    int64_t wb = 0, sb = 0;
    int st = mx_packed(N, K, &wb, &sb);
    if (st != GEMM_OK) return st;
    if (64 * ldaq > INT32_MAX || 64 * ldas > INT32_MAX || ldc > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GEMM_OK;
    DeviceState* ds = current_state(&st);
    if (!ds) return st;
    glk::DeviceInfo info = ds->info;
    info.ws_floats = kMxPartialFloats;
    const glk::Plan p = glk::make_mx_plan(M, N, K, info);
    hipError_t e = hipSuccess;
    if (p.kernel == glk::kKernZero) {
        e = glk::launch_zero_c(static_cast<uint16_t*>(C), M, N, ldc, stream);
    } else {
        Region* rg = nullptr;
        st = region_for(*ds, stream, &rg);
        if (st != GEMM_OK) return st;
        glk::MxArgs a;
        a.Aq = static_cast<const uint8_t*>(Aq);
        a.As = static_cast<const uint8_t*>(As);
        a.Wp = static_cast<const uint8_t*>(Wp);
        a.Sp = static_cast<const uint8_t*>(Sp);
        a.C = static_cast<uint16_t*>(C);
        a.M = (int)M;
        a.N = (int)N;
        a.K = (int)K;
        a.ldaq = (int)ldaq;
        a.ldas = (int)ldas;
        a.ldc = (int)ldc;
        a.tiles = (int)(N / 16);
        a.ks = (int)(K / 128);
        a.kq = (a.ks + 3) / 4;
        a.pieces = p.splits;
        a.nxcd = p.nxcd;
        a.ws = rg->ws;
        a.counters = rg->counters;
        a.A16 = static_cast<const uint16_t*>(A16);
        a.lda16 = (int)lda16;
        a.kpb = 0;
        a.red_off = 0;
        if (fused) {
            const int piece_ks = (a.ks + p.splits - 1) / p.splits;
            const int lds = glk::mx_fused_layout(piece_ks, p.strip / 16, a);
            if (lds < 0) return GEMM_ERR_UNSUPPORTED;
            e = glk::launch_mx_decode_fused(p.strip / 16, a, (int)p.grid, lds, stream);
        } else {
            e = glk::launch_mx_decode(p.mtiles, p.strip / 16, a, (int)p.grid, stream);
        }
    }
    if (e != hipSuccess) return GEMM_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    g_last_plan = glk::plan_json(p, M, N, K);
    return GEMM_OK;
}

// ---- decode product on a packed bf16 weight ------------------------------------------------------

int packed_decode(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* Bp, void* C,
                  int64_t ldc, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0 || lda < K || ldc < N) return GEMM_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && !C) return GEMM_ERR_INVALID_ARG;
    if (M > 0 && K > 0 && !A) return GEMM_ERR_INVALID_ARG;
    if (N > 0 && K > 0 && !Bp) return GEMM_ERR_INVALID_ARG;
    if (M > 64 || (N % 16) || (K % 32)) return GEMM_ERR_UNSUPPORTED;
    if (!aligned(A, 16) || !aligned(Bp, 16) || !aligned(C, 8) || (lda % 8) || (ldc % 4))
        return GEMM_ERR_INVALID_ARG;
    if (N * K * 2 > INT32_MAX || 64 * lda * 2 > INT32_MAX || ldc > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GEMM_OK;
    int st = GEMM_OK;
    DeviceState* ds = current_state(&st);
    if (!ds) return st;
    const glk::Plan p = glk::make_packed_plan(M, N, K, ds->info);
    hipError_t e = hipSuccess;
    if (p.kernel == glk::kKernZero) {
        e = glk::launch_zero_c(static_cast<uint16_t*>(C), M, N, ldc, stream);
    } else {
        Region* rg = nullptr;
        st = region_for(*ds, stream, &rg);
        if (st != GEMM_OK) return st;
        glk::PkArgs a;
        a.A = static_cast<const uint16_t*>(A);
        a.Bp = static_cast<const uint16_t*>(Bp);
        a.C = static_cast<uint16_t*>(C);
        a.M = (int)M;
        a.N = (int)N;
        a.K = (int)K;
        a.lda = (int)lda;
        a.ldc = (int)ldc;
        a.tiles = (int)(N / 16);
        a.ks = (int)(K / 32);
        a.pieces = p.splits;
        a.nxcd = p.nxcd;
        a.ws = rg->ws;
        a.counters = rg->counters;
        e = glk::launch_pk_decode(p.mtiles, p.strip / 16, a, (int)p.grid, stream);
    }
    if (e != hipSuccess) return GEMM_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    g_last_plan = glk::plan_json(p, M, N, K);
    return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_init(int device) {
    if (device < 0 || device >= kMaxDevices) return GEMM_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceState& ds = g_dev[device];
    if (ds.ready.load(std::memory_order_relaxed)) return GEMM_OK;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count) return GEMM_ERR_HIP;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return GEMM_ERR_HIP;
    if (hipSetDevice(device) != hipSuccess) return GEMM_ERR_HIP;
    int rc = GEMM_OK;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) rc = GEMM_ERR_HIP;
    if (rc == GEMM_OK) {
        ds.info.cus = prop.multiProcessorCount;
        // the XCDs (accelerator complex dies) the dispatcher deals workgroups to, round robin;
        // the tile orders keep each XCD's share contiguous (a bijection for any count)
        int xcc = 1;
        if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, device) != hipSuccess || xcc < 1)
            xcc = 1;
        ds.info.nxcd = (ds.info.cus % xcc == 0) ? xcc : 1;
        ds.info.ws_floats = kWsFloats;
        ds.info.ws_counters = kWsCounters;
        if (const char* f = getenv("GEMM_BF16_FORCE_TILE")) ds.info.force_tile_cfg = atoi(f);
        if (hipStreamCreateWithFlags(&ds.clear_stream, hipStreamNonBlocking) != hipSuccess) {
            ds.clear_stream = nullptr;
            rc = GEMM_ERR_HIP;
        }
    }
    // this device's copy of the scratch array: its address, and its counters cleared once here
    // (the kernels return every counter they use to zero)
    if (rc == GEMM_OK && hipGetSymbolAddress(reinterpret_cast<void**>(&ds.scratch_ptr), HIP_SYMBOL(scratch)) != hipSuccess) {
        ds.scratch_ptr = nullptr;
        rc = GEMM_ERR_HIP;
    }
    if (rc == GEMM_OK && (hipMemsetAsync(ds.scratch_ptr, 0, kScratchCounters * sizeof(uint32_t), ds.clear_stream) != hipSuccess ||
                          hipStreamSynchronize(ds.clear_stream) != hipSuccess))
        rc = GEMM_ERR_HIP;
    if (rc == GEMM_OK && glk::configure_skinny_kernels() != hipSuccess) rc = GEMM_ERR_HIP;
    if (rc == GEMM_OK && glk::configure_tile_kernels() != hipSuccess) rc = GEMM_ERR_HIP;
    if (rc == GEMM_OK && glk::configure_mx_kernels() != hipSuccess) rc = GEMM_ERR_HIP;
    if (rc == GEMM_OK && glk::configure_pk_kernels() != hipSuccess) rc = GEMM_ERR_HIP;
    if (rc == GEMM_OK) {
        ds.ready.store(true, std::memory_order_release);
        ++g_ready_count;
    } else if (ds.clear_stream) {
        hipStreamDestroy(ds.clear_stream);
        ds.clear_stream = nullptr;
    }
    hipSetDevice(prev);
    return rc;
}

int gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, void* C, int64_t ldc, gemm_stream_t stream) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, reinterpret_cast<hipStream_t>(stream), 0);
}

int gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                      int64_t ldb, void* C, int64_t ldc, gemm_stream_t stream) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, reinterpret_cast<hipStream_t>(stream), 0, false, true);
}

int gemm_bf16_skinny(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, void* C, int64_t ldc, gemm_stream_t stream) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, reinterpret_cast<hipStream_t>(stream), 1);
}

int gemm_bf16_tiled(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                    int64_t ldb, void* C, int64_t ldc, gemm_stream_t stream) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, reinterpret_cast<hipStream_t>(stream), 2);
}

int gemm_bf16_swiglu(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, void* C, int64_t ldc, gemm_stream_t stream) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, reinterpret_cast<hipStream_t>(stream), 0, true);
}

int gemm_plan_describe(int64_t M, int64_t N, int64_t K, int cus, int flags, char* buf, int len) {
    if (M < 0 || N < 0 || K < 0 || cus <= 0 || (flags & ~15)) return GEMM_ERR_INVALID_ARG;
    if (flags & GEMM_PLAN_PACKED) {
        if (flags != GEMM_PLAN_PACKED) return GEMM_ERR_INVALID_ARG;
        if (M > 64 || (N % 16) || (K % 32)) return GEMM_ERR_UNSUPPORTED;
        glk::DeviceInfo dev;
        dev.cus = cus;
        dev.nxcd = (cus % 8 == 0) ? 8 : 1;
        dev.ws_floats = kWsFloats;
        dev.ws_counters = kWsCounters;
        return copy_out(glk::plan_json(glk::make_packed_plan(M, N, K, dev), M, N, K), buf, len);
    }
    if (flags & GEMM_PLAN_MX) {
        if (flags != GEMM_PLAN_MX) return GEMM_ERR_INVALID_ARG;
        if (M > 64 || (N % 16) || (K % 128)) return GEMM_ERR_UNSUPPORTED;
        glk::DeviceInfo dev;
        dev.cus = cus;
        dev.nxcd = (cus % 8 == 0) ? 8 : 1;
        dev.ws_floats = kMxPartialFloats;
        dev.ws_counters = kWsCounters;
        return copy_out(glk::plan_json(glk::make_mx_plan(M, N, K, dev), M, N, K), buf, len);
    }
    const bool skinny = (flags & GEMM_PLAN_SKINNY) != 0, glu = (flags & GEMM_PLAN_SWIGLU) != 0;
    if (glu && N > INT64_MAX / 2) return GEMM_ERR_INVALID_ARG;
    if (skinny && (M < 1 || M > 64)) return GEMM_ERR_UNSUPPORTED;
    glk::DeviceInfo dev;
    dev.cus = cus;
    dev.nxcd = (cus % 8 == 0) ? 8 : 1;
    dev.ws_floats = kWsFloats;
    dev.ws_counters = kWsCounters;
    const glk::Plan p = glk::make_plan(M, N, K, dev, true, skinny ? 1 : 0, glu);
    return copy_out(glk::plan_json(p, M, N, K), buf, len);
}

int gemm_wave_efficiency(int64_t ctas, int64_t slots, double* efficiency, int64_t* waves) {
    if (ctas < 0 || slots <= 0 || !efficiency || !waves) return GEMM_ERR_INVALID_ARG;
    glk::wave_efficiency(ctas, slots, efficiency, waves);
    return GEMM_OK;
}

int gemm_last_plan(char* buf, int len) {
    std::lock_guard<std::mutex> lk(g_mu);
    return copy_out(g_last_plan, buf, len);
}

const char* gemm_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG";
        case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
        case GEMM_ERR_NOT_INITIALIZED: return "GEMM_ERR_NOT_INITIALIZED";
        case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
        default: return "GEMM_ERR_UNKNOWN";
    }
}

int gemm_finalize(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    int rc = GEMM_OK;
    for (int d = 0; d < kMaxDevices; ++d) {
        DeviceState& ds = g_dev[d];
        if (!ds.ready.load(std::memory_order_relaxed)) continue;
        int prev = -1;
        hipGetDevice(&prev);
        hipSetDevice(d);
        std::lock_guard<std::mutex> rl(ds.mu);
        for (int i = 0; i < ds.nregions; ++i) {
            if (hipFree(ds.regions[i].counters) != hipSuccess) rc = GEMM_ERR_HIP;
            ds.regions[i] = Region();
        }
        ds.nregions = 0;
        if (ds.clear_stream && hipStreamDestroy(ds.clear_stream) != hipSuccess) rc = GEMM_ERR_HIP;
        ds.clear_stream = nullptr;
        ds.ready.store(false, std::memory_order_release);
        hipSetDevice(prev);
    }
    g_ready_count = 0;
    return rc;
}


int gemm_mx_packed_sizes(int64_t N, int64_t K, int64_t* wp_bytes, int64_t* sp_bytes) {
    if (!wp_bytes || !sp_bytes) return GEMM_ERR_INVALID_ARG;
    return mx_packed(N, K, wp_bytes, sp_bytes);
}

int gemm_mx_pack_weight(int64_t N, int64_t K, const void* W, int64_t ldw, void* Wp, void* Sp,
                        gemm_stream_t stream) {
    int64_t wb = 0, sb = 0;
    int st = mx_packed(N, K, &wb, &sb);
    if (st != GEMM_OK) return st;
    if (ldw < K || (N > 0 && K > 0 && (!W || !Wp || !Sp))) return GEMM_ERR_INVALID_ARG;
    if (!aligned(W, 16) || !aligned(Wp, 16) || (ldw % 8)) return GEMM_ERR_INVALID_ARG;
    if (N > INT32_MAX || ldw > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    if (N == 0 || K == 0) return GEMM_OK;
    if (!current_state(&st)) return st;
    return glk::launch_mx_quant(true, static_cast<const uint16_t*>(W), (int)N, (int)K, (int)ldw,
                                static_cast<uint8_t*>(Wp), 0, static_cast<uint8_t*>(Sp), 0,
                                reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

int gemm_mx_quantize_act(int64_t M, int64_t K, const void* A, int64_t lda, void* Aq, int64_t ldaq, void* As,
                         int64_t ldas, gemm_stream_t stream) {
    return mx_quantize_act(M, K, A, lda, Aq, ldaq, As, ldas, reinterpret_cast<hipStream_t>(stream));
}

int gemm_mx_decode(int64_t M, int64_t N, int64_t K, const void* Aq, int64_t ldaq, const void* As,
                   int64_t ldas, const void* Wp, const void* Sp, void* C, int64_t ldc, gemm_stream_t stream) {
    return mx_decode(M, N, K, Aq, ldaq, As, ldas, Wp, Sp, C, ldc, reinterpret_cast<hipStream_t>(stream));
}

int gemm_mx_decode_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* Wp,
                        const void* Sp, void* C, int64_t ldc, gemm_stream_t stream) {
    if (M < 0 || N < 0 || K < 0 || lda < K || ldc < N) return GEMM_ERR_INVALID_ARG;
    if (M > 64 || (N % 16) || (K % 128)) return GEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GEMM_OK;
    if (M > 0 && K > 0 && !A) return GEMM_ERR_INVALID_ARG;
    if (K == 0) return mx_decode(M, N, K, nullptr, 0, nullptr, 0, Wp, Sp, C, ldc, reinterpret_cast<hipStream_t>(stream));
    int st = GEMM_OK;
    DeviceState* ds = current_state(&st);
    if (!ds) return st;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    // one or two rows: converted inside the product, one launch (when the piece's rows fit LDS)
    if (M <= 2) {
        glk::DeviceInfo info = ds->info;
        info.ws_floats = kMxPartialFloats;
        const glk::Plan p = glk::make_mx_plan(M, N, K, info);
        glk::MxArgs probe;
        const int ks = (int)(K / 128);
        if (p.kernel == glk::kKernMx && glk::mx_fused_layout((ks + p.splits - 1) / p.splits, p.strip / 16, probe) >= 0) {
            return mx_decode(M, N, K, nullptr, K, nullptr, K / 32, Wp, Sp, C, ldc, hs, A, lda);
        }
    }
    // the quantised activations go to the workspace tail (both launches on the same stream)
    const int64_t ldaq = (K + 15) / 16 * 16, ldas = K / 32;
    if (M * ldaq + M * ldas + 16 > kMxActBytes) return GEMM_ERR_UNSUPPORTED;
    Region* rg = nullptr;
    st = region_for(*ds, hs, &rg);
    if (st != GEMM_OK) return st;
    uint8_t* base = reinterpret_cast<uint8_t*>(rg->ws + kMxPartialFloats);
    uint8_t* aq = base;
    uint8_t* as = base + (M * ldaq + 15) / 16 * 16;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    st = mx_quantize_act(M, K, A, lda, aq, ldaq, as, ldas, s);
    if (st != GEMM_OK) return st;
    return mx_decode(M, N, K, aq, ldaq, as, ldas, Wp, Sp, C, ldc, s);
}

int gemm_pack_weight_bf16(int64_t K, int64_t N, const void* B, int64_t ldb, void* Bp, gemm_stream_t stream) {
    if (K < 0 || N < 0 || (K % 32) || (N % 16) || ldb < N) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && N > 0 && (!B || !Bp)) return GEMM_ERR_INVALID_ARG;
    if (!aligned(Bp, 16)) return GEMM_ERR_INVALID_ARG;
    if (N * K * 2 > INT32_MAX || ldb > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    if (K == 0 || N == 0) return GEMM_OK;
    int st = GEMM_OK;
    if (!current_state(&st)) return st;
    return glk::launch_pk_pack(static_cast<const uint16_t*>(B), (int)K, (int)N, (int)ldb,
                               static_cast<uint16_t*>(Bp), reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

int gemm_bf16_packed(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* Bp, void* C,
                     int64_t ldc, gemm_stream_t stream) {
    return packed_decode(M, N, K, A, lda, Bp, C, ldc, reinterpret_cast<hipStream_t>(stream));
}

int gemm_peak_mfma_launch(int64_t iters, int blocks, float* sink, uint64_t* cycles,
                          gemm_stream_t stream) {
    if (iters < 0 || blocks <= 0 || !sink || !cycles) return GEMM_ERR_INVALID_ARG;
    return glk::launch_peak_mfma(iters, blocks, sink, cycles, reinterpret_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

// (declared here rather than with the other launchers: the kernels' shared header is part of the
// source digest that ties the committed traffic summaries to the kernels they measured)
extern "C++" {
namespace glk {
hipError_t launch_peak_mfma_data(const void* ops, int64_t iters, int blocks, float* sink, uint64_t* cycles,
                                 hipStream_t s);
}
}

int gemm_peak_mfma_data_launch(const void* ops, int64_t iters, int blocks, float* sink, uint64_t* cycles,
                               gemm_stream_t stream) {
    if (iters < 0 || blocks <= 0 || !ops || !sink || !cycles || (reinterpret_cast<uintptr_t>(ops) & 15))
        return GEMM_ERR_INVALID_ARG;
    return glk::launch_peak_mfma_data(ops, iters, blocks, sink, cycles, reinterpret_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

int gemm_peak_copy_launch(const void* src, void* dst, int64_t bytes, gemm_stream_t stream) {
    if (bytes < 0 || (bytes & 15) || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
        return GEMM_ERR_INVALID_ARG;
    if (bytes > 0 && (!src || !dst)) return GEMM_ERR_INVALID_ARG;
    if (bytes == 0) return GEMM_OK;
    return glk::launch_peak_copy(src, dst, bytes, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

int gemm_peak_read_launch(const void* src, int64_t bytes, uint32_t* sink, gemm_stream_t stream) {
    if (bytes < 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) || !sink)
        return GEMM_ERR_INVALID_ARG;
    if (bytes > 0 && !src) return GEMM_ERR_INVALID_ARG;
    if (bytes == 0) return GEMM_OK;
    return glk::launch_peak_read(src, bytes, sink, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

int gemm_peak_clock_launch(int64_t iters, int blocks, uint64_t* out, gemm_stream_t stream) {
    if (iters < 0 || blocks <= 0 || !out) return GEMM_ERR_INVALID_ARG;
    return glk::launch_peak_clock(iters, blocks, out, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

int gemm_peak_xcc_launch(int blocks, uint32_t* out, gemm_stream_t stream) {
    if (blocks <= 0 || !out) return GEMM_ERR_INVALID_ARG;
    return glk::launch_peak_xcc(blocks, out, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

int gemm_peak_empty_launch(gemm_stream_t stream) {
    return glk::launch_peak_empty(reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? GEMM_OK
                                                                                       : GEMM_ERR_HIP;
}

int gemm_fill_launch(void* dst, int64_t bytes, uint32_t value, gemm_stream_t stream) {
    if (bytes < 0 || (bytes & 3) || (reinterpret_cast<uintptr_t>(dst) & 15)) return GEMM_ERR_INVALID_ARG;
    if (bytes > 0 && !dst) return GEMM_ERR_INVALID_ARG;
    if (bytes == 0) return GEMM_OK;
    return glk::launch_fill(dst, bytes, value, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

}  // extern "C"
