// tra_gemm.hip -- the C-ABI entry points of libtra_gemm.so (declared in
// include/tra_gemm.h): argument checks, choice of rung, launch on the
// caller's stream.
//
// The argument checks follow the pages' interfaces: the CPU and SYCL
// routines of page "[AutoMine++] #2 matmul trial and error"
// (velog.io/@levelstage/AutoMinepp2, sections "Intuitive implementation (by
// CPU)" and "Implementing with SYCL (iGPU)") refuse operands whose inner
// dimensions differ -- here, leading dimensions too small for the stated
// sizes -- and the kernels of page "GEMM kernel test code & optimization
// (1024^3 experiment)" take restrict-qualified operands, so C may not
// overlap A or B.  Errors come back as status codes; nothing throws across
// the ABI.
#include "tra_gemm.h"

#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "gemm_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

// Byte extent [lo, hi) of an r x c row-major view with leading dimension ld.
struct Extent {
    uintptr_t lo, hi;
};

// Returns false if the extent overflows.
bool extent_of(const void *p, int64_t rows, int64_t cols, int64_t ld, Extent &e) {
    if (rows <= 0 || cols <= 0) {
        e.lo = e.hi = reinterpret_cast<uintptr_t>(p);
        return true;
    }
    __int128 elems = static_cast<__int128>(rows - 1) * ld + cols;
    __int128 bytes = elems * static_cast<__int128>(sizeof(float));
    if (bytes > static_cast<__int128>(INT64_MAX)) return false;
    e.lo = reinterpret_cast<uintptr_t>(p);
    e.hi = e.lo + static_cast<uintptr_t>(bytes);
    return e.hi >= e.lo;
}

bool overlaps(const Extent &a, const Extent &b) { return a.lo < b.hi && b.lo < a.hi; }

bool valid_variant(int v) { return v >= TRA_GEMM_AUTO && v < TRA_GEMM_VARIANT_COUNT; }

// The rung AUTO runs for a shape.
int resolve(int variant, int64_t M, int64_t N, int64_t K) {
    if (variant != TRA_GEMM_AUTO) return variant;
    return tra::prefer_stream_k(M, N, K) ? TRA_GEMM_MFMA_STREAMK : TRA_GEMM_MFMA;
}

// The launch plan of a resolved rung (not AUTO).
tra::LaunchPlan plan_rung(int rung, int64_t M, int64_t N, int64_t K) {
    switch (rung) {
        case TRA_GEMM_NAIVE: return tra::plan_naive(M, N, K);
        case TRA_GEMM_LDS_TILED: return tra::plan_lds_tiled(M, N, K);
        case TRA_GEMM_REGBLOCK_DB: return tra::plan_regblock(M, N, K);
        case TRA_GEMM_MFMA_STREAMK: return tra::plan_mfma(M, N, K, true);
        default: return tra::plan_mfma(M, N, K, false);
    }
}

// The library's own workspaces, one per (device, stream) pair -- and per
// thread for hipStreamPerThread, a single handle that names a different
// stream in every thread.  Work on one stream runs in order, so calls on
// that stream may share one buffer.
//
// Growth is stream-ordered and never waits on the host: the old buffer is
// released with hipFreeAsync and the larger one taken with hipMallocAsync,
// both enqueued on the stream itself, so the release happens after every
// kernel already enqueued there has finished with the old buffer.
//
// Locking: g_ws_list_mutex guards only the list (held while an entry is
// found or added).  Each entry has its own mutex, held from the size check
// until the call's kernels are enqueued, so that another thread on the same
// stream cannot release the buffer between the two; calls on different
// streams never wait for each other.
//
// Entries are keyed by the stream handle: a stream destroyed with such calls
// still in flight, whose handle a later stream receives, would share the
// buffer with them unordered -- so a stream with split calls in flight must
// be synchronised before it is destroyed.  Buffers live until
// tra_gemm_release_workspaces() or the end of the process.
struct LibWorkspace {
    int device;
    hipStream_t stream;
    std::thread::id thread;   // set only for hipStreamPerThread
    std::mutex mutex;         // held across one call's size check and enqueue
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_list_mutex;
std::vector<std::unique_ptr<LibWorkspace>> g_ws;

// The entry of (current device, stream[, thread]), created on first use.
hipError_t find_workspace(hipStream_t stream, LibWorkspace **out) {
    int dev = 0;
    const hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const std::thread::id thread =
        stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
    std::lock_guard<std::mutex> lock(g_ws_list_mutex);
    for (const auto &w : g_ws) {
        if (w->device == dev && w->stream == stream && w->thread == thread) {
            *out = w.get();
            return hipSuccess;
        }
    }
    auto w = std::make_unique<LibWorkspace>();
    w->device = dev;
    w->stream = stream;
    w->thread = thread;
    *out = w.get();
    g_ws.push_back(std::move(w));
    return hipSuccess;
}

// Makes w hold at least `bytes` (rounded up to 1 MiB), in stream order;
// the caller holds w->mutex.
hipError_t grow_workspace(LibWorkspace &w, size_t bytes) {
    if (w.bytes >= bytes) return hipSuccess;
    hipError_t err;
    if (w.ptr != nullptr) {
        if ((err = hipFreeAsync(w.ptr, w.stream)) != hipSuccess) return err;
        w.ptr = nullptr;
        w.bytes = 0;
    }
    const size_t grown = (bytes + (1u << 20) - 1) & ~static_cast<size_t>((1u << 20) - 1);
    if ((err = hipMallocAsync(&w.ptr, grown, w.stream)) != hipSuccess) {
        w.ptr = nullptr;
        return err;
    }
    w.bytes = grown;
    return hipSuccess;
}

// Scratch of gemm_f32_variant_noalloc: one array per device, part of the
// library's code object, so that entry point never allocates.  The host
// name `scratch` is only a stand-in for the device array: its device
// address is looked up once per device (hipGetSymbolAddress, on the
// entry point's first call there, with that device current) and that
// address is what the kernels get.  Every call on a device shares the one
// array; nothing in it has to start at zero (each split writes every
// partial tile it later reads).
constexpr size_t kStaticScratchBytes = size_t{32} << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch array.
hipError_t static_scratch(void **out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if ((err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return err;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch(int variant, const tra::GemmArgs &a, void *ws, size_t ws_bytes) {
    switch (variant) {
        case TRA_GEMM_NAIVE: return tra::launch_naive(a);
        case TRA_GEMM_LDS_TILED: return tra::launch_lds_tiled(a);
        case TRA_GEMM_REGBLOCK_DB: return tra::launch_regblock(a);
        case TRA_GEMM_MFMA_STREAMK: return tra::launch_mfma(a, true, ws, ws_bytes);
        default: return tra::launch_mfma(a, false, ws, ws_bytes);
    }
}

tra_status hip_status(hipError_t err) {
    if (err == hipSuccess) return TRA_OK;
    tra::record_hip_error(err);
    return TRA_ERR_HIP;
}

tra::LaunchPlan plan_of(int variant, int64_t M, int64_t N, int64_t K) {
    return plan_rung(resolve(variant, M, N, K), M, N, K);
}

// Host-side checks; launches nothing.  On success with M, N > 0 (noop
// false), `rung` is the rung to run and `plan` its launch.
tra_status check_args(int variant, int64_t M, int64_t N, int64_t K, const float *A,
                      int64_t lda, const float *B, int64_t ldb, const float *C, int64_t ldc,
                      bool &noop, int &rung, tra::LaunchPlan &plan) {
    noop = false;
    if (!valid_variant(variant)) return TRA_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return TRA_ERR_INVALID_ARG;
    if (M == 0 || N == 0) {
        noop = true;
        return TRA_OK;
    }
    if (C == nullptr || ldc < N) return TRA_ERR_INVALID_ARG;
    Extent ec{};
    if (!extent_of(C, M, N, ldc, ec)) return TRA_ERR_INVALID_ARG;
    if (K > 0) {
        if (A == nullptr || B == nullptr || lda < K || ldb < N) return TRA_ERR_INVALID_ARG;
        Extent ea{}, eb{};
        if (!extent_of(A, M, K, lda, ea) || !extent_of(B, K, N, ldb, eb))
            return TRA_ERR_INVALID_ARG;
        if (overlaps(ec, ea) || overlaps(ec, eb)) return TRA_ERR_INVALID_ARG;
    }
    rung = resolve(variant, M, N, K);
    plan = plan_rung(rung, M, N, K);
    if (plan.grid <= 0 || plan.grid > tra::kMaxGrid ||
        plan.grid * plan.block > tra::kMaxGridLanes)
        return TRA_ERR_UNSUPPORTED;
    return TRA_OK;
}

}  // namespace

void tra::record_hip_error(hipError_t err) { g_last_hip_error = static_cast<int>(err); }

extern "C" {

tra_status gemm_f32_variant(int variant, int64_t M, int64_t N, int64_t K, const float *A,
                            int64_t lda, const float *B, int64_t ldb, float *C, int64_t ldc,
                            void *stream) {
    bool noop = false;
    int v = 0;
    tra::LaunchPlan plan{};
    const tra_status st = check_args(variant, M, N, K, A, lda, B, ldb, C, ldc, noop, v, plan);
    if (st != TRA_OK || noop) return st;

    const tra::GemmArgs a{M, N, K, A, lda, B, ldb, C, ldc, static_cast<hipStream_t>(stream)};
    const size_t need = plan.workspace_bytes;
    if (need == 0) return hip_status(launch(v, a, nullptr, 0));
    // A buffer allocated in stream order while the stream is being captured
    // would belong to the graph, not to the library: capture takes the
    // caller's workspace (gemm_f32_variant_ws) instead.
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    hipError_t err = hipStreamIsCapturing(a.stream, &capture);
    if (err != hipSuccess) return hip_status(err);
    if (capture != hipStreamCaptureStatusNone) return TRA_ERR_UNSUPPORTED;
    LibWorkspace *w = nullptr;
    if ((err = find_workspace(a.stream, &w)) != hipSuccess) return hip_status(err);
    std::lock_guard<std::mutex> lock(w->mutex);
    if ((err = grow_workspace(*w, need)) != hipSuccess) return hip_status(err);
    return hip_status(launch(v, a, w->ptr, w->bytes));
}

tra_status gemm_f32_variant_ws(int variant, int64_t M, int64_t N, int64_t K, const float *A,
                               int64_t lda, const float *B, int64_t ldb, float *C, int64_t ldc,
                               void *workspace, size_t workspace_bytes, void *stream) {
    bool noop = false;
    int v = 0;
    tra::LaunchPlan plan{};
    const tra_status st = check_args(variant, M, N, K, A, lda, B, ldb, C, ldc, noop, v, plan);
    if (st != TRA_OK || noop) return st;

    const size_t need = plan.workspace_bytes;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                     (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0))
        return TRA_ERR_INVALID_ARG;
    const tra::GemmArgs a{M, N, K, A, lda, B, ldb, C, ldc, static_cast<hipStream_t>(stream)};
    return hip_status(launch(v, a, workspace, workspace_bytes));
}

tra_status gemm_f32_variant_noalloc(int variant, int64_t M, int64_t N, int64_t K,
                                    const float *A, int64_t lda, const float *B, int64_t ldb,
                                    float *C, int64_t ldc, void *stream) {
    bool noop = false;
    int v = 0;
    tra::LaunchPlan plan{};
    const tra_status st = check_args(variant, M, N, K, A, lda, B, ldb, C, ldc, noop, v, plan);
    if (st != TRA_OK || noop) return st;
    const size_t need = plan.workspace_bytes;
    if (need > kStaticScratchBytes) return TRA_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t err = static_scratch(&ws);
        if (err != hipSuccess) return hip_status(err);
    }
    const tra::GemmArgs a{M, N, K, A, lda, B, ldb, C, ldc, static_cast<hipStream_t>(stream)};
    return hip_status(launch(v, a, ws, need > 0 ? kStaticScratchBytes : 0));
}

tra_status tra_gemm_workspace_size(int variant, int64_t M, int64_t N, int64_t K,
                                   size_t *bytes) {
    if (!valid_variant(variant) || M < 0 || N < 0 || K < 0 || bytes == nullptr)
        return TRA_ERR_INVALID_ARG;
    *bytes = (M == 0 || N == 0) ? 0 : plan_of(variant, M, N, K).workspace_bytes;
    return TRA_OK;
}

tra_status gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                    const float *B, int64_t ldb, float *C, int64_t ldc, void *stream) {
    return gemm_f32_variant(TRA_GEMM_AUTO, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

tra_status tra_gemm_describe(int variant, int64_t M, int64_t N, int64_t K, char *buf,
                             size_t len) {
    if (!valid_variant(variant) || M < 0 || N < 0 || K < 0) return TRA_ERR_INVALID_ARG;
    if (buf == nullptr) return len == 0 ? TRA_OK : TRA_ERR_INVALID_ARG;
    if (len == 0) return TRA_OK;
    const int rung = resolve(variant, M, N, K);
    const tra::LaunchPlan p = plan_rung(rung, M, N, K);
    std::snprintf(buf, len,
                  "variant=%s rung=%s kernel=%s tile=%dx%dx%d grid=%lld block=%d lds_bytes=%d "
                  "stream_k_tiles=%lld stream_k_wgs=%lld split=%s workspace_bytes=%zu",
                  tra_gemm_variant_name(variant),
                  tra_gemm_variant_name(rung), p.kernel, p.bm, p.bn, p.bk,
                  static_cast<long long>(p.grid), p.block, p.lds_bytes,
                  static_cast<long long>(p.sk_tiles), static_cast<long long>(p.sk_wgs),
                  p.split != nullptr ? p.split : "none", p.workspace_bytes);
    return TRA_OK;
}

const char *tra_status_string(int status) {
    switch (status) {
        case TRA_OK: return "ok";
        case TRA_ERR_INVALID_ARG: return "invalid argument";
        case TRA_ERR_UNSUPPORTED: return "unsupported";
        case TRA_ERR_HIP: return "HIP runtime error";
        default: return "unknown";
    }
}

const char *tra_gemm_variant_name(int variant) {
    switch (variant) {
        case TRA_GEMM_AUTO: return "auto";
        case TRA_GEMM_NAIVE: return "naive";
        case TRA_GEMM_LDS_TILED: return "lds_tiled";
        case TRA_GEMM_REGBLOCK_DB: return "regblock_db";
        case TRA_GEMM_MFMA: return "mfma";
        case TRA_GEMM_MFMA_STREAMK: return "mfma_streamk";
        default: return "unknown";
    }
}

int tra_last_hip_error(void) { return g_last_hip_error; }

tra_status tra_gemm_release_workspaces(void) {
    std::lock_guard<std::mutex> list_lock(g_ws_list_mutex);
    int current = -1;
    hipError_t first = hipSuccess;
    for (const auto &w : g_ws) {
        std::lock_guard<std::mutex> lock(w->mutex);
        if (w->ptr == nullptr) continue;
        if (current < 0 && (first = hipGetDevice(&current)) != hipSuccess) break;
        // the stream may be gone: wait for the whole device, then release
        // the buffer on the null stream
        hipError_t err = hipSetDevice(w->device);
        if (err == hipSuccess) err = hipDeviceSynchronize();
        if (err == hipSuccess) err = hipFreeAsync(w->ptr, nullptr);
        if (err == hipSuccess) err = hipStreamSynchronize(nullptr);
        if (err == hipSuccess) {
            w->ptr = nullptr;
            w->bytes = 0;
        } else if (first == hipSuccess) {
            first = err;
        }
    }
    if (current >= 0) {
        const hipError_t back = hipSetDevice(current);
        if (first == hipSuccess) first = back;
    }
    return hip_status(first);
}

}  // extern "C"
