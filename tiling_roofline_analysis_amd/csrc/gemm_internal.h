// gemm_internal.h -- internal interface between the C-ABI entry points
// (tra_gemm.hip) and the kernel rungs (gemm_*.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace tra {

// Arguments of one validated GEMM call: M, N > 0, K >= 0, strides checked.
struct GemmArgs {
    int64_t M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
    hipStream_t stream;
};

// What a rung will launch for a shape (host side; the stream-K split reads
// the current device's CU count and falls back to MI355X's without one).
struct LaunchPlan {
    const char *kernel;   // kernel function name (as profilers print it)
    int bm, bn, bk;       // block tile of C and K step (1 for no tile)
    int64_t grid;         // workgroups
    int block;            // lanes per workgroup
    int lds_bytes;        // LDS per workgroup
    int split_k;          // K partitions (1 = none)
    int64_t sk_tiles;     // tiles shared out by K slice (stream-K), 0 = none
    int64_t sk_wgs;       // workgroups that run them
    size_t workspace_bytes;   // device scratch for partial tiles
};

// Grid limit of one launch (workgroups in the x dimension).
constexpr int64_t kMaxGrid = 2147483647;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// True if p is 16-byte aligned and ld keeps every row 16-byte aligned.
inline bool vec4_ok(const void *p, int64_t ld) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && (ld & 3) == 0;
}

// Keeps a failed launch's hipError_t for tra_last_hip_error() (per thread).
void record_hip_error(hipError_t err);

LaunchPlan plan_naive(int64_t M, int64_t N, int64_t K);
hipError_t launch_naive(const GemmArgs &a);

LaunchPlan plan_lds_tiled(int64_t M, int64_t N, int64_t K);
hipError_t launch_lds_tiled(const GemmArgs &a);

LaunchPlan plan_regblock(int64_t M, int64_t N, int64_t K);
hipError_t launch_regblock(const GemmArgs &a);

// stream_k: share the last partial wave of tiles out by K slice (needs
// `ws`, at least plan_mfma(..).workspace_bytes bytes, when that is > 0).
LaunchPlan plan_mfma(int64_t M, int64_t N, int64_t K, bool stream_k);
hipError_t launch_mfma(const GemmArgs &a, bool stream_k, void *ws, size_t ws_bytes);
// True where the stream-K split is expected to beat one tile per workgroup.
bool prefer_stream_k(int64_t M, int64_t N, int64_t K);

// XCD-aware remap of a linear workgroup id.  The dispatcher hands
// workgroups to the 8 XCDs of an MI355X round-robin (id mod 8), and each
// XCD has its own L2.  The remap gives each XCD a contiguous run of logical
// tile ids so that the tiles it runs at the same time share rows of A and
// columns of B in its L2.  A bijection on [0, n) for any n.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t n) {
    constexpr int64_t kXcds = 8;
    const int64_t q = n / kXcds, r = n % kXcds;
    const int64_t x = bid % kXcds, slot = bid / kXcds;
    return x * q + (x < r ? x : r) + slot;
}

// Logical tile id -> (tile row, tile column) in groups of `group` tile rows
// swept column by column, so that consecutive ids reuse the same B columns
// and a small set of A rows.
__device__ __forceinline__ void grouped_tile(int64_t id, int64_t tiles_m, int64_t tiles_n,
                                             int64_t group, int64_t &tm, int64_t &tn) {
    const int64_t per_group = group * tiles_n;
    const int64_t g = id / per_group;
    const int64_t first = g * group;
    const int64_t rows = (tiles_m - first) < group ? (tiles_m - first) : group;
    const int64_t in = id - g * per_group;
    tm = first + in % rows;
    tn = in / rows;
}

}  // namespace tra
