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
    int64_t sk_tiles;     // tiles shared out by K slice (stream-K), 0 = none
    int64_t sk_wgs;       // workgroups that run them
    const char *split;    // "none", "parts" (K parts in the main launch) or
                          // "runs" (stream-K runs in a launch of their own)
    size_t workspace_bytes;   // device scratch for partial tiles
};

// Limits of one launch: workgroups in the x dimension (the kernels index
// them with int), and work-items in the x dimension, which HIP requires to
// fit 32 bits (grid x block <= 2^32 - 1).
constexpr int64_t kMaxGrid = 2147483647;
constexpr int64_t kMaxGridLanes = 4294967295;

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
__host__ __device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t n) {
    constexpr int64_t kXcds = 8;
    const int64_t q = n / kXcds, r = n % kXcds;
    const int64_t x = bid % kXcds, slot = bid / kXcds;
    return x * q + (x < r ? x : r) + slot;
}

// The same two maps in 32-bit arithmetic, cheaper than the 64-bit
// divisions at the start of every workgroup.  Safe for any launch the host
// accepts: at most 2^32 - 1 lanes, so at most 2^24 workgroups of 256 lanes
// (2^23 of 512), and G * tiles_n stays far below 2^31.
__host__ __device__ __forceinline__ int xcd_remap32(int bid, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = bid & 7, slot = bid >> 3;
    return x * q + (x < r ? x : r) + slot;
}

template <int G>
__host__ __device__ __forceinline__ void grouped_tile32(int id, int tiles_m, int tiles_n, int &tm,
                                                       int &tn) {
    const unsigned per_group = static_cast<unsigned>(G) * static_cast<unsigned>(tiles_n);
    const unsigned g = static_cast<unsigned>(id) / per_group;
    const int first = static_cast<int>(g) * G;
    const int rows = (tiles_m - first) < G ? (tiles_m - first) : G;
    const unsigned in = static_cast<unsigned>(id) - g * per_group;
    const unsigned q = in / static_cast<unsigned>(rows);
    tm = first + static_cast<int>(in - q * static_cast<unsigned>(rows));
    tn = static_cast<int>(q);
}

// Logical tile id -> (tile row, tile column) in groups of `group` tile rows
// swept column by column, so that consecutive ids reuse the same B columns
// and a small set of A rows.
__host__ __device__ __forceinline__ void grouped_tile(int64_t id, int64_t tiles_m, int64_t tiles_n,
                                             int64_t group, int64_t &tm, int64_t &tn) {
    const int64_t per_group = group * tiles_n;
    const int64_t g = id / per_group;
    const int64_t first = g * group;
    const int64_t rows = (tiles_m - first) < group ? (tiles_m - first) : group;
    const int64_t in = id - g * per_group;
    tm = first + in % rows;
    tn = in / rows;
}

// ---- LDS poison (test builds) ----
//
// Built with TRA_LDS_POISON=1 (libtra_gemm_poison.so, for the tests), every
// kernel that stages operands in LDS first fills its LDS with a quiet NaN,
// so that a read of any word that no lane staged -- a wrong index, a row
// padding word, a slice read before it was stored -- makes C NaN, which the
// exact parity checks catch.  In the product build this is nothing.
#ifndef TRA_LDS_POISON
#define TRA_LDS_POISON 0
#endif

__device__ __forceinline__ void lds_poison(float *lds, int words) {
    if constexpr (TRA_LDS_POISON != 0) {
        const int nt = static_cast<int>(blockDim.x * blockDim.y * blockDim.z);
        const int t = static_cast<int>(threadIdx.x +
                                       blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z));
        for (int i = t; i < words; i += nt) lds[i] = __int_as_float(0x7fc00000);
        __syncthreads();
    }
}

// ---- operand loads and tile placement shared by the tiled rungs ----

// X[row][col .. col+3] of a rows x cols row-major matrix, zero outside it.
// Addresses are clamped into the matrix, so every load is valid, and the
// zero is applied with an AND mask on the loaded bits: the loads are
// unconditional (a select would let the compiler predicate each load behind
// a branch and wait for it).  The mask does make the wave wait for the load
// (and every load before it) where it is applied, which is cheap for the
// one slice per tile that runs past K but not for a whole K loop.
__device__ __forceinline__ float4 load4_clamped(const float *X, int64_t ld, int64_t row,
                                                int64_t col, int64_t rows, int64_t cols) {
    const bool rok = row < rows;
    const float *p = X + (rok ? row : rows - 1) * ld;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t c = col + e;
        const float x = p[c < cols ? c : cols - 1];
        const unsigned keep = (rok && c < cols) ? 0xffffffffu : 0u;
        v[e] = __uint_as_float(__float_as_uint(x) & keep);
    }
    return make_float4(v[0], v[1], v[2], v[3]);
}

// Sixteen zero bytes in device memory (one copy per code object), read in
// place of a float4 that lies outside a matrix.
static __device__ __attribute__((aligned(16))) float g_zero4[4] = {0.0f, 0.0f, 0.0f, 0.0f};

// X[row][col .. col+3] as one float4 where that quad lies inside the matrix
// (`in`), else +0: for 16-byte aligned rows and a quad that is wholly
// inside or wholly outside.  The choice is an address select made before
// the load, so nothing waits for the loaded value until it is used.
__device__ __forceinline__ float4 load4_quad(const float *X, int64_t ld, int64_t row,
                                             int64_t col, bool in) {
    return *reinterpret_cast<const float4 *>(in ? X + row * ld + col : &g_zero4[0]);
}

// X[row][col .. col+3] element by element, for a row that lies inside the
// matrix when `row_in`, with +0 for row_in false and for columns at or past
// `cols`; each element outside reads the zero word, as in load4_quad.
__device__ __forceinline__ float4 load4_elems(const float *X, int64_t ld, int64_t row,
                                              int64_t col, bool row_in, int64_t cols) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        v[e] = *(row_in && col + e < cols ? X + row * ld + col + e : &g_zero4[0]);
    return make_float4(v[0], v[1], v[2], v[3]);
}

// How a slice is loaded from global memory.  A tile is always placed
// inside the matrices when they are at least one tile large (see
// tile_origin below), so only the slice that runs past K and matrices
// smaller than a tile need index checks.
//   kVec      A and B rows 16-byte aligned at the tile: float4 loads;
//   kVecA     A aligned, B not (ldb or the tile's first column not a
//             multiple of 4): float4 loads of A, element loads of B;
//   kScalar   element loads of both;
//             (the MFMA rung loads the quads of all three modes as float4s
//             through buffer resources, at 4-byte-aligned offsets where
//             rows are not aligned; the register-blocked rung as written)
//   kChecked  element loads with zeros outside the matrices: the k tail
//             slice, and in the register-blocked rung the tiles larger than
//             the matrix;
//   kEdge     full slices of a tile larger than the matrix when A and B are
//             aligned and N is a multiple of 4: float4 loads, zeros past
//             row M of A and column N of B;
//   kEdgeElem full slices of a tile larger than the matrix otherwise:
//             element loads, zeros past row M of A and column N of B.
enum LoadMode { kVec = 0, kVecA = 1, kScalar = 2, kChecked = 3, kEdge = 4, kEdgeElem = 5 };

__device__ __forceinline__ float4 load4_scalar(const float *p) {
    return make_float4(p[0], p[1], p[2], p[3]);
}

// Where block tile (tm, tn) sits.  A tile that would cross row M (column
// N) of a matrix at least BM rows (BN columns) large is moved back to end at
// row M (column N), so every load of a full slice stays inside the
// matrices with no checks; its first skip_m rows (skip_n columns) belong to
// the tile before it and are not stored.  Only matrices smaller than a tile
// leave tiles that hang over an edge (loaded with checks).
struct Origin {
    int64_t m0, n0;
    int skip_m, skip_n;
};

template <int BM, int BN>
__host__ __device__ __forceinline__ Origin tile_origin(int64_t tm, int64_t tn, int64_t M,
                                                       int64_t N) {
    Origin o{tm * BM, tn * BN, 0, 0};
    if (o.m0 + BM > M && M >= BM) {
        o.skip_m = static_cast<int>(o.m0 + BM - M);
        o.m0 = M - BM;
    }
    if (o.n0 + BN > N && N >= BN) {
        o.skip_n = static_cast<int>(o.n0 + BN - N);
        o.n0 = N - BN;
    }
    return o;
}

}  // namespace tra
