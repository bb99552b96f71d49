// gemm_naive.hip -- rung 1 of the ladder: one lane per element of C.
//
// Page "GEMM kernel test code & optimization (1024^3 experiment)"
// (teach-meaning.tistory.com/1513), sections "How the naive GEMM kernel
// works" and "Memory access pattern": every lane owns one C[row, col], keeps
// one accumulator that starts at zero, walks k = 0..K-1 reading A[row, k] and
// B[k, col] straight from global memory, and stores once; lanes outside C
// return.  All reuse is left to the caches.
//
// gfx950 form: a workgroup is 64 x 4 lanes, so each wave64 covers 64
// consecutive columns of one row.  Its B loads are one contiguous 256-byte
// row segment per k and its A load is the same address for all 64 lanes.
// The grid is one-dimensional (row-major over 64 x 4 tiles) so M and N are
// limited only by the 2^31 - 1 workgroup count.
#include "gemm_internal.h"

namespace tra {
namespace {

constexpr int kNaiveCols = 64;  // lanes along N (one wave)
constexpr int kNaiveRows = 4;   // waves along M

__global__ __launch_bounds__(kNaiveCols * kNaiveRows)
void gemm_naive_f32(int64_t M, int64_t N, int64_t K,
                    const float *__restrict__ A, int64_t lda,
                    const float *__restrict__ B, int64_t ldb,
                    float *__restrict__ C, int64_t ldc, int64_t tiles_n)
{
    const int64_t bid = blockIdx.x;
    const int64_t row = (bid / tiles_n) * kNaiveRows + threadIdx.y;
    const int64_t col = (bid % tiles_n) * kNaiveCols + threadIdx.x;
    if (row >= M || col >= N) return;

    const float *a = A + row * lda;
    const float *b = B + col;
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) acc = fmaf(a[k], b[k * ldb], acc);
    C[row * ldc + col] = acc;
}

}  // namespace

LaunchPlan plan_naive(int64_t M, int64_t N, int64_t /*K*/) {
    LaunchPlan p{};
    p.kernel = "gemm_naive_f32";
    p.bm = kNaiveRows;
    p.bn = kNaiveCols;
    p.bk = 1;
    p.grid = ceil_div(M, kNaiveRows) * ceil_div(N, kNaiveCols);
    p.block = kNaiveCols * kNaiveRows;
    p.lds_bytes = 0;
    return p;
}

hipError_t launch_naive(const GemmArgs &a) {
    const LaunchPlan p = plan_naive(a.M, a.N, a.K);
    const int64_t tiles_n = ceil_div(a.N, kNaiveCols);
    hipLaunchKernelGGL(gemm_naive_f32, dim3(static_cast<uint32_t>(p.grid)),
                       dim3(kNaiveCols, kNaiveRows), 0, a.stream,
                       a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, tiles_n);
    return hipGetLastError();
}

}  // namespace tra
