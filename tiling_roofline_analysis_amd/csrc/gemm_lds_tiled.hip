// gemm_lds_tiled.hip -- rung 2 of the ladder: operand tiles staged once in
// LDS and reused from there, one element of C per lane.
//
// The lever this rung shows is the one the pages build their tiled kernels
// on: a block of C is computed by one workgroup, which copies a slice of A's
// rows and of B's columns into on-chip memory once and then reads every
// staged element as many times as the tile is wide, so global traffic falls
// about as 1/T (page "GEMM kernel test code & optimization (1024^3
// experiment)", teach-meaning.tistory.com/1513, sections "Tile concept",
// "Tile loading step" and "Key idea: reuse through shared memory"; page
// "Roofline & Tiling notes", legato-user-group.github.io/tensor2silicon-lab/
// week04/researchers/jaehyeong, section 3 "Tiling"; page "[AutoMine++] #2
// matmul trial and error", velog.io/@levelstage/AutoMinepp2, section
// "Breaking the memory bottleneck: Tiling", with T = 16 as here).  Elements
// outside the matrices are staged as zeros, so partial tiles need no other
// care.  There is one level of tiling only: each lane keeps a single
// accumulator (register reuse across outputs is rung 3's lever), and the
// group waits twice per slice -- after staging, and before the next
// slice's stores overwrite what slower waves may still read (double
// buffering is rung 3's lever too).
//
// gfx950 design (256 lanes = 4 wave64s; lane t owns C[m0 + t/16][n0 + t%16]):
//   * slices are 64 deep, so a slice costs 2 barriers per 64 multiply-adds;
//   * both operands are kept k-contiguous in LDS with rows padded to 68
//     words, As[m][k] and Bs[n][k] (B transposed): the inner loop takes four
//     k steps from one ds_read_b128 of A and one of B -- two LDS reads per
//     four FMAs instead of two per FMA;
//   * staging: each lane loads one k-contiguous quad of each operand and
//     stores it with one ds_write_b128.  For A that is one float4 along K
//     (16 lanes read 256 contiguous bytes of a row); for B it is four
//     elements down one column, each load instruction reading 64-byte row
//     segments of four rows.  (Loading B as float4 along N and transposing
//     it in the store took four ds_write_b32 per lane, which the compiler
//     pairs into writes two rows apart that collide in the banks: 0.23
//     conflict cycles per LDS instruction.)
//   * bank groups: 68 = 4 (mod 64), so row r starts 4r words into the bank
//     ring.  A wave's A reads touch 4 rows (each broadcast to 16 lanes) and
//     its B reads 16 rows: distinct 4-bank groups.  The stores of 16
//     consecutive lanes cover one A row's 64 words, or the same quad of 16
//     B rows: distinct 4-bank groups again.
// The k order inside each element is 0..K-1, as in the naive rung.
#include "gemm_internal.h"

namespace tra {
namespace {

constexpr int kT = 16;            // tile of C: kT x kT, one element per lane
constexpr int kBK = 64;           // K slice
constexpr int kRow = kBK + 4;     // LDS row stride in words (k contiguous)
constexpr int kLanes = kT * kT;   // 256

// X[row][col .. col+3] of a rows x cols matrix, element by element, zero
// outside it (the edge tiles, unaligned rows and the slice past K); and the
// same for a quad down one column.
__device__ __forceinline__ float4 quad_checked(const float *X, int64_t ld, int64_t row,
                                               int64_t col, int64_t rows, int64_t cols) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (row < rows && col + e < cols) ? X[row * ld + col + e] : 0.0f;
    return make_float4(v[0], v[1], v[2], v[3]);
}

// X[row .. row+3][col] of a rows x cols matrix, zero outside it.
__device__ __forceinline__ float4 column_checked(const float *X, int64_t ld, int64_t row,
                                                 int64_t col, int64_t rows, int64_t cols) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (row + e < rows && col < cols) ? X[(row + e) * ld + col] : 0.0f;
    return make_float4(v[0], v[1], v[2], v[3]);
}

__global__ __launch_bounds__(kLanes)
void gemm_lds_tiled_f32(int64_t M, int64_t N, int64_t K,
                        const float *__restrict__ A, int64_t lda,
                        const float *__restrict__ B, int64_t ldb,
                        float *__restrict__ C, int64_t ldc,
                        int64_t tiles_m, int64_t tiles_n, int vec_a)
{
    __shared__ __attribute__((aligned(16))) float As[kT * kRow];   // As[m][k]
    __shared__ __attribute__((aligned(16))) float Bs[kT * kRow];   // Bs[n][k]
    lds_poison(As, kT * kRow);
    lds_poison(Bs, kT * kRow);

    const int t = static_cast<int>(threadIdx.x);
    int64_t tm, tn;
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
    const int64_t m0 = tm * kT, n0 = tn * kT;

    // this lane's output, and the quads it stages each slice
    const int row = t / kT, col = t % kT;
    const int am = t / (kBK / 4), akq = t % (kBK / 4);   // A: row am, k quad akq
    const int bn = t % kT, bkq = t / kT;                 // B: column bn, k quad bkq

    // Slices below `plain` load with no checks (A as one float4): the tile
    // lies inside both matrices and A's rows are 16-byte aligned.  The
    // choice is the same for every lane of the workgroup.
    const bool inside = vec_a && m0 + kT <= M && n0 + kT <= N;
    const int64_t plain = inside ? K / kBK * kBK : 0;
    const float *pa = A + (m0 + am) * lda + 4 * akq;
    const float *pb = B + 4 * bkq * ldb + n0 + bn;

    float acc = 0.0f;
    // one slice: stage it, wait, accumulate from LDS, wait
    auto slice = [&](float4 a, float4 b) {
        *reinterpret_cast<float4 *>(&As[am * kRow + 4 * akq]) = a;
        *reinterpret_cast<float4 *>(&Bs[bn * kRow + 4 * bkq]) = b;
        __syncthreads();   // the slice is staged
#pragma unroll
        for (int q = 0; q < kBK / 4; ++q) {
            const float4 x = *reinterpret_cast<const float4 *>(&As[row * kRow + 4 * q]);
            const float4 y = *reinterpret_cast<const float4 *>(&Bs[col * kRow + 4 * q]);
            acc = fmaf(x.x, y.x, acc);
            acc = fmaf(x.y, y.y, acc);
            acc = fmaf(x.z, y.z, acc);
            acc = fmaf(x.w, y.w, acc);
        }
        __syncthreads();   // every wave is done with the slice
    };
    int64_t k0 = 0;
    for (; k0 < plain; k0 += kBK) {
        const float *q = pb + k0 * ldb;
        slice(*reinterpret_cast<const float4 *>(pa + k0),
              make_float4(q[0], q[ldb], q[2 * ldb], q[3 * ldb]));
    }
    for (; k0 < K; k0 += kBK)
        slice(quad_checked(A, lda, m0 + am, k0 + 4 * akq, M, K),
              column_checked(B, ldb, k0 + 4 * bkq, n0 + bn, K, N));
    const int64_t gm = m0 + row, gn = n0 + col;
    if (gm < M && gn < N) C[gm * ldc + gn] = acc;
}

}  // namespace

LaunchPlan plan_lds_tiled(int64_t M, int64_t N, int64_t /*K*/) {
    LaunchPlan p{};
    p.kernel = "gemm_lds_tiled_f32";
    p.bm = kT;
    p.bn = kT;
    p.bk = kBK;
    p.grid = ceil_div(M, kT) * ceil_div(N, kT);
    p.block = kLanes;
    p.lds_bytes = 2 * kT * kRow * static_cast<int>(sizeof(float));
    return p;
}

hipError_t launch_lds_tiled(const GemmArgs &a) {
    const LaunchPlan p = plan_lds_tiled(a.M, a.N, a.K);
    const int64_t tiles_m = ceil_div(a.M, kT), tiles_n = ceil_div(a.N, kT);
    hipLaunchKernelGGL(gemm_lds_tiled_f32, dim3(static_cast<uint32_t>(p.grid)), dim3(kLanes), 0,
                       a.stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, tiles_m,
                       tiles_n, static_cast<int>(vec4_ok(a.A, a.lda)));
    return hipGetLastError();
}

}  // namespace tra
