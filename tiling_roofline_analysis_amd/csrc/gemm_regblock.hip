// gemm_regblock.hip -- rung 3 of the ladder: register-blocked VALU GEMM with
// double-buffered LDS.
//
// The pages' argument for tiling is that a staged element is reused as many
// times as the tile is wide, so HBM traffic falls about as 1/T and the
// arithmetic intensity rises (page "Roofline & Tiling notes",
// legato-user-group.github.io/tensor2silicon-lab/week04/researchers/jaehyeong,
// section 3 "Tiling", and the week's key points), while larger tiles cost
// registers/LDS and occupancy, and the staging barriers cost time (page
// "GEMM kernel test code & optimization (1024^3 experiment)", section
// "Key idea: reuse through shared memory").  This rung pushes both levers:
//   * a 128 x 128 block tile of C (each staged element reused 128 times);
//   * each lane holds an 8 x 8 micro-tile of C in VGPRs, so one LDS read
//     feeds 8 FMAs instead of one;
//   * the next K slice is fetched into registers while the current one is
//     consumed from LDS, and two LDS buffers alternate, so each slice needs
//     one barrier instead of two.
//
// gfx950 layout (256 lanes = 4 wave64s, lane t: tx = t % 16, ty = t / 16):
//   rows of C held by a lane:  ty + 16*i, i = 0..7
//   columns held by a lane:    4*tx + j and 64 + 4*tx + j, j = 0..3
//   As[m][k]  k contiguous, row stride 20 words (16 + 4): a wave reads 4
//             consecutive rows at once (one ds_read_b128 each), which land
//             in 4 disjoint bank groups; global float4 rows store as-is.
//   Bs[k][n]  n contiguous, row stride 132 words: a wave reads 64
//             consecutive words per ds_read_b128.
// The arithmetic is VALU fmaf (v_fma_f32); packed-FP32 instructions are
// disabled for this build, so the rung's ceiling is the unpacked FP32 VALU
// rate (about 100 TFLOP/s measured by tra_probe_fma_f32 on MI355X), below
// the 157.3 TFLOP/s FP32 peak that the matrix cores reach.
#include "gemm_internal.h"

namespace tra {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 16;
constexpr int kThreads = 256;
constexpr int kAStride = kBK + 4;    // words per As row
constexpr int kBStride = kBN + 4;    // words per Bs row
constexpr int kAF4 = kBM * kBK / 4 / kThreads;   // float4 of A per lane per slice (2)
constexpr int kBF4 = kBK * kBN / 4 / kThreads;   // float4 of B per lane per slice (2)

// Loads 4 consecutive floats p[0..3] of a row; elements at or past `lim`
// (or the whole group when !row_ok) read as zero.
__device__ __forceinline__ float4 load4(const float *p, bool row_ok, int64_t first,
                                        int64_t lim, bool vec) {
    if (row_ok && vec && first + 3 < lim) return *reinterpret_cast<const float4 *>(p);
    float4 v;
    v.x = (row_ok && first + 0 < lim) ? p[0] : 0.0f;
    v.y = (row_ok && first + 1 < lim) ? p[1] : 0.0f;
    v.z = (row_ok && first + 2 < lim) ? p[2] : 0.0f;
    v.w = (row_ok && first + 3 < lim) ? p[3] : 0.0f;
    return v;
}

__global__ __launch_bounds__(kThreads)
void gemm_regblock_f32(int64_t M, int64_t N, int64_t K,
                       const float *__restrict__ A, int64_t lda,
                       const float *__restrict__ B, int64_t ldb,
                       float *__restrict__ C, int64_t ldc,
                       int64_t tiles_m, int64_t tiles_n,
                       int vec_a, int vec_b, int vec_c)
{
    __shared__ __attribute__((aligned(16))) float As[2][kBM * kAStride];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBK * kBStride];

    const int t = threadIdx.x;
    const int tx = t % 16, ty = t / 16;

    int64_t tm, tn;
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
    const int64_t m0 = tm * kBM, n0 = tn * kBN;

    float4 ra[kAF4], rb[kBF4];
    auto fetch = [&](int64_t k0) {
#pragma unroll
        for (int r = 0; r < kAF4; ++r) {
            const int f = t + kThreads * r;
            const int m = f / (kBK / 4), kq = f % (kBK / 4);
            const int64_t gm = m0 + m, gk = k0 + 4 * kq;
            ra[r] = load4(A + gm * lda + gk, gm < M, gk, K, vec_a);
        }
#pragma unroll
        for (int r = 0; r < kBF4; ++r) {
            const int f = t + kThreads * r;
            const int k = f / (kBN / 4), nq = f % (kBN / 4);
            const int64_t gk = k0 + k, gn = n0 + 4 * nq;
            rb[r] = load4(B + gk * ldb + gn, gk < K, gn, N, vec_b);
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int r = 0; r < kAF4; ++r) {
            const int f = t + kThreads * r;
            const int m = f / (kBK / 4), kq = f % (kBK / 4);
            *reinterpret_cast<float4 *>(&As[buf][m * kAStride + 4 * kq]) = ra[r];
        }
#pragma unroll
        for (int r = 0; r < kBF4; ++r) {
            const int f = t + kThreads * r;
            const int k = f / (kBN / 4), nq = f % (kBN / 4);
            *reinterpret_cast<float4 *>(&Bs[buf][k * kBStride + 4 * nq]) = rb[r];
        }
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    const int64_t slices = ceil_div(K, kBK);
    if (slices > 0) {
        fetch(0);
        stage(0);
        __syncthreads();
    }
    for (int64_t s = 0; s < slices; ++s) {
        const int cur = static_cast<int>(s & 1);
        if (s + 1 < slices) fetch((s + 1) * kBK);
        const float *as = As[cur];
        const float *bs = Bs[cur];
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 4) {
            float4 a4[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                a4[i] = *reinterpret_cast<const float4 *>(&as[(ty + 16 * i) * kAStride + kk]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 b0 = *reinterpret_cast<const float4 *>(&bs[(kk + q) * kBStride + 4 * tx]);
                const float4 b1 = *reinterpret_cast<const float4 *>(&bs[(kk + q) * kBStride + 64 + 4 * tx]);
                const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float a = q == 0 ? a4[i].x : q == 1 ? a4[i].y : q == 2 ? a4[i].z : a4[i].w;
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a, b[j], acc[i][j]);
                }
            }
        }
        if (s + 1 < slices) stage(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: masked stores, float4 when the row segment is whole and aligned.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t gm = m0 + ty + 16 * i;
        if (gm >= M) continue;
        float *crow = C + gm * ldc;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t gn = n0 + 64 * half + 4 * tx;
            const float *v = &acc[i][4 * half];
            if (vec_c && gn + 3 < N) {
                *reinterpret_cast<float4 *>(crow + gn) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (gn + j < N) crow[gn + j] = v[j];
            }
        }
    }
}

}  // namespace

LaunchPlan plan_regblock(int64_t M, int64_t N, int64_t /*K*/) {
    LaunchPlan p{};
    p.kernel = "gemm_regblock_f32";
    p.bm = kBM;
    p.bn = kBN;
    p.bk = kBK;
    p.grid = ceil_div(M, kBM) * ceil_div(N, kBN);
    p.block = kThreads;
    p.lds_bytes = static_cast<int>(2 * (kBM * kAStride + kBK * kBStride) * sizeof(float));
    p.split_k = 1;
    return p;
}

hipError_t launch_regblock(const GemmArgs &a) {
    const LaunchPlan p = plan_regblock(a.M, a.N, a.K);
    const int vec_a = vec4_ok(a.A, a.lda), vec_b = vec4_ok(a.B, a.ldb), vec_c = vec4_ok(a.C, a.ldc);
    hipLaunchKernelGGL(gemm_regblock_f32, dim3(static_cast<uint32_t>(p.grid)), dim3(kThreads),
                       0, a.stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc,
                       ceil_div(a.M, kBM), ceil_div(a.N, kBN), vec_a, vec_b, vec_c);
    return hipGetLastError();
}

}  // namespace tra
