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
//   * a 128 x 128 block tile of C (each staged element reused 128 times;
//     64 x 64 when 128 x 128 tiles would not give every CU one);
//   * each lane holds an 8 x 8 (4 x 4) micro-tile of C in VGPRs, so one LDS
//     read feeds 8 (4) FMAs instead of one;
//   * the next K slice is fetched into registers while the current one is
//     consumed from LDS, and two LDS buffers alternate, so each slice needs
//     one barrier instead of two.
//
// gfx950 layout (256 lanes = 4 wave64s, lane t: tx = t % 16, ty = t / 16),
// for the 128 x 128 tile (the 64 x 64 one keeps i < 4 and the first group):
//   rows of C held by a lane:  ty + 16*i, i = 0..7
//   columns held by a lane:    4*tx + j and 64 + 4*tx + j, j = 0..3
//   As[m][k]  k contiguous, row stride 20 words (16 + 4): a wave reads 4
//             consecutive rows at once (one ds_read_b128 each), which land
//             in 4 disjoint bank groups; global float4 rows store as-is.
//   Bs[k][n]  n contiguous, row stride 132 words: a wave reads 64
//             consecutive words per ds_read_b128.
// The arithmetic is VALU fmaf (v_fma_f32); the library is compiled with
// packed-FP32 instructions disabled, so the rung's ceiling is the unpacked FP32 VALU
// rate (about 100 TFLOP/s measured by tra_probe_fma_f32 on MI355X), below
// the 157.3 TFLOP/s FP32 peak that the matrix cores reach.
#include "gemm_internal.h"

namespace tra {
namespace {

// A block tile of BM x BN with a TM x TN micro-tile per lane; lane t holds
// rows ty + 16*i (i < TM) and columns 64*g + 4*tx + j (g < TN/4, j < 4),
// tx = t % 16, ty = t / 16 -- so BM = 16*TM, and BN = 16*TN with the
// columns in groups of 4 at 64-column strides.
template <int BM_, int BN_, int TM_, int TN_>
struct RegTile {
    static constexpr int BM = BM_, BN = BN_, BK = 16, TM = TM_, TN = TN_;
    static constexpr int THREADS = 256;
    static constexpr int AST = BK + 4;    // words per As row
    static constexpr int BST = BN + 4;    // words per Bs row
    static constexpr int AF4 = BM * BK / 4 / THREADS;   // float4 of A per lane per slice
    static constexpr int BF4 = BK * BN / 4 / THREADS;   // float4 of B per lane per slice
    static_assert(BM == 16 * TM && BN == 16 * TN && TN % 4 == 0, "lane layout");
    static_assert(AF4 >= 1 && BF4 >= 1, "whole float4 per lane");
};

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

template <class T>
__global__ __launch_bounds__(T::THREADS)
void gemm_regblock_f32(int64_t M, int64_t N, int64_t K,
                       const float *__restrict__ A, int64_t lda,
                       const float *__restrict__ B, int64_t ldb,
                       float *__restrict__ C, int64_t ldc,
                       int64_t tiles_m, int64_t tiles_n,
                       int vec_a, int vec_b, int vec_c)
{
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK, TM = T::TM, TN = T::TN;
    constexpr int AST = T::AST, BST = T::BST;
    __shared__ __attribute__((aligned(16))) float As[2][BM * AST];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * BST];

    const int t = threadIdx.x;
    const int tx = t % 16, ty = t / 16;

    int64_t tm, tn;
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;

    float4 ra[T::AF4], rb[T::BF4];
    auto fetch = [&](int64_t k0) {
#pragma unroll
        for (int r = 0; r < T::AF4; ++r) {
            const int f = t + T::THREADS * r;
            const int m = f / (BK / 4), kq = f % (BK / 4);
            const int64_t gm = m0 + m, gk = k0 + 4 * kq;
            ra[r] = load4(A + gm * lda + gk, gm < M, gk, K, vec_a);
        }
#pragma unroll
        for (int r = 0; r < T::BF4; ++r) {
            const int f = t + T::THREADS * r;
            const int k = f / (BN / 4), nq = f % (BN / 4);
            const int64_t gk = k0 + k, gn = n0 + 4 * nq;
            rb[r] = load4(B + gk * ldb + gn, gk < K, gn, N, vec_b);
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int r = 0; r < T::AF4; ++r) {
            const int f = t + T::THREADS * r;
            const int m = f / (BK / 4), kq = f % (BK / 4);
            *reinterpret_cast<float4 *>(&As[buf][m * AST + 4 * kq]) = ra[r];
        }
#pragma unroll
        for (int r = 0; r < T::BF4; ++r) {
            const int f = t + T::THREADS * r;
            const int k = f / (BN / 4), nq = f % (BN / 4);
            *reinterpret_cast<float4 *>(&Bs[buf][k * BST + 4 * nq]) = rb[r];
        }
    };

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    const int64_t slices = ceil_div(K, BK);
    if (slices > 0) {
        fetch(0);
        stage(0);
        __syncthreads();
    }
    for (int64_t s = 0; s < slices; ++s) {
        const int cur = static_cast<int>(s & 1);
        if (s + 1 < slices) fetch((s + 1) * BK);
        const float *as = As[cur];
        const float *bs = Bs[cur];
#pragma unroll
        for (int kk = 0; kk < BK; kk += 4) {
            float4 a4[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a4[i] = *reinterpret_cast<const float4 *>(&as[(ty + 16 * i) * AST + kk]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float b[TN];
#pragma unroll
                for (int g = 0; g < TN / 4; ++g) {
                    const float4 v =
                        *reinterpret_cast<const float4 *>(&bs[(kk + q) * BST + 64 * g + 4 * tx]);
                    b[4 * g + 0] = v.x;
                    b[4 * g + 1] = v.y;
                    b[4 * g + 2] = v.z;
                    b[4 * g + 3] = v.w;
                }
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const float a = q == 0 ? a4[i].x : q == 1 ? a4[i].y : q == 2 ? a4[i].z : a4[i].w;
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a, b[j], acc[i][j]);
                }
            }
        }
        if (s + 1 < slices) stage(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: masked stores, float4 when the row segment is whole and aligned.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t gm = m0 + ty + 16 * i;
        if (gm >= M) continue;
        float *crow = C + gm * ldc;
#pragma unroll
        for (int g = 0; g < TN / 4; ++g) {
            const int64_t gn = n0 + 64 * g + 4 * tx;
            const float *v = &acc[i][4 * g];
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

// 128 x 128 tiles with 8 x 8 micro-tiles; 64 x 64 tiles with 4 x 4 when the
// large tiles would leave CUs idle (fewer than one per CU: 1024^3 has 64).
using RegLarge = RegTile<128, 128, 8, 8>;
using RegSmall = RegTile<64, 64, 4, 4>;

constexpr int64_t kCUs = 256;

bool small_tiles(int64_t M, int64_t N) {
    return ceil_div(M, RegLarge::BM) * ceil_div(N, RegLarge::BN) < kCUs;
}

template <class T>
LaunchPlan plan_reg(int64_t M, int64_t N, const char *name) {
    LaunchPlan p{};
    p.kernel = name;
    p.bm = T::BM;
    p.bn = T::BN;
    p.bk = T::BK;
    p.grid = ceil_div(M, T::BM) * ceil_div(N, T::BN);
    p.block = T::THREADS;
    p.lds_bytes = static_cast<int>(2 * (T::BM * T::AST + T::BK * T::BST) * sizeof(float));
    p.split_k = 1;
    return p;
}

template <class T>
hipError_t launch_reg(const GemmArgs &a) {
    const int64_t tm = ceil_div(a.M, T::BM), tn = ceil_div(a.N, T::BN);
    const int vec_a = vec4_ok(a.A, a.lda), vec_b = vec4_ok(a.B, a.ldb), vec_c = vec4_ok(a.C, a.ldc);
    hipLaunchKernelGGL(gemm_regblock_f32<T>, dim3(static_cast<uint32_t>(tm * tn)),
                       dim3(T::THREADS), 0, a.stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb,
                       a.C, a.ldc, tm, tn, vec_a, vec_b, vec_c);
    return hipGetLastError();
}

}  // namespace

LaunchPlan plan_regblock(int64_t M, int64_t N, int64_t /*K*/) {
    return small_tiles(M, N) ? plan_reg<RegSmall>(M, N, "gemm_regblock_f32<64x64, 4x4>")
                             : plan_reg<RegLarge>(M, N, "gemm_regblock_f32<128x128, 8x8>");
}

hipError_t launch_regblock(const GemmArgs &a) {
    return small_tiles(a.M, a.N) ? launch_reg<RegSmall>(a) : launch_reg<RegLarge>(a);
}

}  // namespace tra
