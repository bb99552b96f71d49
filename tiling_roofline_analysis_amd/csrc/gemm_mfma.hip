// gemm_mfma.hip -- rung 4 of the ladder: CDNA matrix cores on binary32
// inputs (v_mfma_f32_32x32x2_f32), double-buffered LDS.
//
// This is the same tiled scheme as the pages' kernels -- C is cut into
// blocks, the K axis into slices staged in on-chip memory with zeros outside
// the matrices, partial dot products accumulate in registers and C is stored
// once when the K axis is done (page "Roofline & Tiling notes",
// legato-user-group.github.io/tensor2silicon-lab/week04/researchers/jaehyeong,
// section 3 "Tiling" and figure 5; page "GEMM kernel test code &
// optimization (1024^3 experiment)", teach-meaning.tistory.com/1513, section
// "Shared-memory tiled GEMM") -- with the per-slice inner product done by
// matrix-core instructions instead of lane FMAs.
//
// One v_mfma_f32_32x32x2_f32 multiplies a 32x2 A fragment by a 2x32 B
// fragment into a 32x32 binary32 accumulator held 16 words per lane:
//   A operand:  lane l supplies A[l % 32][h]      (h = l / 32)
//   B operand:  lane l supplies B[h][l % 32]
//   result:     lane l, word r holds C[8*(r/4) + 4*h + r%4][l % 32]
// A wave owns a WM x WN piece of the block tile as (WM/32) x (WN/32) such
// accumulators; the block has (BM/WM) x (BN/WN) waves.
//
// K order inside a slice of BK: MFMA step s (0 <= s < BK/2) gives lane half
// h the k index h*BK/2 + s.  Any bijection of k is the same sum; this one
// lets a lane fetch its A values for the whole slice as BK/2 contiguous
// words (ds_read_b128) instead of one word per step.
//
// LDS layout (per buffer):
//   As[m][k]  k contiguous, row stride BK + 4 words.  A global float4 along k
//             stores as one ds_write_b128; fragment reads (32 rows, stride
//             BK+4 = 20 words for BK = 16) fall in disjoint bank groups.
//   Bs[k][n]  n contiguous, row stride BN + 4 words, so the two lane halves
//             (rows k and k + BK/2) do not collide.
// Global loads are float4 along the contiguous axis of each operand (A: k,
// B: n) when the base is 16-byte aligned and the leading dimension is a
// multiple of 4; otherwise element loads.  Either way out-of-range elements
// are stored as zeros (exact +0 in every sum).
//
// Workgroup ids are remapped so each of the 8 XCDs runs a compact patch of
// tiles (shared L2 traffic), in groups of 8 tile rows.
#include "gemm_internal.h"

namespace tra {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

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

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    static constexpr int FM = WM / 32, FN = WN / 32;       // accumulators per wave
    // A single accumulator per wave would chain every MFMA on the previous
    // one; then alternate two accumulators and add them at the end.
    static constexpr int NACC = (FM * FN == 1) ? 2 : 1;
    static constexpr int AST = BK + 4, BST = BN + 4;       // LDS row strides (words)
    static constexpr int A_F4 = BM * BK / 4 / THREADS;     // float4 of A per lane per slice
    static constexpr int B_F4 = BK * BN / 4 / THREADS;     // float4 of B per lane per slice
    static constexpr int LDS_WORDS = 2 * (BM * AST + BK * BST);
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be 32x32 blocks");
    static_assert(BM % WM == 0 && BN % WN == 0, "block tile must be whole wave tiles");
    static_assert(BK % 8 == 0, "BK must be a multiple of 8 (b128 fragment reads)");
    static_assert(A_F4 * 4 * THREADS == BM * BK, "A slice must split evenly over lanes");
    static_assert(B_F4 * 4 * THREADS == BK * BN, "B slice must split evenly over lanes");
};

template <class T>
__global__ __launch_bounds__(T::THREADS)
void gemm_mfma_f32(int64_t M, int64_t N, int64_t K,
                   const float *__restrict__ A, int64_t lda,
                   const float *__restrict__ B, int64_t ldb,
                   float *__restrict__ C, int64_t ldc,
                   int64_t tiles_m, int64_t tiles_n, int vec_a, int vec_b)
{
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK, WM = T::WM, WN = T::WN;
    constexpr int FM = T::FM, FN = T::FN, NACC = T::NACC;
    constexpr int AST = T::AST, BST = T::BST, THREADS = T::THREADS;
    constexpr int HALF = BK / 2;

    __shared__ __attribute__((aligned(16))) float lds[T::LDS_WORDS];
    float *const As0 = lds;
    float *const Bs0 = lds + 2 * BM * AST;

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int wm0 = (wave / T::WAVES_N) * WM;
    const int wn0 = (wave % T::WAVES_N) * WN;

    int64_t tm, tn;
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;

    float4 ra[T::A_F4], rb[T::B_F4];
    auto fetch = [&](int64_t k0) {
#pragma unroll
        for (int r = 0; r < T::A_F4; ++r) {
            const int f = t + THREADS * r;
            const int m = f / (BK / 4), kq = f % (BK / 4);
            const int64_t gm = m0 + m, gk = k0 + 4 * kq;
            ra[r] = load4(A + gm * lda + gk, gm < M, gk, K, vec_a);
        }
#pragma unroll
        for (int r = 0; r < T::B_F4; ++r) {
            const int f = t + THREADS * r;
            const int k = f / (BN / 4), nq = f % (BN / 4);
            const int64_t gk = k0 + k, gn = n0 + 4 * nq;
            rb[r] = load4(B + gk * ldb + gn, gk < K, gn, N, vec_b);
        }
    };
    auto stage = [&](int buf) {
        float *as = As0 + buf * BM * AST;
        float *bs = Bs0 + buf * BK * BST;
#pragma unroll
        for (int r = 0; r < T::A_F4; ++r) {
            const int f = t + THREADS * r;
            const int m = f / (BK / 4), kq = f % (BK / 4);
            *reinterpret_cast<float4 *>(&as[m * AST + 4 * kq]) = ra[r];
        }
#pragma unroll
        for (int r = 0; r < T::B_F4; ++r) {
            const int f = t + THREADS * r;
            const int k = f / (BN / 4), nq = f % (BN / 4);
            *reinterpret_cast<float4 *>(&bs[k * BST + 4 * nq]) = rb[r];
        }
    };

    f32x16 acc[NACC][FM][FN];
#pragma unroll
    for (int c = 0; c < NACC; ++c)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[c][i][j][r] = 0.0f;

    const int64_t slices = ceil_div(K, BK);
    if (slices > 0) {
        fetch(0);
        stage(0);
        __syncthreads();
    }
    for (int64_t s = 0; s < slices; ++s) {
        const int cur = static_cast<int>(s & 1);
        if (s + 1 < slices) fetch((s + 1) * BK);
        const float *as = As0 + cur * BM * AST;
        const float *bs = Bs0 + cur * BK * BST;
        // A fragments for the whole slice: lane holds A[row][h*HALF + q].
        float af[FM][HALF];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const float *src = &as[(wm0 + 32 * i + l32) * AST + h * HALF];
#pragma unroll
            for (int q = 0; q < HALF; q += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(src + q);
                af[i][q + 0] = v.x;
                af[i][q + 1] = v.y;
                af[i][q + 2] = v.z;
                af[i][q + 3] = v.w;
            }
        }
#pragma unroll
        for (int q = 0; q < HALF; ++q) {
            float bf[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[j] = bs[(h * HALF + q) * BST + wn0 + 32 * j + l32];
            const int c = NACC == 1 ? 0 : (q & 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[c][i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][q], bf[j],
                                                                        acc[c][i][j], 0, 0, 0);
        }
        if (s + 1 < slices) stage(cur ^ 1);
        __syncthreads();
    }
    if (NACC == 2) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[0][i][j] += acc[NACC - 1][i][j];
    }

    // Epilogue: word r of accumulator (i, j) is row 8*(r/4) + 4*h + r%4,
    // column l32 of that 32x32 block.  Each store covers two 128-byte row
    // segments per wave.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t gn = n0 + wn0 + 32 * j + l32;
            if (gn >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gm = m0 + wm0 + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (gm < M) C[gm * ldc + gn] = acc[0][i][j][r];
            }
        }
    }
}

// Tile shapes.  Large: 256x128 block, 4 waves of 128x64 (8 accumulators
// each, 128 words), 2 workgroups per CU.  Small: 64x64 block, 4 waves of
// 32x32, for shapes with too few large tiles to fill 256 CUs.
using TileLarge = MfmaTile<256, 128, 16, 128, 64>;
using TileSmall = MfmaTile<64, 64, 32, 32, 32>;

constexpr int64_t kCUs = 256;

template <class T>
LaunchPlan plan_for(int64_t M, int64_t N, const char *name) {
    LaunchPlan p{};
    p.kernel = name;
    p.bm = T::BM;
    p.bn = T::BN;
    p.bk = T::BK;
    p.grid = ceil_div(M, T::BM) * ceil_div(N, T::BN);
    p.block = T::THREADS;
    p.lds_bytes = static_cast<int>(T::LDS_WORDS * sizeof(float));
    p.split_k = 1;
    return p;
}

// Large tiles when they give at least one workgroup per CU, else small.
bool use_large(int64_t M, int64_t N) {
    return ceil_div(M, TileLarge::BM) * ceil_div(N, TileLarge::BN) >= kCUs;
}

template <class T>
hipError_t launch_tile(const GemmArgs &a) {
    const int64_t tm = ceil_div(a.M, T::BM), tn = ceil_div(a.N, T::BN);
    hipLaunchKernelGGL(gemm_mfma_f32<T>, dim3(static_cast<uint32_t>(tm * tn)), dim3(T::THREADS),
                       0, a.stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, tm, tn,
                       static_cast<int>(vec4_ok(a.A, a.lda)),
                       static_cast<int>(vec4_ok(a.B, a.ldb)));
    return hipGetLastError();
}

}  // namespace

LaunchPlan plan_mfma(int64_t M, int64_t N, int64_t /*K*/) {
    return use_large(M, N) ? plan_for<TileLarge>(M, N, "gemm_mfma_f32<256x128x16, wave 128x64>")
                           : plan_for<TileSmall>(M, N, "gemm_mfma_f32<64x64x32, wave 32x32>");
}

hipError_t launch_mfma(const GemmArgs &a) {
    return use_large(a.M, a.N) ? launch_tile<TileLarge>(a) : launch_tile<TileSmall>(a);
}

}  // namespace tra
