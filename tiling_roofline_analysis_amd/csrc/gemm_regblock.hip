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
//     64 x 64 when there are too few 128 x 128 tiles to give every CU two,
//     or they split unevenly over the CUs);
//   * each lane holds an 8 x 8 (4 x 4) micro-tile of C in VGPRs, so one LDS
//     read feeds 8 (4) FMAs instead of one;
//   * the next K slice is fetched into registers while the current one is
//     consumed from LDS, and two LDS buffers alternate, so each slice needs
//     one barrier instead of two;
//   * a tile at the bottom or right edge is moved back inside the matrix
//     (tile_origin), so full slices load with no bounds checks; only the
//     slice that runs past K, and matrices smaller than a tile, load with
//     checks;
//   * with no more 64 x 64 tiles than CUs (1024^3), one 256-lane workgroup
//     per tile would leave one wave per SIMD to hide the latencies of a
//     VALU loop; there the tile's workgroup has 2-4 lane groups, each
//     running an equal share of the K slices in LDS buffers of its own, and
//     their partial tiles are added in a fixed order at the end.
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
// packed-FP32 instructions disabled, so the rung's ceiling is the unpacked
// FP32 VALU rate (about 100 TFLOP/s measured by tra_probe_fma_f32 on
// MI355X), below the 157.3 TFLOP/s FP32 peak that the matrix cores reach.
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

struct RbCtx {
    int64_t M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    int64_t m0, n0;   // the tile's corner (placed by tile_origin)
    int t;
};

// Loads slice k0 .. k0+BK of the A and B tiles into registers, in MODE.
// Staging slot f moves quad kq of row m of A (BK = 16: four quads a row).
// Plain: four consecutive slots take the four quads of one row and 16
// consecutive slots four consecutive rows, whose LDS stores (rows 20 words
// apart) put rows a and a+3 in the same banks: 0.26 conflict cycles per LDS
// instruction.  SPREAD: the 16 slots take rows a, a+4, a+8 and a+12 of a
// 16-row group, which start in bank groups 5a, 5a+4, 5a+8 and 5a+12 (mod
// 16): no conflict, and each row is still read as one 64-byte segment by
// four consecutive lanes.  The index costs registers the 256-lane kernels
// cannot spare (the 64x64 kernel went from 80 to 86 VGPRs, a wave less per
// SIMD: 2048^3 7% and 3000 x 2049 x 1531 4.5% slower); the K-split kernel,
// one workgroup a CU, takes it (1024^3 32.6 -> 30.7 us).  The same map
// written through a helper function compiled the K-split kernel's loop
// with other registers and gained nothing, so it is written out here.
template <class T, int MODE, bool SPREAD>
__device__ __forceinline__ void rb_fetch(const RbCtx &c, int64_t k0, float4 (&ra)[T::AF4],
                                         float4 (&rb)[T::BF4]) {
    constexpr int BK = T::BK, BN = T::BN;
    static_assert(BK == 16 && T::BM % 16 == 0, "four quads a row, rows in groups of 16");
#pragma unroll
    for (int r = 0; r < T::AF4; ++r) {
        const int f = c.t + T::THREADS * r;
        const int m = SPREAD ? (f >> 6) * 16 + ((f >> 4) & 3) + 4 * ((f >> 2) & 3) : f / (BK / 4),
                  kq = SPREAD ? f & 3 : f % (BK / 4);
        const float *p = c.A + (c.m0 + m) * c.lda + k0 + 4 * kq;
        if (MODE == kVec || MODE == kVecA) ra[r] = *reinterpret_cast<const float4 *>(p);
        else if (MODE == kScalar) ra[r] = load4_scalar(p);
        else ra[r] = load4_clamped(c.A, c.lda, c.m0 + m, k0 + 4 * kq, c.M, c.K);
    }
#pragma unroll
    for (int r = 0; r < T::BF4; ++r) {
        const int f = c.t + T::THREADS * r;
        const int k = f / (BN / 4), nq = f % (BN / 4);
        const float *p = c.B + (k0 + k) * c.ldb + c.n0 + 4 * nq;
        if (MODE == kVec) rb[r] = *reinterpret_cast<const float4 *>(p);
        else if (MODE == kVecA || MODE == kScalar) rb[r] = load4_scalar(p);
        else rb[r] = load4_clamped(c.B, c.ldb, k0 + k, c.n0 + 4 * nq, c.K, c.N);
    }
}

template <class T, bool SPREAD>
__device__ __forceinline__ void rb_stage(float *as, float *bs, int t, const float4 (&ra)[T::AF4],
                                         const float4 (&rb)[T::BF4]) {
    constexpr int BK = T::BK, BN = T::BN;
#pragma unroll
    for (int r = 0; r < T::AF4; ++r) {
        const int f = t + T::THREADS * r;
        const int m = SPREAD ? (f >> 6) * 16 + ((f >> 4) & 3) + 4 * ((f >> 2) & 3) : f / (BK / 4),
                  kq = SPREAD ? f & 3 : f % (BK / 4);
        *reinterpret_cast<float4 *>(&as[m * T::AST + 4 * kq]) = ra[r];
    }
#pragma unroll
    for (int r = 0; r < T::BF4; ++r) {
        const int f = t + T::THREADS * r;
        const int k = f / (BN / 4), nq = f % (BN / 4);
        *reinterpret_cast<float4 *>(&bs[k * T::BST + 4 * nq]) = rb[r];
    }
}

// acc += the slice held in LDS (as, bs): each LDS read of 4 k of A feeds
// TN FMAs per k, each read of 4 columns of B feeds TM.
template <class T>
__device__ __forceinline__ void rb_compute(const float *as, const float *bs, int tx, int ty,
                                           float (&acc)[T::TM][T::TN]) {
    constexpr int BK = T::BK, TM = T::TM, TN = T::TN;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
        float4 a4[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a4[i] = *reinterpret_cast<const float4 *>(&as[(ty + 16 * i) * T::AST + kk]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float b[TN];
#pragma unroll
            for (int g = 0; g < TN / 4; ++g) {
                const float4 v =
                    *reinterpret_cast<const float4 *>(&bs[(kk + q) * T::BST + 64 * g + 4 * tx]);
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
        // The 8 x 8 micro-tile is issued one group of 4 k at a time (4096^3:
        // 2651 -> 1573 us against leaving the order to the compiler); the
        // 4 x 4 one runs better without the fence (1024^3: 53.5 against
        // 55.6 us).
        if constexpr (TM * TN >= 64) __builtin_amdgcn_sched_barrier(0);
    }
}

// The K loop of one tile: all of K, or with RANGE the slices s0 .. s0+n-1
// (n >= 1; at most the last of them runs past K).  Slices that lie wholly
// inside K load in MODE with no checks and no branch in the loop; the slice
// that runs past K (if any) loads with checks.  A call makes one workgroup
// barrier per slice.  (Without RANGE the first slice is 0 at compile time:
// a run-time start made the compiler's code for the whole-K loop up to 55%
// slower, at 1000^3.)
template <class T, int MODE, bool RANGE = false, bool SPREAD = false>
__device__ __forceinline__ void rb_k_loop(const RbCtx &c, float *As, float *Bs, int tx, int ty,
                                          float (&acc)[T::TM][T::TN], int64_t first = 0,
                                          int64_t count = 0) {
    constexpr int BK = T::BK;
    constexpr int AW = T::BM * T::AST, BW = BK * T::BST;   // words per LDS buffer
    const int64_t s0 = RANGE ? first : 0;
    const int64_t slices = RANGE ? count : ceil_div(c.K, BK);
    const int64_t full = RANGE ? (c.K / BK - s0 < count ? c.K / BK - s0 : count) : c.K / BK;
    if (slices <= 0) return;
    float4 ra[T::AF4], rb[T::BF4];
    if (full > 0) rb_fetch<T, MODE, SPREAD>(c, s0 * BK, ra, rb);
    else rb_fetch<T, kChecked, SPREAD>(c, s0 * BK, ra, rb);
    rb_stage<T, SPREAD>(As, Bs, c.t, ra, rb);
    __syncthreads();
    int64_t s = 0;
    for (; s + 1 < full; ++s) {
        const int cur = static_cast<int>(s & 1);
        rb_fetch<T, MODE, SPREAD>(c, (s0 + s + 1) * BK, ra, rb);
        rb_compute<T>(As + cur * AW, Bs + cur * BW, tx, ty, acc);
        rb_stage<T, SPREAD>(As + (cur ^ 1) * AW, Bs + (cur ^ 1) * BW, c.t, ra, rb);
        __syncthreads();
    }
    // One or two slices are left: slice s, and the slice past K if there
    // is one.  (Written out rather than as a loop: as a loop it made the
    // compiler keep two slices' worth of values live and spill the 8 x 8
    // tile's registers.)
    if (s + 1 < slices) {
        const int cur = static_cast<int>(s & 1);
        rb_fetch<T, kChecked, SPREAD>(c, (s0 + s + 1) * BK, ra, rb);
        rb_compute<T>(As + cur * AW, Bs + cur * BW, tx, ty, acc);
        rb_stage<T, SPREAD>(As + (cur ^ 1) * AW, Bs + (cur ^ 1) * BW, c.t, ra, rb);
        __syncthreads();
        ++s;
    }
    const int cur = static_cast<int>(s & 1);
    rb_compute<T>(As + cur * AW, Bs + cur * BW, tx, ty, acc);
}

// Stores rows and columns of the tile at o that it owns (a moved tile's
// first skip_m rows and skip_n columns belong to the tile before it): the
// float4 v = C[o.m0 + r][o.n0 + col .. col+3], as one store where all four
// columns are owned, in range and aligned.
__device__ __forceinline__ void rb_store4(float *C, int64_t ldc, int64_t M, int64_t N,
                                          const Origin &o, int r, int col, float4 v, int vec_c) {
    const int64_t gm = o.m0 + r, gn = o.n0 + col;
    if (r < o.skip_m || gm >= M) return;
    float *crow = C + gm * ldc;
    if (vec_c && col >= o.skip_n && gn + 3 < N && (gn & 3) == 0) {
        *reinterpret_cast<float4 *>(crow + gn) = v;
    } else {
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (col + j >= o.skip_n && gn + j < N) crow[gn + j] = e[j];
    }
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
    constexpr int BM = T::BM, BN = T::BN, TM = T::TM, TN = T::TN;
    __shared__ __attribute__((aligned(16))) float As[2 * BM * T::AST];
    __shared__ __attribute__((aligned(16))) float Bs[2 * T::BK * T::BST];
    lds_poison(As, 2 * BM * T::AST);
    lds_poison(Bs, 2 * T::BK * T::BST);

    const int t = threadIdx.x;
    const int tx = t % 16, ty = t / 16;

    int64_t tm, tn;
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
    const Origin o = tile_origin<BM, BN>(tm, tn, M, N);
    const RbCtx c{M, N, K, A, lda, B, ldb, o.m0, o.n0, t};

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    const bool inside = o.m0 + BM <= M && o.n0 + BN <= N;
    if (!inside) rb_k_loop<T, kChecked>(c, As, Bs, tx, ty, acc);
    else if (vec_a && vec_b && (o.n0 & 3) == 0) rb_k_loop<T, kVec>(c, As, Bs, tx, ty, acc);
    else if (vec_a) rb_k_loop<T, kVecA>(c, As, Bs, tx, ty, acc);
    else rb_k_loop<T, kScalar>(c, As, Bs, tx, ty, acc);

    // Epilogue: rows and columns of the tile that it owns (a moved tile's
    // first skip_m rows and skip_n columns belong to the tile before it),
    // float4 stores where four columns are owned, in range and aligned.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = ty + 16 * i;
        const int64_t gm = o.m0 + r;
        if (r < o.skip_m || gm >= M) continue;
        float *crow = C + gm * ldc;
#pragma unroll
        for (int g = 0; g < TN / 4; ++g) {
            const int col = 64 * g + 4 * tx;
            const int64_t gn = o.n0 + col;
            const float *v = &acc[i][4 * g];
            if (vec_c && col >= o.skip_n && gn + 3 < N && (gn & 3) == 0) {
                *reinterpret_cast<float4 *>(crow + gn) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (col + j >= o.skip_n && gn + j < N) crow[gn + j] = v[j];
            }
        }
    }
}

// The K axis split inside one workgroup of KS x 256 lanes: lane group g
// runs the tile's slices [g n / KS, (g+1) n / KS) (n = KS x a whole number
// of slices, so every group makes the same number of barriers) in LDS
// buffers of its own, and the KS partial tiles are added in group order
// through LDS at the end.  With fewer tiles than CUs, one 256-lane
// workgroup per tile leaves each SIMD one wave to hide the LDS and memory
// latency of a VALU loop; KS groups give it KS.
template <class T, int KS>
__global__ __launch_bounds__(T::THREADS * KS)
void gemm_regblock_f32_ks(int64_t M, int64_t N, int64_t K,
                          const float *__restrict__ A, int64_t lda,
                          const float *__restrict__ B, int64_t ldb,
                          float *__restrict__ C, int64_t ldc,
                          int64_t tiles_m, int64_t tiles_n,
                          int vec_a, int vec_b, int vec_c)
{
    constexpr int BM = T::BM, BN = T::BN, TM = T::TM, TN = T::TN;
    constexpr int GW = 2 * BM * T::AST + 2 * T::BK * T::BST;   // LDS words per group
    constexpr int PST = BN + 4;                                 // partial tile row stride
    constexpr int WORDS = KS * GW > KS * BM * PST ? KS * GW : KS * BM * PST;
    static_assert(TN == 4, "one float4 of C per micro-tile row");
    __shared__ __attribute__((aligned(16))) float lds[WORDS];
    lds_poison(lds, WORDS);

    const int g = static_cast<int>(threadIdx.x) / T::THREADS;
    const int t = static_cast<int>(threadIdx.x) % T::THREADS;
    const int tx = t % 16, ty = t / 16;
    int64_t tm, tn;
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
    const Origin o = tile_origin<BM, BN>(tm, tn, M, N);
    const RbCtx c{M, N, K, A, lda, B, ldb, o.m0, o.n0, t};

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    const int64_t per = ceil_div(K, T::BK) / KS;
    float *As = lds + g * GW;
    float *Bs = As + 2 * BM * T::AST;
    const bool inside = o.m0 + BM <= M && o.n0 + BN <= N;
    if (!inside)
        rb_k_loop<T, kChecked, true, true>(c, As, Bs, tx, ty, acc, g * per, per);
    else if (vec_a && vec_b && (o.n0 & 3) == 0)
        rb_k_loop<T, kVec, true, true>(c, As, Bs, tx, ty, acc, g * per, per);
    else if (vec_a)
        rb_k_loop<T, kVecA, true, true>(c, As, Bs, tx, ty, acc, g * per, per);
    else
        rb_k_loop<T, kScalar, true, true>(c, As, Bs, tx, ty, acc, g * per, per);

    // the partial tiles, row-major with rows of PST words, then each lane
    // adds one float4 of the tile over the groups and stores it
    __syncthreads();
    float *part = lds + g * BM * PST;
#pragma unroll
    for (int i = 0; i < TM; ++i)
        *reinterpret_cast<float4 *>(&part[(ty + 16 * i) * PST + 4 * tx]) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    __syncthreads();
    constexpr int Q = BM * BN / 4;                       // float4 of C per tile
#pragma unroll
    for (int q = static_cast<int>(threadIdx.x); q < Q; q += T::THREADS * KS) {
        const int r = q / (BN / 4), col = 4 * (q % (BN / 4));
        float4 s = *reinterpret_cast<const float4 *>(&lds[r * PST + col]);
#pragma unroll
        for (int h = 1; h < KS; ++h) {
            const float4 v = *reinterpret_cast<const float4 *>(&lds[(h * BM + r) * PST + col]);
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
        rb_store4(C, ldc, M, N, o, r, col, s, vec_c);
    }
}

// 128 x 128 tiles with 8 x 8 micro-tiles, or 64 x 64 tiles with 4 x 4.
// The large tile runs best at two or more tiles per CU (three workgroups
// fit on one); it is used when there are at least 2 x 256 of them and they
// split over the CUs about as evenly as the small ones.  Measured on
// MI355X: 2048^3 (256 large tiles) 342 -> 230 us on small tiles; 3072^3
// (576 large tiles, 2.25 a CU) 877 -> 731 us; 2048x4096x2048 (512) and
// 4096^3 (1024) faster on large ones (394 against 435 us).
using RegLarge = RegTile<128, 128, 8, 8>;
using RegSmall = RegTile<64, 64, 4, 4>;

constexpr int64_t kCUs = 256;

bool small_tiles(int64_t M, int64_t N) {
    const int64_t large = ceil_div(M, RegLarge::BM) * ceil_div(N, RegLarge::BN);
    const int64_t small = ceil_div(M, RegSmall::BM) * ceil_div(N, RegSmall::BN);
    if (large < 2 * kCUs) return true;
    // rounds of tiles per CU over the ideal, for each size
    const double waste_large = static_cast<double>(ceil_div(large, kCUs) * kCUs) / large;
    const double waste_small = static_cast<double>(ceil_div(small, kCUs) * kCUs) / small;
    return waste_large > 1.1 * waste_small;
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
    return p;
}

// The in-workgroup K split, for at most one small tile per CU: the number
// of lane groups, 4, 3 or 2 (the first that cuts K's slices into equal
// runs of at least 4), or 0 for no split.  Measured on MI355X with four
// groups: 1024^3 53.7 -> 32.7 us, 1024^2 x 4096 204 -> 120 us.
int split_k_groups(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ceil_div(M, RegSmall::BM) * ceil_div(N, RegSmall::BN);
    const int64_t slices = ceil_div(K, RegSmall::BK);
    if (!small_tiles(M, N) || tiles > kCUs) return 0;
    for (int ks : {4, 3, 2})
        if (slices % ks == 0 && slices >= 4 * ks) return ks;
    return 0;
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

template <int KS>
hipError_t launch_reg_ks(const GemmArgs &a) {
    using T = RegSmall;
    const int64_t tm = ceil_div(a.M, T::BM), tn = ceil_div(a.N, T::BN);
    const int vec_a = vec4_ok(a.A, a.lda), vec_b = vec4_ok(a.B, a.ldb), vec_c = vec4_ok(a.C, a.ldc);
    hipLaunchKernelGGL((gemm_regblock_f32_ks<T, KS>), dim3(static_cast<uint32_t>(tm * tn)),
                       dim3(T::THREADS * KS), 0, a.stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb,
                       a.C, a.ldc, tm, tn, vec_a, vec_b, vec_c);
    return hipGetLastError();
}

}  // namespace

LaunchPlan plan_regblock(int64_t M, int64_t N, int64_t K) {
    static const char *const ks_names[] = {nullptr, nullptr, "gemm_regblock_f32_ks<64x64, 4x4, K in 2>",
                                           "gemm_regblock_f32_ks<64x64, 4x4, K in 3>",
                                           "gemm_regblock_f32_ks<64x64, 4x4, K in 4>"};
    if (const int ks = split_k_groups(M, N, K)) {
        LaunchPlan p = plan_reg<RegSmall>(M, N, ks_names[ks]);
        p.block = RegSmall::THREADS * ks;
        p.lds_bytes = ks * p.lds_bytes;
        return p;
    }
    return small_tiles(M, N) ? plan_reg<RegSmall>(M, N, "gemm_regblock_f32<64x64, 4x4>")
                             : plan_reg<RegLarge>(M, N, "gemm_regblock_f32<128x128, 8x8>");
}

hipError_t launch_regblock(const GemmArgs &a) {
    switch (split_k_groups(a.M, a.N, a.K)) {
        case 4: return launch_reg_ks<4>(a);
        case 3: return launch_reg_ks<3>(a);
        case 2: return launch_reg_ks<2>(a);
        default: return small_tiles(a.M, a.N) ? launch_reg<RegSmall>(a) : launch_reg<RegLarge>(a);
    }
}

}  // namespace tra
