// gemm_mfma.hip -- rung 4 of the ladder: CDNA matrix cores on binary32
// inputs (v_mfma_f32_32x32x2_f32), software-pipelined LDS staging.
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
// accumulators; the block has (BM/WM) x (BN/WN) waves per K group.
//
// K groups (KG): the waves of a block form KG groups; group g takes the k
// range [g*BK/KG, (g+1)*BK/KG) of every slice, and at the end groups
// 1..KG-1 hand their partial sums to group 0 through LDS, added in group
// order (deterministic).  More waves per CU without smaller tiles.
//
// K order inside a group's part of a slice (SUB = BK/KG wide): MFMA step q
// (0 <= q < SUB/2) gives lane half h the k index g*SUB + h*SUB/2 + q.  Any
// bijection of k is the same sum; this one lets a lane fetch its A values for
// the slice as contiguous words (ds_read_b128) instead of one per step.
//
// LDS layout (two buffers):
//   As[m][k]  k contiguous, row stride BK + 4 words: a global float4 along k
//             stores as one ds_write_b128, and 8 consecutive rows read by
//             ds_read_b128 fall in disjoint bank groups.
//   Bs[k][n]  n contiguous, row stride BN + 4 words.
//
// Pipeline (slice s lives in LDS buffer s % 2; NR register sets hold the
// slices fetched from global memory but not yet stored to LDS):
//   iteration s:  read the fragments of slice s+1 from LDS;
//                 store slice s+2 (registers) into buffer s % 2;
//                 fetch slice s+2+NR from global memory into the freed set;
//                 run the MFMAs of slice s from registers;  barrier.
// Each global load has NR iterations to arrive and every LDS access of an
// iteration overlaps that iteration's MFMAs.
//
// Global loads: whole tiles with 16-byte-aligned rows (base aligned, ld a
// multiple of 4) use float4 loads without checks, whole tiles of unaligned
// operands element loads without checks; edge tiles load elements at
// clamped, always-valid addresses and select zero outside the matrices (no
// branches).  Out-of-range elements are +0 in every sum.
//
// Workgroup ids are remapped so each of the 8 XCDs runs a compact patch of
// tiles (shared L2 traffic), in groups of 8 tile rows.
#include "gemm_internal.h"

namespace tra {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WM_, int WN_, int KG_, int NR_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int KG = KG_;                         // K groups of waves
    static constexpr int NR = NR_;                         // register sets in flight
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int WAVES = WAVES_M * WAVES_N;        // waves per K group
    static constexpr int THREADS = 64 * WAVES * KG;
    static constexpr int FM = WM / 32, FN = WN / 32;       // accumulators per wave
    static constexpr int SUB = BK / KG, HALF = SUB / 2;    // k per group per slice
    static constexpr int AST = BK + 4, BST = BN + 4;       // LDS row strides (words)
    static constexpr int A_VEC = BM * BK / 4, B_VEC = BK * BN / 4;   // float4 per slice
    static constexpr int A_F4 = (A_VEC + THREADS - 1) / THREADS;     // per lane
    static constexpr int B_F4 = (B_VEC + THREADS - 1) / THREADS;
    static constexpr int STAGE_WORDS = 2 * (BM * AST + BK * BST);
    static constexpr int RED_WORDS = (KG - 1) * BM * BN;            // K-group hand-off
    static constexpr int LDS_WORDS = STAGE_WORDS > RED_WORDS ? STAGE_WORDS : RED_WORDS;
    static constexpr int UNROLL = NR == 4 ? 4 : 2;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be 32x32 blocks");
    static_assert(BM % WM == 0 && BN % WN == 0, "block tile must be whole wave tiles");
    static_assert(HALF % 4 == 0, "each lane half needs a multiple of 4 k per slice");
    static_assert(BK % 4 == 0 && BN % 4 == 0, "float4 staging");
    static_assert(NR == 1 || NR == 2 || NR == 4, "1, 2 or 4 register sets");
};

// X[row][col .. col+3] of a rows x cols row-major matrix, zero outside it.
// Addresses are clamped into the matrix, so every load is valid, and the
// zero is applied with an AND mask on the loaded bits: the loads are
// unconditional (a select would let the compiler predicate each load behind
// a branch and wait for it).
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

template <class T>
struct Ctx {
    int64_t M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    int64_t m0, n0;
    int t;
};

// How a slice is loaded from global memory.
//   kVec     whole tile inside the matrices, 16-byte-aligned rows: float4
//            loads, no checks;
//   kScalar  whole tile inside, rows not 16-byte aligned: four element
//            loads per group, no checks;
//   kEdge    the tile crosses an edge of A or B: element loads at clamped
//            addresses, zero selected outside.
enum LoadMode { kVec = 0, kScalar = 1, kEdge = 2 };

__device__ __forceinline__ float4 load4_scalar(const float *p) {
    return make_float4(p[0], p[1], p[2], p[3]);
}

// Loads slice k0 .. k0+BK of the A and B tiles into registers.
template <class T, int MODE>
__device__ __forceinline__ void fetch(const Ctx<T> &c, int64_t k0, float4 (&ra)[T::A_F4],
                                      float4 (&rb)[T::B_F4]) {
#pragma unroll
    for (int r = 0; r < T::A_F4; ++r) {
        const int f = c.t + T::THREADS * r;
        if (T::A_VEC % T::THREADS != 0 && f >= T::A_VEC) break;
        const int m = f / (T::BK / 4), kq = f % (T::BK / 4);
        const float *p = c.A + (c.m0 + m) * c.lda + k0 + 4 * kq;
        if (MODE == kVec) ra[r] = *reinterpret_cast<const float4 *>(p);
        else if (MODE == kScalar) ra[r] = load4_scalar(p);
        else ra[r] = load4_clamped(c.A, c.lda, c.m0 + m, k0 + 4 * kq, c.M, c.K);
    }
#pragma unroll
    for (int r = 0; r < T::B_F4; ++r) {
        const int f = c.t + T::THREADS * r;
        if (T::B_VEC % T::THREADS != 0 && f >= T::B_VEC) break;
        const int k = f / (T::BN / 4), nq = f % (T::BN / 4);
        const float *p = c.B + (k0 + k) * c.ldb + c.n0 + 4 * nq;
        if (MODE == kVec) rb[r] = *reinterpret_cast<const float4 *>(p);
        else if (MODE == kScalar) rb[r] = load4_scalar(p);
        else rb[r] = load4_clamped(c.B, c.ldb, k0 + k, c.n0 + 4 * nq, c.K, c.N);
    }
}

// Stores one slice from registers into LDS buffer `buf`.
template <class T>
__device__ __forceinline__ void stage(float *lds, int buf, int t, const float4 (&ra)[T::A_F4],
                                      const float4 (&rb)[T::B_F4]) {
    float *as = lds + buf * T::BM * T::AST;
    float *bs = lds + 2 * T::BM * T::AST + buf * T::BK * T::BST;
#pragma unroll
    for (int r = 0; r < T::A_F4; ++r) {
        const int f = t + T::THREADS * r;
        if (T::A_VEC % T::THREADS != 0 && f >= T::A_VEC) break;
        const int m = f / (T::BK / 4), kq = f % (T::BK / 4);
        *reinterpret_cast<float4 *>(&as[m * T::AST + 4 * kq]) = ra[r];
    }
#pragma unroll
    for (int r = 0; r < T::B_F4; ++r) {
        const int f = t + T::THREADS * r;
        if (T::B_VEC % T::THREADS != 0 && f >= T::B_VEC) break;
        const int k = f / (T::BN / 4), nq = f % (T::BN / 4);
        *reinterpret_cast<float4 *>(&bs[k * T::BST + 4 * nq]) = rb[r];
    }
}

template <class T>
struct Frag {
    float a[T::FM][T::HALF];   // A[row][kbase + q]
    float b[T::HALF][T::FN];   // B[kbase + q][col]
};

template <class T>
__device__ __forceinline__ void read_frags(const float *lds, int buf, int arow, int bcol,
                                           int kbase, Frag<T> &fr) {
    const float *as = lds + buf * T::BM * T::AST;
    const float *bs = lds + 2 * T::BM * T::AST + buf * T::BK * T::BST;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        const float *src = &as[(arow + 32 * i) * T::AST + kbase];
#pragma unroll
        for (int q = 0; q < T::HALF; q += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(src + q);
            fr.a[i][q + 0] = v.x;
            fr.a[i][q + 1] = v.y;
            fr.a[i][q + 2] = v.z;
            fr.a[i][q + 3] = v.w;
        }
    }
#pragma unroll
    for (int q = 0; q < T::HALF; ++q)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) fr.b[q][j] = bs[(kbase + q) * T::BST + bcol + 32 * j];
}

// MFMA steps q0 .. q1-1 of one slice.
template <class T, int q0, int q1>
__device__ __forceinline__ void mfmas(const Frag<T> &fr, f32x16 (&acc)[T::FM][T::FN]) {
#pragma unroll
    for (int q = q0; q < q1; ++q)
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fr.a[i][q], fr.b[q][j],
                                                                 acc[i][j], 0, 0, 0);
}

// The K loop of one block tile.  MODE applies to the full slices; the k tail
// slice (K not a multiple of BK) always takes edge loads.
template <class T, int MODE>
__device__ __forceinline__ void k_loop(const Ctx<T> &c, float *lds, int arow, int bcol,
                                       int kbase, f32x16 (&acc)[T::FM][T::FN]) {
    constexpr int BK = T::BK, NR = T::NR, U = T::UNROLL;
    const int64_t slices = ceil_div(c.K, BK);
    const int64_t full = c.K / BK;            // slices with no k tail
    if (slices == 0) return;

    float4 ra[NR][T::A_F4], rb[NR][T::B_F4];
    Frag<T> fr[2];
    auto fetch_any = [&](int64_t j, int set) {
        if (MODE != kEdge && j < full) fetch<T, MODE>(c, j * BK, ra[set], rb[set]);
        else fetch<T, kEdge>(c, j * BK, ra[set], rb[set]);
    };

    // Prologue: slices 0 and 1 into LDS (loaded together when there are two
    // register sets), slices 2 .. NR+1 into registers, fragments of slice 0
    // into fr[0].
    fetch_any(0, 0);
    if (NR >= 2 && slices > 1) fetch_any(1, 1);
    stage<T>(lds, 0, c.t, ra[0], rb[0]);
    if (slices > 1) {
        if (NR < 2) fetch_any(1, 0);
        stage<T>(lds, 1, c.t, ra[1 % NR], rb[1 % NR]);
    }
#pragma unroll
    for (int j = 2; j < NR + 2; ++j)
        if (j < slices) fetch_any(j, j % NR);
    __syncthreads();
    read_frags<T>(lds, 0, arow, bcol, kbase, fr[0]);
    __syncthreads();   // buffer 0 is rewritten in iteration 0

    // Iteration s: fragment set s % 2, register set of slice s+2 is
    // (s+2) % NR.  `guarded` only in the last few iterations.  The order is
    // pinned with scheduling barriers: the fragment reads, the first half of
    // the MFMAs, the LDS stores and global loads, the second half of the
    // MFMAs, the workgroup barrier.  (Left alone, the compiler sinks the
    // MFMAs below the workgroup barrier, which makes them wait for the
    // global loads and LDS stores instead of covering them.)
    auto step = [&](int64_t s, int fp, int rp, bool guarded) {
        if (!guarded || s + 1 < slices) read_frags<T>(lds, fp ^ 1, arow, bcol, kbase, fr[fp ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfmas<T, 0, T::HALF / 2>(fr[fp], acc);
        __builtin_amdgcn_sched_barrier(0);
        if (!guarded || s + 2 < slices) {
            stage<T>(lds, fp, c.t, ra[rp], rb[rp]);
            if (!guarded) fetch<T, MODE>(c, (s + 2 + NR) * BK, ra[rp], rb[rp]);
            else if (s + 2 + NR < slices) fetch_any(s + 2 + NR, rp);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfmas<T, T::HALF / 2, T::HALF>(fr[fp], acc);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    const int64_t limit = MODE != kEdge ? full : slices;   // the main loop fetches below this
    int64_t s = 0;
    for (; s + U - 1 + 2 + NR < limit; s += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(s + u, u & 1, (u + 2) % NR, false);
    }
    // Tail: the last few slices, with checks.  s is a multiple of U here.
    for (; s < slices; s += U) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s + u < slices) step(s + u, u & 1, (u + 2) % NR, true);
    }
}

template <class T>
__global__ __launch_bounds__(T::THREADS)
void gemm_mfma_f32(int64_t M, int64_t N, int64_t K,
                   const float *__restrict__ A, int64_t lda,
                   const float *__restrict__ B, int64_t ldb,
                   float *__restrict__ C, int64_t ldc,
                   int64_t tiles_m, int64_t tiles_n, int vec_a, int vec_b)
{
    constexpr int BM = T::BM, BN = T::BN, WM = T::WM, WN = T::WN;
    constexpr int FM = T::FM, FN = T::FN, KG = T::KG;

    __shared__ __attribute__((aligned(16))) float lds[T::LDS_WORDS];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int grp = wave / T::WAVES;            // K group of this wave
    const int wig = wave % T::WAVES;            // wave within its group
    const int wm0 = (wig / T::WAVES_N) * WM;
    const int wn0 = (wig % T::WAVES_N) * WN;
    const int kbase = grp * T::SUB + h * T::HALF;   // this lane's first k in a slice

    int64_t tm, tn;
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const Ctx<T> c{M, N, K, A, lda, B, ldb, m0, n0, t};

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const bool whole = (m0 + BM <= M) && (n0 + BN <= N);
    if (whole && vec_a && vec_b)
        k_loop<T, kVec>(c, lds, wm0 + l32, wn0 + l32, kbase, acc);
    else if (whole)
        k_loop<T, kScalar>(c, lds, wm0 + l32, wn0 + l32, kbase, acc);
    else
        k_loop<T, kEdge>(c, lds, wm0 + l32, wn0 + l32, kbase, acc);

    if (KG > 1) {
        // K groups 1..KG-1 hand their partial sums to group 0 through LDS
        // (the K loop ended with a barrier after its last LDS read); group 0
        // adds them in group order, one 32x32 block at a time.
        constexpr int PER_WAVE = FM * FN * 16 * 64;
        if (grp > 0) {
            float *dst = lds + ((grp - 1) * T::WAVES + wig) * PER_WAVE + lane;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((i * FN + j) * 16 + r) * 64] = acc[i][j][r];
        }
        __syncthreads();
        if (grp > 0) return;
        // A rolled loop over the groups keeps one group's values live at a
        // time (unrolled, the compiler hoists every read and spills).
#pragma unroll 1
        for (int g = 1; g < KG; ++g) {
            const float *src = lds + ((g - 1) * T::WAVES + wig) * PER_WAVE + lane;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] += src[((i * FN + j) * 16 + r) * 64];
        }
    }

    // Epilogue: word r of accumulator (i, j) is row 8*(r/4) + 4*h + r%4,
    // column l32 of that 32x32 block.  Each store covers two 128-byte row
    // segments per wave.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t gn = n0 + wn0 + 32 * j + l32;
            if (whole) {
                float *cp = C + (m0 + wm0 + 32 * i + 4 * h) * ldc + gn;
#pragma unroll
                for (int r = 0; r < 16; ++r) cp[(8 * (r / 4) + (r % 4)) * ldc] = acc[i][j][r];
                __builtin_amdgcn_sched_barrier(0);   // one block's addresses live at a time
                continue;
            }
            if (gn >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gm = m0 + wm0 + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (gm < M) C[gm * ldc + gn] = acc[i][j][r];
            }
        }
    }
}

// Tile shapes (chosen by timing candidates on MI355X):
//   Large  128x128x16, 4 waves of 64x64, two register sets, 2 workgroups per
//          CU: shapes with at least 4 such tiles per CU (4096^3).
//   Many   64x64x32, 4 waves of 32x32: many small tiles and short K
//          (3000x2049x1531).
//   Few    64x64x64, four K groups of 2 waves of 32x64 (8 waves), one
//          register set: about one tile per CU or long K (1024^3,
//          16384x64x16384).
using TileLarge = MfmaTile<128, 128, 16, 64, 64, 1, 2>;
using TileMany = MfmaTile<64, 64, 32, 32, 32, 1, 2>;
using TileFew = MfmaTile<64, 64, 64, 32, 64, 4, 1>;

constexpr int64_t kCUs = 256;

enum class Shape { kLarge, kMany, kFew };

Shape pick(int64_t M, int64_t N, int64_t K) {
    const int64_t large_tiles = ceil_div(M, TileLarge::BM) * ceil_div(N, TileLarge::BN);
    if (large_tiles >= 4 * kCUs) return Shape::kLarge;
    const int64_t small_tiles = ceil_div(M, TileMany::BM) * ceil_div(N, TileMany::BN);
    if (small_tiles > 2 * kCUs && K < 4096) return Shape::kMany;
    return Shape::kFew;
}

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

LaunchPlan plan_mfma(int64_t M, int64_t N, int64_t K) {
    switch (pick(M, N, K)) {
        case Shape::kLarge: return plan_for<TileLarge>(M, N, "gemm_mfma_f32<128x128x16, 4 waves>");
        case Shape::kMany: return plan_for<TileMany>(M, N, "gemm_mfma_f32<64x64x32, 4 waves>");
        default: return plan_for<TileFew>(M, N, "gemm_mfma_f32<64x64x64, 4 K groups>");
    }
}

hipError_t launch_mfma(const GemmArgs &a) {
    switch (pick(a.M, a.N, a.K)) {
        case Shape::kLarge: return launch_tile<TileLarge>(a);
        case Shape::kMany: return launch_tile<TileMany>(a);
        default: return launch_tile<TileFew>(a);
    }
}

}  // namespace tra
