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
// accumulators; the block has (BM/WM) x (BN/WN) waves.
//
// K order inside a slice: MFMA step q (0 <= q < BK/2) gives lane half h the
// k index h*BK/2 + q.  Any bijection of k is the same sum; this one lets a
// lane fetch its A values for the slice as contiguous words (ds_read_b128)
// instead of one per step.
//
// LDS layout (two buffers):
//   As[m][k]  k contiguous, row stride BK + 4 words: a global float4 along k
//             stores as one ds_write_b128, and 16 consecutive rows read (or
//             stored) at one k quad fall in disjoint bank groups; staging
//             spreads each group of 16 lanes' stores over all 64 banks
//             (a_quad_of).
//   Bs[k][n]  n contiguous, row stride BN + 4 words.
//
// Pipeline (slice s lives in LDS buffer s % 2; NR register sets hold the
// slices fetched from global memory but not yet stored to LDS):
//   iteration s:  read the fragments of slice s+1 from LDS;
//                 store slice s+2 (registers) into buffer s % 2;
//                 fetch slice s+2+NR from global memory into the freed set;
//                 run the MFMAs of slice s from registers;  barrier.
// Each global load has NR iterations to arrive and every LDS access of an
// iteration overlaps that iteration's MFMAs; the memory instructions are
// issued between the MFMAs (il_order) rather than in bursts.
//
// Direct staging (k_loop_dma): where every load is an aligned float4 inside
// the matrices and K is a multiple of 4 -- the common case of contiguous
// operands -- the 64 x 64 tiles move their slices from global memory
// straight into a ring of S LDS stages (buffer_load_dwordx4 ... lds), with no
// register sets and no LDS stores; the slice that runs past K, if any,
// reads a zero word for the quads past K.  The layout and the waits are
// described at Dma below.
//
// Global loads: a tile that would cross row M or column N is moved back
// inside the matrices (its rows and columns shared with the neighbouring
// tile are not stored), so full slices load without checks: float4 loads
// for 16-byte-aligned rows (base aligned, ld a multiple of 4), element
// loads otherwise.  Out-of-range elements are +0 in every sum.  The slice
// that runs past K loads elements at clamped, always-valid addresses and
// masks out the elements outside the matrices (no branches).  Full slices
// of a matrix smaller than a tile (M < BM or N < BN) load whole float4s
// when the rows are aligned and N is a multiple of 4: a quad outside the
// matrix reads a zero word instead, chosen by address, so no mask has to
// wait for the load (masking every slice where it is loaded made each
// slice wait out the memory latency: 16384x32x16384 took 1109 us, now
// 327 us).  Otherwise they load single elements, each element outside the
// matrices from the zero word.
//
// Workgroup ids are remapped so each of the 8 XCDs runs a compact patch of
// tiles (shared L2 traffic), in groups of 8 tile rows.
//
// Split along K (the tile count versus CU count trade-off of page
// "Roofline & Tiling notes", key points): the tiles of the last partial
// wave are shared out by K slice and their partial sums added in K order.
// Two forms, chosen per shape: when the split tiles fit in half a wave,
// each is cut into equal parts that run in the same launch as the
// data-parallel tiles (gemm_mfma_f32_parts, then gemm_mfma_f32_fixup);
// otherwise runs of slices that may cross tiles go to up to one wave of
// workgroups in a launch of their own (gemm_mfma_f32_sk, then the fixup at
// the start of gemm_mfma_f32) -- the decomposition of Osama et al.,
// "Stream-K: Work-centric Parallel Decomposition for Dense Matrix-Matrix
// Multiplication on the GPU", 2023.
#include "gemm_internal.h"

#include <algorithm>
#include <atomic>

namespace tra {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WM_, int WN_, int NR_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NR = NR_;                         // register sets in flight
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int FM = WM / 32, FN = WN / 32;       // accumulators per wave
    static constexpr int HALF = BK / 2;                    // MFMA steps per slice
    static constexpr int AST = BK + 4, BST = BN + 4;       // LDS row strides (words)
    static constexpr int A_VEC = BM * BK / 4, B_VEC = BK * BN / 4;   // float4 per slice
    static constexpr int A_F4 = (A_VEC + THREADS - 1) / THREADS;     // per lane
    static constexpr int B_F4 = (B_VEC + THREADS - 1) / THREADS;
    static constexpr int LDS_WORDS = 2 * (BM * AST + BK * BST);
    static constexpr int UNROLL = NR == 4 ? 4 : 2;
    // Tile rows per group of the tile order (grouped_tile).  One XCD runs 32
    // workgroups at once, one a CU; 4 rows of 256 x 128 tiles make that a
    // 1024 x 1024 block of C (A and B slices of equal size), where 8 rows
    // made it 2048 x 512 (25% more operand bytes per slice from memory).
    static constexpr int GROUP = BM == 256 ? 4 : 8;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be 32x32 blocks");
    static_assert(BM % WM == 0 && BN % WN == 0, "block tile must be whole wave tiles");
    static_assert(HALF % 4 == 0, "each lane half needs a multiple of 4 k per slice");
    static_assert(BK % 4 == 0 && BN % 4 == 0, "float4 staging");
    static_assert(NR == 1 || NR == 2 || NR == 4, "1, 2 or 4 register sets");
};

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

// The row m and k quad kq of A that staging lane-slot f moves.  Four
// consecutive slots take the four quads of one row (a contiguous 64-byte
// segment of A, one request); the 16 slots that store together take rows
// a, a+4, a+8 and a+12 of a 16-row group.  With rows BK + 4 = 20 words
// apart, row m starts at 4-bank group 5m mod 16, so those rows start at
// groups 5a, 5a+4, 5a+8 and 5a+12: four disjoint runs of four groups, all
// 64 banks once.  (Four consecutive rows instead put rows a and a+3 in the
// same banks: one conflict cycle per LDS instruction.  Giving 16
// consecutive slots one quad of 16 rows removed the conflicts too, but cost
// 2% at 1024^3 with cold caches: neighbouring lanes then read different
// rows.)
template <class T>
__device__ __forceinline__ void a_quad_of(int f, int &m, int &kq) {
    static_assert(T::BK == 16 && T::BM % 16 == 0, "4 quads per row, rows in groups of 16");
    m = (f >> 6) * 16 + ((f >> 4) & 3) + 4 * ((f >> 2) & 3);
    kq = f & 3;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A raw buffer resource over the bytes from base on (word 3, 0x00020000, is
// the 32-bit data format that gfx9 raw buffer loads take).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const float *base) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, 0x7fffffff, 0x00020000);
}

// The float4 at base + voff bytes (voff < 2^31), through a buffer resource:
// base is wave-uniform, so a slice's loads differ only in the scalar base
// and each lane's 32-bit offset stays fixed over the K loop, where a
// global load needs a 64-bit vector add per slice beside the MFMAs (4096^3
// 1.9%, 2048^3 2.2%, 2560^3 2.5% slower).  voff need only be a multiple of
// 4: rows that are not 16-byte aligned load their quads this way too, in
// place of four element loads (3000 x 2049 x 1531 +4.3%, 1024^2 x 1002
// +4.8%, 2047 x 1023 x 2047 +4.6%, 4095^3 +2.1%, but 3000^2 x 1002 -3.6%;
// four 4-byte buffer loads per quad ran a third slower than either).
__device__ __forceinline__ float4 bload4(const float *base, uint32_t voff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(base), voff, 0, 0);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

// Loads slice k0 .. k0+BK of the A and B tiles into registers.  The full-
// slice modes (kVec, kVecA, kScalar) load through buffer resources at byte
// offsets from the tile's corner, which tile_pass makes sure stay below
// 2^31.
template <class T, int MODE>
__device__ __forceinline__ void fetch(const Ctx<T> &c, int64_t k0, float4 (&ra)[T::A_F4],
                                      float4 (&rb)[T::B_F4]) {
#pragma unroll
    for (int r = 0; r < T::A_F4; ++r) {
        const int f = c.t + T::THREADS * r;
        if (T::A_VEC % T::THREADS != 0 && f >= T::A_VEC) break;
        int m, kq;
        a_quad_of<T>(f, m, kq);
        if (MODE == kVec || MODE == kVecA || MODE == kScalar)
            ra[r] = bload4(c.A + c.m0 * c.lda + k0,
                           static_cast<uint32_t>((m * c.lda + 4 * kq) * 4));
        else if (MODE == kEdge)
            ra[r] = load4_quad(c.A, c.lda, c.m0 + m, k0 + 4 * kq, c.m0 + m < c.M);
        else if (MODE == kEdgeElem)
            ra[r] = load4_elems(c.A, c.lda, c.m0 + m, k0 + 4 * kq, c.m0 + m < c.M, c.K);
        else ra[r] = load4_clamped(c.A, c.lda, c.m0 + m, k0 + 4 * kq, c.M, c.K);
    }
#pragma unroll
    for (int r = 0; r < T::B_F4; ++r) {
        const int f = c.t + T::THREADS * r;
        if (T::B_VEC % T::THREADS != 0 && f >= T::B_VEC) break;
        const int k = f / (T::BN / 4), nq = f % (T::BN / 4);
        if (MODE == kVec || MODE == kVecA || MODE == kScalar)
            rb[r] = bload4(c.B + k0 * c.ldb + c.n0,
                           static_cast<uint32_t>((k * c.ldb + 4 * nq) * 4));
        else if (MODE == kEdge)
            rb[r] = load4_quad(c.B, c.ldb, k0 + k, c.n0 + 4 * nq, c.n0 + 4 * nq < c.N);
        else if (MODE == kEdgeElem)
            rb[r] = load4_elems(c.B, c.ldb, k0 + k, c.n0 + 4 * nq, true, c.N);
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
        int m, kq;
        a_quad_of<T>(f, m, kq);
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

// Issue order of one full iteration: each MFMA of the slice is followed by
// a share of the memory instructions -- the LDS reads of the next slice's
// fragments after the first half of the MFMAs, the LDS stores and global
// loads after the second half -- so that no burst of memory instructions
// leaves the matrix pipe idle.  (Measured against issuing them in blocks
// between the halves: 1-16% faster on every tile shape.)
template <int I, int NM, int RPM, int WPM, int VPM>
__device__ __forceinline__ void il_schedule() {
    if constexpr (I < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
        if constexpr (I < NM / 2) {
            __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);    // LDS reads
        } else {
            __builtin_amdgcn_sched_group_barrier(0x200, WPM, 0);    // LDS stores
            __builtin_amdgcn_sched_group_barrier(0x020, VPM, 0);    // global loads
        }
        il_schedule<I + 1, NM, RPM, WPM, VPM>();
    }
}

template <class T, int MODE>
__device__ __forceinline__ void il_order() {
    constexpr int NM = T::HALF * T::FM * T::FN;
    constexpr int FIRST = NM / 2 > 0 ? NM / 2 : 1;
    constexpr int SECOND = NM - NM / 2 > 0 ? NM - NM / 2 : 1;
    constexpr int NDR = T::FM * (T::HALF / 4) + (T::HALF * T::FN + 1) / 2;
    constexpr int NDW = T::A_F4 + T::B_F4;
    constexpr int NVM = (MODE == kEdgeElem || MODE == kChecked ? 4 : 1) * (T::A_F4 + T::B_F4);
    il_schedule<0, NM, (NDR + FIRST - 1) / FIRST, (NDW + SECOND - 1) / SECOND,
                (NVM + SECOND - 1) / SECOND>();
}

// The K loop over slices s0 .. s0+n-1 of one block tile (n >= 1).  Full
// slices load in MODE; the slice that runs past K (the last one when K is
// not a multiple of BK) loads with every index checked.
template <class T, int MODE>
__device__ __forceinline__ void k_loop(const Ctx<T> &c, float *lds, int arow, int bcol,
                                       int kbase, f32x16 (&acc)[T::FM][T::FN], int64_t s0,
                                       int64_t n) {
    constexpr int BK = T::BK, NR = T::NR, U = T::UNROLL;
    const int64_t full = c.K / BK - s0;        // slices s0+j, j < full, are full
    const int64_t limit = full < n ? full : n;

    float4 ra[NR][T::A_F4], rb[NR][T::B_F4];
    Frag<T> fr[2];
    auto fetch_any = [&](int64_t j, int set) {
        if (j < limit) fetch<T, MODE>(c, (s0 + j) * BK, ra[set], rb[set]);
        else fetch<T, kChecked>(c, (s0 + j) * BK, ra[set], rb[set]);
    };

    // Iteration s: fragment set s % 2, register set of slice s+2 is
    // (s+2) % NR.  Each iteration reads the fragments of slice s+1, runs
    // the MFMAs of slice s, stores slice s+2 to LDS, fetches slice s+2+NR
    // and ends at a workgroup barrier.  Full iterations are issued in the
    // interleaved order of il_order; the last few (`guarded`, with checks)
    // in blocks pinned by scheduling barriers: the fragment reads, half the
    // MFMAs, the LDS stores and global loads, the other half.  (Left alone,
    // the compiler sinks the MFMAs below the workgroup barrier, which makes
    // them wait for the global loads and LDS stores instead of covering
    // them.)
    auto step = [&](int64_t s, int fp, int rp, bool guarded) {
        if (!guarded) {
            __builtin_amdgcn_sched_barrier(0);
            read_frags<T>(lds, fp ^ 1, arow, bcol, kbase, fr[fp ^ 1]);
            mfmas<T, 0, T::HALF>(fr[fp], acc);
            stage<T>(lds, fp, c.t, ra[rp], rb[rp]);
            fetch<T, MODE>(c, (s0 + s + 2 + NR) * BK, ra[rp], rb[rp]);
            il_order<T, MODE>();
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            return;
        }
        if (s + 1 < n) read_frags<T>(lds, fp ^ 1, arow, bcol, kbase, fr[fp ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfmas<T, 0, T::HALF / 2>(fr[fp], acc);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 2 < n) {
            stage<T>(lds, fp, c.t, ra[rp], rb[rp]);
            if (s + 2 + NR < n) fetch_any(s + 2 + NR, rp);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfmas<T, T::HALF / 2, T::HALF>(fr[fp], acc);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    // Fragments of slice 0 into fr[0], once slices 0 and 1 are in LDS.
    auto first_frags = [&]() {
        __syncthreads();
        read_frags<T>(lds, 0, arow, bcol, kbase, fr[0]);
        __syncthreads();   // buffer 0 is rewritten in iteration 0
    };
    // The last slices, with checks, from slice s (a multiple of U) on.
    auto tail = [&](int64_t s) {
        for (; s < n; s += U) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s + u < n) step(s + u, u & 1, (u + 2) % NR, true);
        }
    };

    // Prologue: slices 0 and 1 into LDS (loaded together when there are two
    // register sets), slices 2 .. NR+1 into registers.
    //
    // When the interleaved loop runs at least once, every prologue slice is
    // full and the prologue issues the same loads on every path, with no
    // branch.  The loop is entered from that prologue only: the compiler
    // places each wait for global loads by counting the loads still in
    // flight, and where a loop is entered from paths with different load
    // counts it assumes the fewest -- which made the wait before each LDS
    // store cover all but the last few loads, i.e. the slice fetched one
    // iteration earlier instead of NR iterations earlier (measured: 6.5% of
    // the 64x64 loop at 1024^2 x 4096, 2.4% at 4096^3).
    // The scheduling barriers keep each slice's loads behind the previous
    // slice's, as in the loop, so that waiting for one slice never waits for
    // a later one.
    if (U - 1 + 2 + NR < limit) {
        fetch<T, MODE>(c, s0 * BK, ra[0], rb[0]);
        __builtin_amdgcn_sched_barrier(0);
        if (NR >= 2) fetch<T, MODE>(c, (s0 + 1) * BK, ra[1 % NR], rb[1 % NR]);
        __builtin_amdgcn_sched_barrier(0);
        stage<T>(lds, 0, c.t, ra[0], rb[0]);
        if (NR < 2) fetch<T, MODE>(c, (s0 + 1) * BK, ra[0], rb[0]);
        stage<T>(lds, 1, c.t, ra[1 % NR], rb[1 % NR]);
#pragma unroll
        for (int j = 2; j < NR + 2; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            fetch<T, MODE>(c, (s0 + j) * BK, ra[j % NR], rb[j % NR]);
        }
        __builtin_amdgcn_sched_barrier(0);
        first_frags();
        int64_t s = 0;
        for (; s + U - 1 + 2 + NR < limit; s += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) step(s + u, u & 1, (u + 2) % NR, false);
        }
        tail(s);
        return;
    }
    fetch_any(0, 0);
    if (NR >= 2 && n > 1) fetch_any(1, 1);
    stage<T>(lds, 0, c.t, ra[0], rb[0]);
    if (n > 1) {
        if (NR < 2) fetch_any(1, 0);
        stage<T>(lds, 1, c.t, ra[1 % NR], rb[1 % NR]);
    }
#pragma unroll
    for (int j = 2; j < NR + 2; ++j)
        if (j < n) fetch_any(j, j % NR);
    first_frags();
    tail(0);
}

// ---- direct staging: global memory to LDS without registers ----
//
// gfx950's 16-byte loads into LDS (global_load_lds_dwordx4, and the buffer
// form used by dma16b) write 16 bytes per lane straight into LDS, lane i
// of a wave at byte 16 i past a wave-uniform base (M0): the data lands in
// no register, needs no ds_write and no wait before one.
// Each instruction moves 1 KB per wave, so a slice is laid out in 1 KB
// blocks:
//   A block: 16 rows of the slice, 4 quads a row (rows 16 words apart);
//            quad q of row m is stored at position q ^ ((m >> 2) & 3), so
//            the 16 rows that 16 consecutive lanes read at one quad
//            (ds_read_b128) start in 16 distinct 4-bank groups;
//   B block: 256 / BN rows of BN words; blocks are 256 + PADB words apart,
//            so the two lane halves, which read rows k and k + BK/2 of the
//            slice, fall in opposite halves of the 64 banks.
// Which global quad a lane loads is chosen to fit that layout: four
// consecutive lanes still read one row's 64 contiguous bytes of A, sixteen
// (BN = 64) or thirty-two (BN = 128) one row's bytes of B.
//
// S stages, each a __shared__ array of its own (so the compiler can tell
// them apart and does not make a fragment read wait for the loads still in
// flight into other stages); slice s lives in stage s % S.  Iteration s
// reads the fragments of slice s+1, runs the MFMAs of slice s and issues
// the loads of slice s+S into the stage of slice s (free: its fragments
// were read in iteration s-1, before the barrier that ended it).  It ends
// by waiting for this wave's loads of slice s+2 and a workgroup barrier,
// after which every wave's share of slice s+2 is in LDS and every wave has
// read the fragments of slice s+1.  S = 6, so 4 slices stay in flight
// across a barrier (with 4 stages 16384 x 64 x 16384, which streams A from
// HBM, lost 23% against the register path, and 1024^3, 2048 x 1024 x 512
// and 3000^2 x 1000 ran 0.8 to 1.4% slower than with 6; 8 stages gained
// 1.5% on 16384 x 64 x 16384 but lost 1% at 1024^3, 1.8% at
// 2048 x 1024 x 512 and 4.4% at 5264 x 2016 x 240).  Six stages of 8448
// bytes let three workgroups share a CU.  With no register sets the kernel
// is the same for the Many and Deep tiles, so both launch one
// instantiation (DmaTile).  Timed against the register path (medians of
// 7 interleaved rounds, one box): 1024^3 +4.5%, 1024^2 x 512 +4.4%,
// 2048 x 1024 x 512 +4.9%, 3000^2 x 1000 +3.9%, 3072^2 x 2048 +2.2%,
// 16384 x 64 x 2048 +1.5%; 16384 x 64 x 16384, which HBM and power hold,
// within 0.4%.  The 8-wave tiles keep the register path: their loop
// already runs at 98% of the MFMA rate at 4096^3 (direct loads: within
// 0.2%), and the 128 x 128 tile's ring would let two workgroups share a CU
// where its registers allow one (2048^3 and 2560^3 1% slower).
template <class T>
struct Dma {
    static constexpr bool USED = T::BM == 64;               // the 64 x 64 tiles only
    static constexpr int S = 6;                             // stages
    static constexpr int RPB = 256 / T::BN;                 // B rows per block
    static constexpr int PADB = 32 * RPB / T::HALF;         // words between B blocks
    static constexpr int A_WORDS = T::BM * T::BK;
    static constexpr int B_BLOCK = 256 + PADB;
    static constexpr int B_WORDS = T::BK / RPB * B_BLOCK;
    static constexpr int STAGE = A_WORDS + B_WORDS;         // words per stage
    static constexpr int A_INS = T::BM * T::BK / 4 / T::THREADS;   // per wave and slice
    static constexpr int B_INS = T::BK * T::BN / 4 / T::THREADS;
    static constexpr int NV = A_INS + B_INS;
    static_assert(!USED || (T::BK == 16 && 256 % T::BN == 0 && T::HALF % RPB == 0),
                  "block layout");
    static_assert(!USED || (A_INS >= 1 && B_INS >= 1 && A_INS * T::THREADS * 4 == T::BM * T::BK &&
                            B_INS * T::THREADS * 4 == T::BK * T::BN),
                  "every wave moves whole blocks");
    static_assert(T::WM % 16 == 0, "a lane's rows share (row >> 2) & 3");
    static_assert((S - 2) * NV < 64 && S >= 4 && S <= 8 && S % 2 == 0,
                  "vmcnt range, stage arrays, fragment buffers alternate");
};

// The tile a direct-load launch of tile T runs: T with two register sets,
// which direct staging does not use.
template <class T>
using DmaTile = MfmaTile<T::BM, T::BN, T::BK, T::WM, T::WN, 2>;

// s_waitcnt vmcnt(VM) lgkmcnt(0), expcnt not waited for (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// The end of a direct-load iteration: this wave's loads older than the
// last VM are in LDS and its LDS reads are done; then the workgroup
// barrier.  (__syncthreads would wait for every direct load in flight.)
// The empty asm keeps the compiler from moving memory accesses across it.
template <int VM>
__device__ __forceinline__ void dma_sync() {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<VM>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One direct load: 16 bytes per lane from src to LDS at dst + 16 lane
// (dst is the wave's base, the same for every lane).
__device__ __forceinline__ void dma16(const float *src, float *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// The same through a buffer resource (buf_rsrc): 16 bytes per lane from
// base + voff bytes (base wave-uniform, voff < 2^31 per lane).  The per-lane
// part of the address then stays one 32-bit register for the
// whole K loop and each slice moves only the uniform base, in scalar
// registers: the 64-bit vector adds that global loads need per slice
// competed with the MFMAs (1024^3 6.1%, 512 x 4096 x 4096 6.1% and
// 1024^2 x 2048 6.7% slower with them).
__device__ __forceinline__ void dma16b(const float *base, uint32_t voff, float *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_rsrc(base), dst, 16, voff, 0, 0, 0);
}

template <class T>
struct DmaLane {
    const float *pa[Dma<T>::A_INS];   // this lane's A quad of slice 0, per instruction
    const float *pb[Dma<T>::B_INS];   // this lane's B quad of slice 0
    uint32_t oa[Dma<T>::A_INS];       // the same as byte offsets from the tile's corner
    uint32_t ob[Dma<T>::B_INS];
    const float *abase, *bbase;       // the tile's corner: A at row m0, B at column n0
    int wa, wb;                       // the wave's first A and B block in a stage (words)
    int ra, rb;                       // this lane's fragment offsets in a stage (words)
};

template <class T>
__device__ __forceinline__ DmaLane<T> dma_lane(const Ctx<T> &c, int arow, int bcol, int kbase) {
    using D = Dma<T>;
    DmaLane<T> d;
    const int lane = c.t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(c.t >> 6);
#pragma unroll
    for (int i = 0; i < D::A_INS; ++i) {
        const int g = (i * T::WAVES + wave) * 64 + lane;   // float4 of the slice's A
        const int m = g >> 2, q = (g & 3) ^ ((m >> 2) & 3);
        d.pa[i] = c.A + (c.m0 + m) * c.lda + 4 * q;
        d.oa[i] = static_cast<uint32_t>((m * c.lda + 4 * q) * 4);
    }
#pragma unroll
    for (int i = 0; i < D::B_INS; ++i) {
        const int g = (i * T::WAVES + wave) * 64 + lane;   // float4 of the slice's B
        const int k = g / (T::BN / 4), nq = g % (T::BN / 4);
        d.pb[i] = c.B + k * c.ldb + c.n0 + 4 * nq;
        d.ob[i] = static_cast<uint32_t>((k * c.ldb + 4 * nq) * 4);
    }
    d.abase = c.A + c.m0 * c.lda;
    d.bbase = c.B + c.n0;
    d.wa = wave * 256;
    d.wb = D::A_WORDS + wave * D::B_BLOCK;
    d.ra = arow * 16;
    d.rb = D::A_WORDS + (kbase / D::RPB) * D::B_BLOCK + (kbase % D::RPB) * T::BN + bcol;
    return d;
}

// Issues the direct loads of the slice starting at k0 into a stage.
template <class T>
__device__ __forceinline__ void dma_issue(const DmaLane<T> &d, float *stage, int64_t k0,
                                          int64_t ldb) {
    using D = Dma<T>;
#pragma unroll
    for (int i = 0; i < D::A_INS; ++i)
        dma16b(d.abase + k0, d.oa[i], stage + d.wa + i * T::WAVES * 256);
#pragma unroll
    for (int i = 0; i < D::B_INS; ++i)
        dma16b(d.bbase + k0 * ldb, d.ob[i], stage + d.wb + i * T::WAVES * D::B_BLOCK);
}

// The same loads for the slice that runs past K (K a multiple of 4, so a
// quad of A along k lies wholly inside or outside): a quad of A past K, or
// a row of B past K, loads the 16-byte zero word instead.
template <class T>
__device__ __forceinline__ void dma_issue_tail(const DmaLane<T> &d, float *stage, int64_t k0,
                                               int64_t K, int64_t ldb, int t) {
    using D = Dma<T>;
    const int lane = t & 63, wave = t >> 6;
#pragma unroll
    for (int i = 0; i < D::A_INS; ++i) {
        const int g = (i * T::WAVES + wave) * 64 + lane;
        const int m = g >> 2, q = (g & 3) ^ ((m >> 2) & 3);
        dma16(k0 + 4 * q < K ? d.pa[i] + k0 : &g_zero4[0], stage + d.wa + i * T::WAVES * 256);
    }
#pragma unroll
    for (int i = 0; i < D::B_INS; ++i) {
        const int g = (i * T::WAVES + wave) * 64 + lane;
        const int k = g / (T::BN / 4);
        dma16(k0 + k < K ? d.pb[i] + k0 * ldb : &g_zero4[0],
              stage + d.wb + i * T::WAVES * D::B_BLOCK);
    }
}

// A lane's fragments of the slice in a stage: A rows arow + 32 i, k quads
// kbase / 4 + qq (stored at quad position ^ ((row >> 2) & 3), which is the
// same for all of the lane's rows); B rows kbase + q, columns bcol + 32 j.
template <class T>
__device__ __forceinline__ void dma_frags(const DmaLane<T> &d, const float *stage, int kbase,
                                          Frag<T> &fr) {
    using D = Dma<T>;
    const int x = (static_cast<int>(threadIdx.x) >> 2) & 3;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
#pragma unroll
        for (int qq = 0; qq < T::HALF / 4; ++qq) {
            const int pos = ((kbase >> 2) + qq) ^ x;
            const float4 v =
                *reinterpret_cast<const float4 *>(stage + d.ra + 32 * 16 * i + 4 * pos);
            fr.a[i][4 * qq + 0] = v.x;
            fr.a[i][4 * qq + 1] = v.y;
            fr.a[i][4 * qq + 2] = v.z;
            fr.a[i][4 * qq + 3] = v.w;
        }
    }
#pragma unroll
    for (int q = 0; q < T::HALF; ++q)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
            fr.b[q][j] = stage[d.rb + (q / D::RPB) * D::B_BLOCK + (q % D::RPB) * T::BN + 32 * j];
}

// Issue order of a direct-load iteration: each MFMA followed by a share of
// the fragment reads (first half of the MFMAs) or of the direct loads
// (second half), as il_order does for the register path.
template <int I, int NM, int RPM, int VPM>
__device__ __forceinline__ void dma_schedule() {
    if constexpr (I < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
        if constexpr (I < NM / 2)
            __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);    // LDS reads
        else
            __builtin_amdgcn_sched_group_barrier(0x010, VPM, 0);    // direct loads
        dma_schedule<I + 1, NM, RPM, VPM>();
    }
}

template <class T>
__device__ __forceinline__ void dma_order() {
    constexpr int NM = T::HALF * T::FM * T::FN;
    constexpr int FIRST = NM / 2, SECOND = NM - NM / 2;
    constexpr int NDR = T::FM * (T::HALF / 4) + (T::HALF * T::FN + 1) / 2;
    dma_schedule<0, NM, (NDR + FIRST - 1) / FIRST, (Dma<T>::NV + SECOND - 1) / SECOND>();
}

// The last R slices of a tile, s .. s + R - 1 (s a multiple of S, so slice
// s + j is in stage j % S; S <= R <= 2 S), each iteration J a copy of its
// own: slices s + S .. s + R - 1 are still to load (the one past K, if
// any, with its check), and each wait is for exactly the slice that the
// next iteration reads, so the last load has landed two iterations before
// the end and the kernel ends with no load in flight.  A loop over these
// iterations with run-time conditions made the compiler wait for every
// load in flight before each fragment read (it could no longer tell the
// stages apart): 1024^3 1.7%, 1024^2 x 1000 6% and 16384 x 64 x 2048 5%
// slower.
template <class T, bool TAIL, int R, int J = 0>
__device__ __forceinline__ void dma_last(const Ctx<T> &c, const DmaLane<T> &d,
                                         float *const *stg, int kbase, Frag<T> (&fr)[2],
                                         f32x16 (&acc)[T::FM][T::FN], int64_t s) {
    if constexpr (J < R) {
        using D = Dma<T>;
        constexpr int S = D::S;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (J + 1 < R) dma_frags<T>(d, stg[(J + 1) % S], kbase, fr[(J + 1) & 1]);
        mfmas<T, 0, T::HALF>(fr[J & 1], acc);
        if constexpr (J + S < R) {
            if constexpr (TAIL && J + S == R - 1)
                dma_issue_tail<T>(d, stg[J % S], (s + J + S) * T::BK, c.K, c.ldb, c.t);
            else
                dma_issue<T>(d, stg[J % S], (s + J + S) * T::BK, c.ldb);
            dma_order<T>();
        }
        if constexpr (J + 3 <= R) {
            // slice s + J + 2 is in; the slices after it up to the last
            // one issued may still be on their way
            constexpr int LAST = J + S < R - 1 ? J + S : R - 1;
            dma_sync<(LAST - J - 2) * D::NV>();
        }
        dma_last<T, TAIL, R, J + 1>(c, d, stg, kbase, fr, acc, s);
    }
}

// dma_last for the run-time count r, S <= r <= 2 S (wave-uniform).
template <class T, bool TAIL, int R>
__device__ __forceinline__ void dma_last_r(int r, const Ctx<T> &c, const DmaLane<T> &d,
                                           float *const *stg, int kbase, Frag<T> (&fr)[2],
                                           f32x16 (&acc)[T::FM][T::FN], int64_t s) {
    if constexpr (R <= 2 * Dma<T>::S) {
        if (r == R)
            dma_last<T, TAIL, R>(c, d, stg, kbase, fr, acc, s);
        else
            dma_last_r<T, TAIL, R + 1>(r, c, d, stg, kbase, fr, acc, s);
    }
}

// The K loop over the n slices of a tile when every load is an aligned
// float4 inside the matrices (A and B rows 16-byte aligned, the tile
// inside) and every slice is full -- or, with TAIL, every slice but the
// last, which runs past K (K a multiple of 4); n >= 2 S + 1.  stg: the S
// stage arrays.
template <class T, bool TAIL>
__device__ __forceinline__ void k_loop_dma(const Ctx<T> &c, float *const *stg, int arow,
                                           int bcol, int kbase, f32x16 (&acc)[T::FM][T::FN],
                                           int64_t n) {
    using D = Dma<T>;
    constexpr int S = D::S, BK = T::BK;
    const DmaLane<T> d = dma_lane<T>(c, arow, bcol, kbase);
    Frag<T> fr[2];
    // prologue: slices 0 .. S-1 in flight
#pragma unroll
    for (int j = 0; j < S; ++j) dma_issue<T>(d, stg[j], j * BK, c.ldb);
    // wait for slices 0 and 1, read the fragments of 0, and let every wave
    // finish that read before iteration 0 reloads stage 0
    dma_sync<(S - 2) * D::NV>();
    dma_frags<T>(d, stg[0], kbase, fr[0]);
    dma_sync<(S - 2) * D::NV>();
    int64_t s = 0;
    // with TAIL the slice past K is left to dma_last, which checks it
    int64_t loads = n;
    if constexpr (TAIL) loads = n - 1;
    for (; s + S - 1 + S < loads; s += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            dma_frags<T>(d, stg[(u + 1) % S], kbase, fr[(u + 1) & 1]);
            mfmas<T, 0, T::HALF>(fr[u & 1], acc);
            dma_issue<T>(d, stg[u], (s + u + S) * BK, c.ldb);
            dma_order<T>();
            dma_sync<(S - 2) * D::NV>();
        }
    }
    // the last R = n - s slices, S <= R <= 2 S (n >= 2 S + 1; with TAIL
    // R >= S + 1, so the slice past K is loaded there)
    dma_last_r<T, TAIL, S>(static_cast<int>(n - s), c, d, stg, kbase, fr, acc, s);
}

// How the work of one launch is cut up.  Logical tiles [0, sk_tiles) --
// the last partial wave of tiles -- are shared out by K slice
// ("stream-K"): their tiles x ipt slices are split into sk_wgs contiguous
// runs, q + 1 slices for the first rm workgroups and q for the rest, so
// every such workgroup does the same amount of work.  A workgroup that
// covers a whole tile stores it to C; one that covers part of a tile
// stores its partial sum to the workspace (slot 2w for the first tile of
// its run, 2w + 1 for the last), and the fixup adds the partial sums of
// each such tile in K order.  The remaining tiles [sk_tiles, tiles) are
// done one per workgroup ("data-parallel").  sk_tiles = 0 is the plain
// one-tile-per-workgroup launch.
// Counts that fit 32 bits: tiles (the grid is below 2^31) and stream-K
// slices (the split is only planned when sk_tiles * ipt < 2^30, which keeps
// every intermediate of sk_begin / sk_owner below 2^31).
struct SkPlan {
    int64_t ipt;        // K slices per tile, ceil(K / BK)
    float *ws;          // 2 * sk_wgs partial tiles, BM x BN row-major each
    int tiles_m, tiles_n;
    int sk_tiles;       // logical tiles done by stream-K workgroups
    int sk_wgs;         // stream-K workgroups (the first sk_wgs ids)
    int q, rm;          // slices per stream-K workgroup: q + 1 for w < rm, else q
};

// First slice (in the stream-K slice order) of stream-K workgroup w.
__host__ __device__ __forceinline__ int sk_begin(const SkPlan &p, int w) {
    return w * p.q + (w < p.rm ? w : p.rm);
}

// Stream-K workgroup that runs slice `it`.
__host__ __device__ __forceinline__ int sk_owner(const SkPlan &p, int it) {
    const int big = p.rm * (p.q + 1);
    return it < big ? it / (p.q + 1) : p.rm + (it - big) / p.q;
}

// Workspace slot of the partial sum of tile `tile` by stream-K workgroup w.
__host__ __device__ __forceinline__ int sk_slot(const SkPlan &p, int w, int tile) {
    return 2 * w + (tile == sk_begin(p, w) / static_cast<int>(p.ipt) ? 0 : 1);
}

// The other form of the split, used when the split tiles fit in half a
// wave: logical tiles [0, sk_tiles) are each cut into `parts` runs of
// whole K slices, one workgroup each, that run in the same launch as the
// data-parallel tiles [sk_tiles, tiles) -- so they fill the CUs that the
// last wave of whole tiles leaves idle, where stream-K's runs need a
// launch of their own first.  A part stores its partial sum to workspace
// slot tile * parts + part; a second, small launch adds each tile's parts
// in K order.
struct PartPlan {
    int64_t ipt;        // K slices per tile, ceil(K / BK)
    float *ws;          // sk_tiles * parts partial tiles, BM x BN row-major each
    int tiles_m, tiles_n;
    int sk_tiles;       // logical tiles split in parts
    int parts;          // K parts per split tile, 2 .. 8
};

// First slice of part j of a split tile (parts differ by at most a slice).
__host__ __device__ __forceinline__ int64_t part_begin(const PartPlan &p, int j) {
    return static_cast<int64_t>(j) * p.ipt / p.parts;
}

// One pass of the block tile at (c.m0, c.n0) over slices s0 .. s0+n-1
// (n = 0: a zero tile).  Stores rows [row_lo, rows) and columns
// [col_lo, cols) of the tile to `out` (its corner, leading dimension ldo).
// DMA (dma_mode): 1 when the host found every slice full with aligned
// float4 rows inside the matrices, 2 when the same holds but the last slice
// runs past K (K a multiple of 4); stg then holds the direct-load stages.
template <class T, bool ALIGNED = false, int DMA = 0>
__device__ __forceinline__ void tile_pass(const Ctx<T> &c, int vec_a, int vec_b, float *lds,
                                          int64_t s0, int64_t n, float *out, int64_t ldo,
                                          int row_lo, int64_t rows, int col_lo, int64_t cols,
                                          float *const *stg = nullptr) {
    constexpr int BM = T::BM, BN = T::BN, WM = T::WM, WN = T::WN;
    constexpr int FM = T::FM, FN = T::FN;

    const int t = c.t;
    const int lane = t & 63, wave = t >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int wm0 = (wave / T::WAVES_N) * WM;
    const int wn0 = (wave % T::WAVES_N) * WN;
    const int kbase = h * T::HALF;              // this lane's first k in a slice

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if constexpr (DMA == 1) {
        k_loop_dma<T, false>(c, stg, wm0 + l32, wn0 + l32, kbase, acc, n);
    } else if constexpr (DMA == 2) {
        k_loop_dma<T, true>(c, stg, wm0 + l32, wn0 + l32, kbase, acc, n);
    } else if (ALIGNED && n > 0) {
        // the host found every tile inside the matrices with float4 rows
        k_loop<T, kVec>(c, lds, wm0 + l32, wn0 + l32, kbase, acc, s0, n);
    } else if (n > 0) {
        const bool inside = (c.m0 + BM <= c.M) && (c.n0 + BN <= c.N);
        // a tile larger than the matrix (M < BM or N < BN) loads whole
        // float4s when its rows are aligned and N is a multiple of 4 (then
        // so is n0, and a quad is wholly inside or outside)
        const bool quads = vec_a && vec_b && (c.N & 3) == 0 && (c.n0 & 3) == 0;
        // kVec, kVecA and kScalar load through buffer resources at byte
        // offsets from the tile's corner, below 2^31 only while rows of A
        // are fewer than 2^31 / (4 BM) floats apart and rows of B fewer
        // than 2^31 / (4 BK); farther apart, the element loads of kEdgeElem
        const bool bufok = BM * c.lda * 4 <= INT32_MAX && T::BK * c.ldb * 4 <= INT32_MAX;
        if (!inside && quads)
            k_loop<T, kEdge>(c, lds, wm0 + l32, wn0 + l32, kbase, acc, s0, n);
        else if (!inside || !bufok)
            k_loop<T, kEdgeElem>(c, lds, wm0 + l32, wn0 + l32, kbase, acc, s0, n);
        else if (vec_a && vec_b && (c.n0 & 3) == 0)
            k_loop<T, kVec>(c, lds, wm0 + l32, wn0 + l32, kbase, acc, s0, n);
        else if (vec_a)
            k_loop<T, kVecA>(c, lds, wm0 + l32, wn0 + l32, kbase, acc, s0, n);
        else
            k_loop<T, kScalar>(c, lds, wm0 + l32, wn0 + l32, kbase, acc, s0, n);
    }

    // Epilogue: word r of accumulator (i, j) is row 8*(r/4) + 4*h + r%4,
    // column l32 of that 32x32 block.  Each store covers two 128-byte row
    // segments per wave.
    const bool whole = row_lo == 0 && col_lo == 0 && rows >= BM && cols >= BN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int cn = wn0 + 32 * j + l32;
            if (whole) {
                float *cp = out + (wm0 + 32 * i + 4 * h) * ldo + cn;
#pragma unroll
                for (int r = 0; r < 16; ++r) cp[(8 * (r / 4) + (r % 4)) * ldo] = acc[i][j][r];
                __builtin_amdgcn_sched_barrier(0);   // one block's addresses live at a time
                continue;
            }
            if (cn < col_lo || cn >= cols) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int cm = wm0 + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (cm >= row_lo && cm < rows) out[cm * ldo + cn] = acc[i][j][r];
            }
        }
    }
}

// Float4 chunks of one fixup workgroup: a stream-K tile is finished by
// BM*BN/4 / THREADS workgroups, one float4 per lane.
template <class T>
constexpr int fix_chunks() {
    return T::BM * T::BN / 4 / T::THREADS;
}

// Stores the float4 `s` of a fixup chunk, C[gm][gn .. gn+3], leaving the
// columns the tile shares with its left neighbour (col < skip_n) and those
// past N.
__device__ __forceinline__ void store_chunk(float4 s, float *C, int64_t ldc, int64_t N,
                                            int64_t gm, int64_t gn, int col, int skip_n,
                                            int vec_c) {
    float *cp = C + gm * ldc + gn;
    if (vec_c && col >= skip_n && (gn & 3) == 0 && gn + 3 < N) {
        *reinterpret_cast<float4 *>(cp) = s;
    } else {
        const float e[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (col + q >= skip_n && gn + q < N) cp[q] = e[q];
    }
}

// Adds the partial sums of one chunk of a stream-K tile in K order (so the
// result does not depend on which workgroup finished first) and stores it
// to C.  Tiles that a single stream-K workgroup covered were stored by it.
template <class T>
__device__ __forceinline__ void sk_fixup(int job, int64_t M, int64_t N, float *C, int64_t ldc,
                                         const SkPlan &p, int vec_c) {
    constexpr int BM = T::BM, BN = T::BN;
    static_assert(BM * BN / 4 % T::THREADS == 0, "whole fixup chunks");
    const int tile = job / fix_chunks<T>();
    const int f = (job % fix_chunks<T>()) * T::THREADS + static_cast<int>(threadIdx.x);
    const int ipt = static_cast<int>(p.ipt);
    const int w_lo = sk_owner(p, tile * ipt);
    const int w_hi = sk_owner(p, (tile + 1) * ipt - 1);
    if (w_lo == w_hi) return;
    int64_t tm, tn;
    grouped_tile(tile, p.tiles_m, p.tiles_n, T::GROUP, tm, tn);
    const Origin o = tile_origin<BM, BN>(tm, tn, M, N);
    const int row = f / (BN / 4), col = 4 * (f % (BN / 4));
    const int64_t gm = o.m0 + row, gn = o.n0 + col;
    if (row < o.skip_m || gm >= M) return;
    auto part = [&](int w) {
        return reinterpret_cast<const float4 *>(
            p.ws + static_cast<int64_t>(sk_slot(p, w, tile)) * (BM * BN))[f];
    };
    float4 s = part(w_lo);
    // the loads of several partial sums are in flight at once; the adds
    // stay in K order
#pragma unroll 8
    for (int w = w_lo + 1; w <= w_hi; ++w) {
        const float4 v = part(w);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    float *cp = C + gm * ldc + gn;
    if (vec_c && col >= o.skip_n && (gn & 3) == 0 && gn + 3 < N) {
        *reinterpret_cast<float4 *>(cp) = s;
    } else {
        const float e[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (col + q >= o.skip_n && gn + q < N) cp[q] = e[q];
    }
}

// The same for a tile split in parts: its parts' partial sums in K order.
template <class T>
__device__ __forceinline__ void part_fixup(int job, int64_t M, int64_t N, float *C, int64_t ldc,
                                           const PartPlan &p, int vec_c) {
    constexpr int BM = T::BM, BN = T::BN;
    const int tile = job / fix_chunks<T>();
    const int f = (job % fix_chunks<T>()) * T::THREADS + static_cast<int>(threadIdx.x);
    int64_t tm, tn;
    grouped_tile(tile, p.tiles_m, p.tiles_n, T::GROUP, tm, tn);
    const Origin o = tile_origin<BM, BN>(tm, tn, M, N);
    const int row = f / (BN / 4), col = 4 * (f % (BN / 4));
    const int64_t gm = o.m0 + row, gn = o.n0 + col;
    if (row < o.skip_m || gm >= M) return;
    const float4 *part = reinterpret_cast<const float4 *>(
                             p.ws + static_cast<int64_t>(tile) * p.parts * (BM * BN)) + f;
    float4 s = part[0];
#pragma unroll 8
    for (int j = 1; j < p.parts; ++j) {
        const float4 v = part[static_cast<int64_t>(j) * (BM * BN / 4)];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    store_chunk(s, C, ldc, N, gm, gn, col, o.skip_n, vec_c);
}

// The main launch: workgroups [0, sk_tiles * fix_chunks) finish the
// stream-K tiles (the stream-K launch has completed before this one
// starts), the rest run one data-parallel tile each.  Without a split
// (sk_tiles = 0) every workgroup runs one tile.  ALIGNED: the host found
// that every tile lies inside the matrices and loads whole float4s (see
// aligned_launch), so the kernel holds that load mode's K loop alone --
// a third of the code, whose first fetch into the instruction cache of
// every CU is part of each launch's fixed cost (1024^3: 19.59 -> 19.44 us).
// DMA (dma_mode, 1 or 2): in addition the slices are full, or all but the
// last, and the K loop stages them with direct loads (k_loop_dma) in S
// stage arrays instead of the two register-staged buffers.
template <class T, bool ALIGNED, int DMA = 0>
__global__ __launch_bounds__(T::THREADS)
void gemm_mfma_f32(int64_t M, int64_t N, int64_t K,
                   const float *__restrict__ A, int64_t lda,
                   const float *__restrict__ B, int64_t ldb,
                   float *__restrict__ C, int64_t ldc, SkPlan p, int vec_a, int vec_b,
                   int vec_c)
{
    static_assert(!DMA || (ALIGNED && Dma<T>::USED), "direct loads: aligned 64 x 64 tiles");
    constexpr int WORDS = DMA ? 4 : T::LDS_WORDS;
    constexpr int SN = DMA ? Dma<T>::S : 0;
    constexpr int STAGE = DMA ? Dma<T>::STAGE : 4;
    __shared__ __attribute__((aligned(16))) float lds[WORDS];
    __shared__ __attribute__((aligned(16))) float st0[0 < SN ? STAGE : 4];
    __shared__ __attribute__((aligned(16))) float st1[1 < SN ? STAGE : 4];
    __shared__ __attribute__((aligned(16))) float st2[2 < SN ? STAGE : 4];
    __shared__ __attribute__((aligned(16))) float st3[3 < SN ? STAGE : 4];
    __shared__ __attribute__((aligned(16))) float st4[4 < SN ? STAGE : 4];
    __shared__ __attribute__((aligned(16))) float st5[5 < SN ? STAGE : 4];
    __shared__ __attribute__((aligned(16))) float st6[6 < SN ? STAGE : 4];
    __shared__ __attribute__((aligned(16))) float st7[7 < SN ? STAGE : 4];
    float *const stg[8] = {st0, st1, st2, st3, st4, st5, st6, st7};
    if constexpr (DMA) {
#pragma unroll
        for (int j = 0; j < SN; ++j) lds_poison(stg[j], STAGE);
    } else {
        lds_poison(lds, WORDS);
    }

    const int bid = static_cast<int>(blockIdx.x);
    const int fix = p.sk_tiles * fix_chunks<T>();
    if (bid < fix) {
        sk_fixup<T>(bid, M, N, C, ldc, p, vec_c);
        return;
    }
    const int dp = p.tiles_m * p.tiles_n - p.sk_tiles;
    const int tile = p.sk_tiles + xcd_remap32(bid - fix, dp);
    int tm, tn;
    grouped_tile32<T::GROUP>(tile, p.tiles_m, p.tiles_n, tm, tn);
    const Origin o = tile_origin<T::BM, T::BN>(tm, tn, M, N);
    const Ctx<T> c{M, N, K, A, lda, B, ldb, o.m0, o.n0, static_cast<int>(threadIdx.x)};
    const int64_t rows = M - o.m0 < T::BM ? M - o.m0 : T::BM;
    const int64_t cols = N - o.n0 < T::BN ? N - o.n0 : T::BN;
    tile_pass<T, ALIGNED, DMA>(c, vec_a, vec_b, lds, 0, p.ipt, C + o.m0 * ldc + o.n0, ldc,
                               o.skip_m, rows, o.skip_n, cols, stg);
}

// The stream-K launch: workgroup w runs slices [sk_begin(w), sk_begin(w+1))
// of the stream-K tiles in order, one segment per tile it touches.  A
// segment that covers a whole tile is stored to C; a partial one to the
// workspace slot of (w, tile).
template <class T>
__global__ __launch_bounds__(T::THREADS) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_mfma_f32_sk(int64_t M, int64_t N, int64_t K,
                      const float *__restrict__ A, int64_t lda,
                      const float *__restrict__ B, int64_t ldb,
                      float *__restrict__ C, int64_t ldc, SkPlan p, int vec_a, int vec_b)
{
    __shared__ __attribute__((aligned(16))) float lds[T::LDS_WORDS];
    lds_poison(lds, T::LDS_WORDS);

    const int ipt = static_cast<int>(p.ipt);
    const int w = static_cast<int>(xcd_remap(blockIdx.x, p.sk_wgs));
    const int end = sk_begin(p, w + 1);
    int it = sk_begin(p, w);
    Ctx<T> c{M, N, K, A, lda, B, ldb, 0, 0, 0};
    for (;;) {
        const int tile = it / ipt, kb = it - tile * ipt;
        const int ke = ipt < kb + (end - it) ? ipt : kb + (end - it);
        int64_t tm, tn;
        grouped_tile(tile, p.tiles_m, p.tiles_n, T::GROUP, tm, tn);
        const Origin o = tile_origin<T::BM, T::BN>(tm, tn, M, N);
        c.m0 = o.m0;
        c.n0 = o.n0;
        float *out;
        int64_t ldo, rows, cols;
        int row_lo, col_lo;
        if (kb == 0 && ke == ipt) {            // the whole K range: final values
            out = C + o.m0 * ldc + o.n0;
            ldo = ldc;
            row_lo = o.skip_m;
            col_lo = o.skip_n;
            rows = M - o.m0 < T::BM ? M - o.m0 : T::BM;
            cols = N - o.n0 < T::BN ? N - o.n0 : T::BN;
        } else {                                // part of it: a partial sum
            out = p.ws + static_cast<int64_t>(sk_slot(p, w, tile)) * (T::BM * T::BN);
            ldo = T::BN;
            row_lo = col_lo = 0;
            rows = T::BM;
            cols = T::BN;
        }
        // The lane id and the leading dimensions are laundered per segment:
        // otherwise the compiler hoists the addresses of every load mode out
        // of the segment loop and keeps them live at once (spilling).  The
        // operand pointers are not: through the asm they lost their global
        // address space, the loads became flat loads, and the LDS waits
        // before every barrier then waited for them too -- the whole memory
        // latency once per slice (1152^2 x 8192: 198 -> 193 us without).
        int lane_id = static_cast<int>(threadIdx.x);
        asm volatile("" : "+v"(lane_id));
        c.t = lane_id;
        asm volatile("" : "+s"(c.lda), "+s"(c.ldb));
        tile_pass<T>(c, vec_a, vec_b, lds, kb, ke - kb, out, ldo, row_lo, rows, col_lo, cols);
        it += ke - kb;
        if (it >= end) break;
        __syncthreads();   // LDS is reused by the next segment
    }
}

// The main launch of a split in parts: workgroups [0, sk_tiles * parts)
// run one K part each and store its partial sum to the workspace, the rest
// one data-parallel tile each.  (A kernel of its own: its second tile pass
// in gemm_mfma_f32 would change that kernel's code for every launch.)
template <class T>
__global__ __launch_bounds__(T::THREADS)
void gemm_mfma_f32_parts(int64_t M, int64_t N, int64_t K,
                         const float *__restrict__ A, int64_t lda,
                         const float *__restrict__ B, int64_t ldb,
                         float *__restrict__ C, int64_t ldc, PartPlan p, int vec_a, int vec_b)
{
    __shared__ __attribute__((aligned(16))) float lds[T::LDS_WORDS];
    lds_poison(lds, T::LDS_WORDS);

    const int bid = static_cast<int>(blockIdx.x);
    const int split = p.sk_tiles * p.parts;
    int tile, part = -1;
    if (bid < split) {
        const int w = static_cast<int>(xcd_remap(bid, split));
        tile = w / p.parts;
        part = w - tile * p.parts;
    } else {
        const int dp = p.tiles_m * p.tiles_n - p.sk_tiles;
        tile = p.sk_tiles + static_cast<int>(xcd_remap(bid - split, dp));
    }
    int64_t tm, tn;
    grouped_tile(tile, p.tiles_m, p.tiles_n, T::GROUP, tm, tn);
    const Origin o = tile_origin<T::BM, T::BN>(tm, tn, M, N);
    const Ctx<T> c{M, N, K, A, lda, B, ldb, o.m0, o.n0, static_cast<int>(threadIdx.x)};
    if (part >= 0) {                       // a part: the whole block tile to its slot
        const int64_t s0 = part_begin(p, part);
        tile_pass<T>(c, vec_a, vec_b, lds, s0, part_begin(p, part + 1) - s0,
                     p.ws + static_cast<int64_t>(tile * p.parts + part) * (T::BM * T::BN), T::BN,
                     0, T::BM, 0, T::BN);
        return;
    }
    const int64_t rows = M - o.m0 < T::BM ? M - o.m0 : T::BM;
    const int64_t cols = N - o.n0 < T::BN ? N - o.n0 : T::BN;
    tile_pass<T>(c, vec_a, vec_b, lds, 0, p.ipt, C + o.m0 * ldc + o.n0, ldc, o.skip_m, rows,
                 o.skip_n, cols);
}

// After gemm_mfma_f32_parts: sk_tiles * fix_chunks workgroups add each
// split tile's partial sums.
template <class T>
__global__ __launch_bounds__(T::THREADS)
void gemm_mfma_f32_fixup(int64_t M, int64_t N, float *__restrict__ C, int64_t ldc, PartPlan p,
                         int vec_c)
{
    part_fixup<T>(static_cast<int>(blockIdx.x), M, N, C, ldc, p, vec_c);
}

// Tile shapes (chosen by timing candidates on MI355X, interleaved and
// repeated on one warm GPU):
//   Large  256x128x16, 8 waves of 64x64, four register sets: shapes with
//          at least 4 tiles of 128x128 per CU (4096^3: 512 such tiles), or
//          a whole number of 256x128 tiles per CU.
//   Mid    128x128x16, 8 waves of 64x32: about one 128x128 tile per CU
//          (2048^3: 256 tiles), or one to two per CU with K >= 2048.
//   Many   64x64x16, 4 waves of 32x32, two register sets: every other
//          shape with K <= 1024 (1024^3).
//   Deep   the Many tile with four register sets in flight, for K > 1024
//          (3000x2049x1531, 16384x64x16384).
// With the loop's waits exact (see k_loop), the 16-deep slices of the Many
// and Deep tiles beat 32-deep ones by 1-2.5% on most shapes, and need 124
// VGPRs instead of about 200.
using TileLarge = MfmaTile<256, 128, 16, 64, 64, 4>;
using TileMid = MfmaTile<128, 128, 16, 64, 32, 2>;
using TileMany = MfmaTile<64, 64, 16, 32, 32, 2>;
using TileDeep = MfmaTile<64, 64, 16, 32, 32, 4>;

constexpr int64_t kMi355xCUs = 256;

enum class Shape { kLarge, kMid, kMany, kDeep };

// Fraction of a padded bm x bn tile grid that lies inside M x N.
double cover(int64_t M, int64_t N, int64_t bm, int64_t bn) {
    return static_cast<double>(M) * static_cast<double>(N) /
           (static_cast<double>(ceil_div(M, bm) * bm) * static_cast<double>(ceil_div(N, bn) * bn));
}

Shape pick(int64_t M, int64_t N, int64_t K) {
    const int64_t cus = kMi355xCUs;
    const int64_t tiles128 = ceil_div(M, 128) * ceil_div(N, 128);
    const int64_t large = ceil_div(M, 256) * ceil_div(N, 128);
    // Short K (at most 16 slices) with M >= 2048: 64x64 tiles, several a CU,
    // so that one tile's first loads and stores overlap another's MFMAs;
    // on a single larger tile per CU they do not (4096^2 x 128 47.1 -> 42.8
    // us, 2048x4096x128 25.9 -> 23.1, 4096^2 x 224 66.5 -> 62.6, 6144^2 x
    // 256 179 -> 155, 16384^2 x 256 1166 -> 1119, 2048^2 x 256 21.2 ->
    // 19.7, 16384x4096x256 285 -> 279).  Not with K = 512 (2048^2 x 512
    // 35.6 -> 40.7 us) nor for smaller M (1000x4096x256 21.7 -> 23.9,
    // 500x8192x256 21.8 -> 24.0; 1024x4096x256 gained, 21.1 -> 19.8).
    if (K <= 256 && M >= 2048) return Shape::kMany;
    // The larger tiles only where they waste no more of the edges than
    // 64x64 tiles (at most 3% more of the tile grid outside M x N): with
    // N = 64 half of every 128-wide tile lies outside the matrix, with
    // M = 64 three quarters of every 256-high one.  Against the larger
    // tiles: 32768x64x8192 517 -> 289 us, 64x65536x4096 973 -> 320,
    // 128x65536x2048 497 -> 277, 16384x192x4096 237 -> 191, 384x16384x4096
    // 462 -> 362, 640x32768x2048 704 -> 612, 2049x32768x1024 1075 -> 1000,
    // 2049x8192x4096 1046 -> 1000, 65536x300x2048 711 -> 665.
    const double c64 = cover(M, N, 64, 64);
    const bool fit256 = cover(M, N, 256, 128) >= 0.97 * c64;
    const bool fit128 = cover(M, N, 128, 128) >= 0.97 * c64;
    // With K <= 1024, only when the 256x128 tiles fill the CUs to within 5%
    // of whole waves: the split that evens out a partial last wave does not
    // pay for itself on so few slices, and the 64x64 tiles, many a CU, are
    // even by themselves (against 256x128 tiles split in parts or runs:
    // 4608^2 x 512 195 -> 165 us, 3072x6144x512 162 -> 145, 4608^2 x 1024
    // 337 -> 313, 6144x3072x1024 289 -> 272, 6144^2 x 512 303 -> 285,
    // 6144^2 x 1024 558 -> 541, 7168^2 x 1024 756 -> 732; with K = 2048
    // the split forms were within 1.4%)
    const bool even256 = K > 1024 || 20 * large >= 19 * ceil_div(large, cus) * cus;
    // Large: about 4 tiles of 128x128 per CU, or a whole number of 256x128
    // tiles per CU (4096x2048x1024: 135 -> 126 us against 64x64 tiles)
    if (fit256 && even256 && (tiles128 >= 4 * cus || (large >= cus && large % cus == 0)))
        return Shape::kLarge;
    if (fit128 && 4 * tiles128 > 3 * cus && tiles128 <= cus) return Shape::kMid;
    // Mid also for one to two 128x128 tiles per CU once K is long enough to
    // pay for the stream-K split that evens them out, unless 128x128 tiles
    // waste more of the edges (3000x2049x1531 stays on 64x64 tiles):
    // 2304^3 207 -> 193 us, 1536x4096x4096 386 -> 382 us
    if (fit128 && tiles128 > cus && tiles128 < 2 * cus && K >= 2048) return Shape::kMid;
    // and for exactly three 128x128 tiles per CU, which leave no partial
    // wave (2048x6144x4096 710 -> 695 us, 3072x4096x8192 1419 -> 1379,
    // 6144x2048x3072 537 -> 525, 2048x6144x2048 +0.9%; within 2% either
    // way with K <= 1024)
    if (fit128 && tiles128 == 3 * cus && K >= 2048) return Shape::kMid;
    return K > 1024 ? Shape::kDeep : Shape::kMany;
}

// Compute units of the current device (MI355X's 256 if it cannot be read).
int64_t device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kMi355xCUs;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();
        return kMi355xCUs;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Workgroups of `kernel` per CU that the split is planned for: `planned`
// (what gfx950 holds), or fewer if the device's occupancy query says it
// holds fewer.  (Planning with more than `planned` when a build happens to
// fit one more workgroup would change which tiles are split, and with it
// the timings the split's rules were fitted to.)
template <class T>
int64_t resident_per_cu(const void *kernel, std::atomic<int> &cache, int planned) {
    int n = cache.load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, T::THREADS, 0) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();
        return planned;
    }
    n = std::min(n, planned);
    cache.store(n, std::memory_order_relaxed);
    return n;
}

// The stream-K kernel (held at no fewer than 2 waves per SIMD): planned
// at one 8-wave workgroup per CU and three 4-wave ones.
template <class T>
int64_t resident_sk() {
    static std::atomic<int> cache{0};
    return resident_per_cu<T>(reinterpret_cast<const void *>(gemm_mfma_f32_sk<T>), cache,
                              T::THREADS == 512 ? 1 : 3);
}

// gemm_mfma_f32_parts: gfx950 holds one 8-wave workgroup per CU (over 128
// VGPRs), and three (four register sets, 152 VGPRs) or four (two, 128) of
// the 4-wave ones.
template <class T>
int64_t resident_parts() {
    static std::atomic<int> cache{0};
    return resident_per_cu<T>(reinterpret_cast<const void *>(gemm_mfma_f32_parts<T>), cache,
                              T::THREADS == 512 ? 1 : (T::NR == 4 ? 3 : 4));
}

// The work split of a launch: stream-K runs (sk), or parts (pp.parts > 0),
// or neither (sk.sk_tiles = 0: every tile data-parallel).
struct Split {
    SkPlan sk;
    PartPlan pp;
};

// Without stream-K, or when the tiles fill whole waves of resident
// workgroups, every tile is data-parallel.  Otherwise the tiles of the last
// partial wave (all tiles if there are fewer than one wave) are split along
// K:
//   * in parts, when at least two parts of each fit in one wave of
//     gemm_mfma_f32_parts and the parts spread evenly over the CUs (at
//     most one a CU, or no CU more than 10% above the mean): as many parts
//     as fit, at most 8 and with at least 2 slices each.  (Uneven parts
//     lose to runs: 1152^2 x 8192, 648 half tiles on 256 CUs, 192 against
//     188 us.);
//   * else in stream-K runs over up to one wave of the stream-K kernel,
//     each with at least 2 slices and at least an eighth of a tile's, so a
//     tile has at most about 8 partial sums to add.  Whole-tile parts
//     cannot even out a remainder of more than half a wave: 136 tiles of
//     256 x 128 left on 256 CUs need about half a tile more per CU, which
//     runs that cross tiles give (4608^2 x 4096: 1228 us with runs, 1393
//     unsplit).
template <class T>
Split plan_split(int64_t M, int64_t N, int64_t K, bool stream_k) {
    Split r{};
    SkPlan &p = r.sk;
    const int64_t tiles_m = ceil_div(M, T::BM), tiles_n = ceil_div(N, T::BN);
    const int64_t tiles = tiles_m * tiles_n;
    p.ipt = ceil_div(K, T::BK);
    if (tiles > kMaxGrid) return r;   // rejected before launch
    p.tiles_m = static_cast<int>(tiles_m);
    p.tiles_n = static_cast<int>(tiles_n);
    if (!stream_k || p.ipt < 2) return r;
    const int64_t cus = device_cus();
    const int64_t wave = cus * resident_parts<T>();
    if (tiles % wave != 0) {
        const int64_t sk_tiles = tiles % wave;
        const int64_t parts = std::min<int64_t>({8, p.ipt / 2, wave / sk_tiles});
        const int64_t n = sk_tiles * parts;
        if (parts >= 2 && (n <= cus || 10 * ceil_div(n, cus) * cus <= 11 * n)) {
            p.sk_tiles = static_cast<int>(sk_tiles);
            r.pp = PartPlan{p.ipt, nullptr, p.tiles_m, p.tiles_n, p.sk_tiles,
                            static_cast<int>(parts)};
            return r;
        }
    }
    const int64_t slots = device_cus() * resident_sk<T>();
    if (tiles % slots == 0) return r;
    const int64_t sk_tiles = tiles % slots;
    const int64_t total = sk_tiles * p.ipt;
    if (total > (kMaxGrid >> 1)) return r;   // slice arithmetic must fit 32 bits
    const int64_t min_slices = std::max<int64_t>(2, ceil_div(p.ipt, 8));
    const int64_t sk_wgs = std::max<int64_t>(1, std::min(slots, total / min_slices));
    p.sk_tiles = static_cast<int>(sk_tiles);
    p.sk_wgs = static_cast<int>(sk_wgs);
    p.q = static_cast<int>(total / sk_wgs);
    p.rm = static_cast<int>(total % sk_wgs);
    return r;
}

// Workgroups that run the split: the parts, or the stream-K runs.
inline int64_t split_wgs(const Split &r) {
    return r.pp.parts > 0 ? static_cast<int64_t>(r.pp.sk_tiles) * r.pp.parts : r.sk.sk_wgs;
}

// Partial tiles: one per part, or two per stream-K workgroup.
template <class T>
size_t workspace_bytes(const Split &r) {
    const size_t slots = static_cast<size_t>(split_wgs(r)) * (r.pp.parts > 0 ? 1 : 2);
    return slots * T::BM * T::BN * sizeof(float);
}

// Workgroups of the main launch: every tile, plus the extra parts of the
// split tiles, or the fixup chunks after the first of each stream-K tile.
template <class T>
int64_t main_grid(const Split &r) {
    const int64_t extra = r.pp.parts > 0 ? r.pp.parts : fix_chunks<T>();
    return static_cast<int64_t>(r.sk.tiles_m) * r.sk.tiles_n +
           static_cast<int64_t>(r.sk.sk_tiles) * (extra - 1);
}

// How the main launch stages its slices: 0 through registers; with direct
// loads when every tile lies inside the matrices with float4 rows
// (aligned_launch) and there are the 2 S + 1 slices the direct-load K loop
// needs -- 1 when every slice is full, 2 when the last one runs past K and
// K is a multiple of 4 (so a quad of A along k is wholly inside or outside
// the matrix).  Short K gains most: 1024^2 x 208 (13 slices) +8%,
// 5264 x 2016 x 240 +5%, 4848 x 1608 x 496 +5%, 2048 x 1024 x 256 +4.5%.
inline int dma_mode(bool aligned, int64_t K, int64_t bk, int64_t stages, int64_t bm,
                    int64_t lda, int64_t ldb) {
    const int64_t n = ceil_div(K, bk);
    if (!aligned || n < 2 * stages + 1) return 0;
    // a lane's byte offset from the tile's corner fits the buffer loads'
    // 31 bits (rows of A up to 8 M floats apart, of B up to 32 M)
    if (bm * lda * 4 > INT32_MAX || bk * ldb * 4 > INT32_MAX) return 0;
    if (K % bk == 0) return 1;
    return K % 4 == 0 ? 2 : 0;
}

// `name`, or `dma_name` when the main launch stages with direct loads
// (planned for 16-byte-aligned operands with lda = K, ldb = N, and only for
// launches without a split, see launch_tile).
template <class T>
LaunchPlan plan_for(int64_t M, int64_t N, int64_t K, bool stream_k, const char *name,
                    const char *dma_name) {
    const Split r = plan_split<T>(M, N, K, stream_k);
    const bool aligned = (K & 3) == 0 && M >= T::BM && N >= T::BN && (N & 3) == 0;
    const bool dma = Dma<T>::USED && r.sk.sk_tiles == 0 &&
                     dma_mode(aligned, K, T::BK, Dma<T>::S, T::BM, K, N);
    LaunchPlan p{};
    p.kernel = dma ? dma_name : name;
    p.bm = T::BM;
    p.bn = T::BN;
    p.bk = T::BK;
    p.grid = main_grid<T>(r);
    p.block = T::THREADS;
    p.lds_bytes = static_cast<int>((dma ? Dma<T>::S * Dma<T>::STAGE : T::LDS_WORDS) *
                                   sizeof(float));
    p.sk_tiles = r.sk.sk_tiles;
    p.sk_wgs = split_wgs(r);
    p.split = r.pp.parts > 0 ? "parts" : (r.sk.sk_wgs > 0 ? "runs" : "none");
    p.workspace_bytes = workspace_bytes<T>(r);
    return p;
}

// True when every tile of the launch lies inside the matrices (M >= BM and
// N >= BN, so tile_origin moves the edge tiles inside) and loads float4s:
// A and B rows 16-byte aligned, and every tile's first column a multiple
// of 4 (the columns of the moved last tile start at N - BN).
template <class T>
bool aligned_launch(const GemmArgs &a, int vec_a, int vec_b) {
    return vec_a && vec_b && a.M >= T::BM && a.N >= T::BN && (a.N & 3) == 0;
}

// Launches on the caller's stream: the stream-K runs and then the main
// launch (which first adds their partial sums), or the parts with the
// data-parallel tiles and then their fixup, or the main launch alone.
template <class T>
hipError_t launch_tile(const GemmArgs &a, bool stream_k, void *ws, size_t ws_bytes) {
    Split r = plan_split<T>(a.M, a.N, a.K, stream_k);
    if (workspace_bytes<T>(r) > ws_bytes || (split_wgs(r) > 0 && ws == nullptr))
        return hipErrorInvalidValue;
    // float4 loads (buffer loads, see fetch) need a lane's byte offset from
    // the tile's corner below 2^31: rows of A up to 2^31 / (4 BM) floats
    // apart, rows of B up to 2^31 / (4 BK); farther apart, element loads
    const int vec_a = vec4_ok(a.A, a.lda) && T::BM * a.lda * 4 <= INT32_MAX;
    const int vec_b = vec4_ok(a.B, a.ldb) && T::BK * a.ldb * 4 <= INT32_MAX;
    const int vec_c = vec4_ok(a.C, a.ldc);
    const dim3 grid(static_cast<uint32_t>(main_grid<T>(r)));
    hipError_t err;
    if (r.pp.parts > 0) {
        PartPlan &p = r.pp;
        p.ws = static_cast<float *>(ws);
        hipLaunchKernelGGL(gemm_mfma_f32_parts<T>, grid, dim3(T::THREADS), 0, a.stream, a.M, a.N,
                           a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, p, vec_a, vec_b);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(gemm_mfma_f32_fixup<T>,
                           dim3(static_cast<uint32_t>(p.sk_tiles * fix_chunks<T>())),
                           dim3(T::THREADS), 0, a.stream, a.M, a.N, a.C, a.ldc, p, vec_c);
        return hipGetLastError();
    }
    SkPlan &p = r.sk;
    p.ws = static_cast<float *>(ws);
    if (p.sk_wgs > 0) {
        hipLaunchKernelGGL(gemm_mfma_f32_sk<T>, dim3(static_cast<uint32_t>(p.sk_wgs)),
                           dim3(T::THREADS), 0, a.stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb,
                           a.C, a.ldc, p, vec_a, vec_b);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    // fixups of the stream-K tiles, then the data-parallel tiles.  Direct
    // loads only without a split: the splits' plans were fitted to the
    // register-staged kernel, and a stage ring that changes how many
    // workgroups a CU holds breaks them (2560^3, 128 x 128 tiles with
    // stream-K runs, went from 256 to 402 us when direct loads let two
    // workgroups share a CU; the 64 x 64 ring holds three a CU, where the
    // register-staged kernels hold four and three)
    const bool aligned = aligned_launch<T>(a, vec_a, vec_b);
    if constexpr (Dma<T>::USED) {
        const int mode =
            p.sk_tiles == 0 ? dma_mode(aligned, a.K, T::BK, Dma<T>::S, T::BM, a.lda, a.ldb) : 0;
        if (mode == 1)
            hipLaunchKernelGGL((gemm_mfma_f32<DmaTile<T>, true, 1>), grid, dim3(T::THREADS), 0,
                               a.stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, p,
                               vec_a, vec_b, vec_c);
        else if (mode == 2)
            hipLaunchKernelGGL((gemm_mfma_f32<DmaTile<T>, true, 2>), grid, dim3(T::THREADS), 0,
                               a.stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, p,
                               vec_a, vec_b, vec_c);
        if (mode != 0) return hipGetLastError();
    }
    if (aligned)
        hipLaunchKernelGGL((gemm_mfma_f32<T, true>), grid, dim3(T::THREADS), 0, a.stream, a.M,
                           a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, p, vec_a, vec_b, vec_c);
    else
        hipLaunchKernelGGL((gemm_mfma_f32<T, false>), grid, dim3(T::THREADS), 0, a.stream, a.M,
                           a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, p, vec_a, vec_b, vec_c);
    return hipGetLastError();
}

}  // namespace

LaunchPlan plan_mfma(int64_t M, int64_t N, int64_t K, bool stream_k) {
    switch (pick(M, N, K)) {
        case Shape::kLarge:
            return plan_for<TileLarge>(M, N, K, stream_k,
                                       "gemm_mfma_f32<256x128x16, 8 waves, 4 sets>", nullptr);
        case Shape::kMid:
            return plan_for<TileMid>(M, N, K, stream_k, "gemm_mfma_f32<128x128x16, 8 waves>",
                                     nullptr);
        case Shape::kMany:
            return plan_for<TileMany>(M, N, K, stream_k, "gemm_mfma_f32<64x64x16, 4 waves>",
                                      "gemm_mfma_f32<64x64x16, 4 waves, 6 LDS stages>");
        default:
            return plan_for<TileDeep>(M, N, K, stream_k,
                                      "gemm_mfma_f32<64x64x16, 4 waves, 4 sets>",
                                      "gemm_mfma_f32<64x64x16, 4 waves, 6 LDS stages>");
    }
}

// AUTO's choice, from timings of the split against one tile per workgroup
// on MI355X.  The split needs K to have at least 8 slices to share out,
// and then pays
//   * when some CUs would have no tile and the time that sharing saves --
//     (1 - tiles/CUs) of one tile's slices at the measured per-CU MFMA
//     rate (148 TFLOP/s over 256 CUs) -- covers the second launch (8 us;
//     200x300x4100: 20 tiles, 65 -> 18 us; 8192x64x2048: 128 tiles, 34 ->
//     29 us; not 768x768x1024: 144 tiles, 19 against 22 us);
//   * otherwise when one tile per workgroup would leave some CUs a whole
//     tile more work than the mean by at least 10% (split in parts), or in
//     stream-K runs, which need a launch of their own, by at least 10%
//     (256 x 128 tile), 15% (128 x 128) or 25% (64 x 64), and the product
//     is large enough (>= 4 GFLOP) to hide the second launch.  Measured on
//     64 x 64 tiles:
//     parts at 3-8% above the mean lost 0-3%, at 10.8%, 11.6% and 15.5%
//     (3000x2049x1531) gained 2%, 3% and 5%; runs at 5-15% ranged from -5%
//     to +3%, at 18.5% (2304^2 x 1000) lost 14% and at 58% (1152^2 x 8192)
//     gained 20%.  On the 8-wave tiles, one workgroup a CU: parts at 11%
//     (6144^2 x 1024) +6%, 28% (5000^2 x 1000) +21% (both now take 64x64
//     tiles, see pick); runs at 18.5%
//     (4608^2 x 4096) +11%, 28% (2560^3) +12%.
template <class T>
bool stream_k_pays(int64_t M, int64_t N, int64_t K) {
    const Split r = plan_split<T>(M, N, K, true);
    const SkPlan &p = r.sk;
    if (p.sk_tiles == 0 || p.ipt < 8) return false;
    const int64_t cus = device_cus();
    const int64_t tiles = static_cast<int64_t>(p.tiles_m) * p.tiles_n;
    if (tiles < cus) {
        const double slice_s = 2.0 * T::BM * T::BN * T::BK / (148e12 / 256);
        const double saved = (1.0 - static_cast<double>(tiles) / static_cast<double>(cus)) *
                             static_cast<double>(p.ipt) * slice_s;
        return saved >= 8e-6;
    }
    if (2.0 * static_cast<double>(M) * static_cast<double>(N) * static_cast<double>(K) < 4e9)
        return false;
    const double over = static_cast<double>(ceil_div(tiles, cus) * cus) /
                        static_cast<double>(tiles) - 1.0;
    // runs: 10% on the 256 x 128 tile (5880 x 3806 x 4096 +6.8%, 5659 x 4937
    // x 4096 +10.9% at 11% and 14%; +0.4 to +4.5% at 6-7%), 15% on the
    // 128 x 128 tile (at 7% and K = 2048 the runs lost 4-5%), 25% on the
    // 64 x 64 tiles
    const double runs = T::BM == 256 ? 0.10 : (T::THREADS == 512 ? 0.15 : 0.25);
    return over >= (r.pp.parts > 0 ? 0.10 : runs);
}

bool prefer_stream_k(int64_t M, int64_t N, int64_t K) {
    switch (pick(M, N, K)) {
        case Shape::kLarge: return stream_k_pays<TileLarge>(M, N, K);
        case Shape::kMid: return stream_k_pays<TileMid>(M, N, K);
        case Shape::kMany: return stream_k_pays<TileMany>(M, N, K);
        default: return stream_k_pays<TileDeep>(M, N, K);
    }
}

hipError_t launch_mfma(const GemmArgs &a, bool stream_k, void *ws, size_t ws_bytes) {
    switch (pick(a.M, a.N, a.K)) {
        case Shape::kLarge: return launch_tile<TileLarge>(a, stream_k, ws, ws_bytes);
        case Shape::kMid: return launch_tile<TileMid>(a, stream_k, ws, ws_bytes);
        case Shape::kMany: return launch_tile<TileMany>(a, stream_k, ws, ws_bytes);
        default: return launch_tile<TileDeep>(a, stream_k, ws, ws_bytes);
    }
}

}  // namespace tra
