/*
 * tra_gemm.h -- C ABI of the MI355X (gfx950) single-precision GEMM library
 * libtra_gemm.so.
 *
 * The operation is C = A x B on row-major binary32 matrices:
 *
 *     C[i*ldc + j] := sum over k < K of A[i*lda + k] * B[k*ldb + j]
 *                     for 0 <= i < M, 0 <= j < N.
 *
 * Definition: page "GEMM kernel test code & optimization (1024^3 experiment)"
 * (teach-meaning.tistory.com/1513), section "Mathematical definition" (one
 * k-sum per element of C, 2*M*N*K flops) and section "Memory layout"
 * (row-major: A[row*K + k], B[k*N + col], C[row*N + col]; here the leading
 * dimensions lda, ldb, ldc generalise K, N, N).  The result overwrites C:
 * the accumulator starts at zero and is stored once, as in both kernels of
 * that page (sections "How the naive GEMM kernel works" and "Shared-memory
 * tiled GEMM").  Elements of C outside the first N columns of each row are
 * never touched.
 *
 * Ownership and memory: A, B and C are device pointers owned by the caller
 * (for example torch tensors on the current HIP device).  No entry point
 * allocates, frees or copies host memory; all work is enqueued on `stream`.
 * Only the stream-K variant needs device scratch (partial tiles, see
 * TRA_GEMM_MFMA_STREAMK): gemm_f32_variant_ws takes it from the caller and
 * allocates nothing; gemm_f32 and gemm_f32_variant use a workspace that the
 * library allocates on first need for each (device, stream) pair -- for
 * hipStreamPerThread, for each (device, thread) -- and keeps until
 * tra_gemm_release_workspaces() or the end of the process.  When a call
 * needs more, the buffer grows in stream order (hipFreeAsync of the old one
 * and hipMallocAsync of the new one, both on `stream`): nothing waits on
 * the host, and calls on different streams never wait for each other.
 * The pair is keyed by the stream's handle, and calls on one handle rely on
 * the stream's order: synchronise a stream that has such calls in flight
 * before destroying it, since a stream created later may be given the same
 * handle.  While `stream` is being captured into a graph these two entry
 * points refuse a call that needs scratch (TRA_ERR_UNSUPPORTED): capture
 * takes gemm_f32_variant_ws, whose buffer the caller keeps alive for as
 * long as the graph.
 *
 * Asynchrony: gemm_f32 and gemm_f32_variant return once the kernels are
 * enqueued on `stream` (a hipStream_t; NULL means the null stream of the
 * current device).  Synchronise the stream before reading C on the host.
 *
 * Errors: every entry point returns a tra_status and never throws.  The
 * argument checks run on the host before anything is enqueued; a rejected
 * call leaves C untouched.  A launch failure returns TRA_ERR_HIP and keeps
 * the hipError_t for tra_last_hip_error() (per calling thread).
 *
 * Numerics: products and sums are binary32 with round-to-nearest-even.  The
 * order of the k-sum depends on the variant and tile shape, so results on
 * general inputs may differ between variants in the last bits; inputs whose
 * partial sums are all exactly representable (e.g. small integers) give
 * identical bits in every variant.
 */
#ifndef TRA_GEMM_H
#define TRA_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the ABI are the only ones the library exports. */
#define TRA_API __attribute__((visibility("default")))

typedef enum tra_status {
    TRA_OK = 0,
    TRA_ERR_INVALID_ARG = 1,   /* a size, stride, pointer or variant is invalid */
    TRA_ERR_UNSUPPORTED = 2,   /* valid but beyond this library (e.g. grid too large) */
    TRA_ERR_HIP = 3            /* the HIP runtime reported an error */
} tra_status;

/*
 * The kernel ladder.  Each rung is a hand-written gfx950 kernel and each
 * handles shapes that are not tile multiples by zero-filling the staged
 * tiles and masking the stores.
 *   NAIVE        one lane per element of C, K-loop straight from global
 *                memory (page "GEMM kernel test code & optimization
 *                (1024^3 experiment)", section "How the naive GEMM kernel
 *                works").
 *   LDS_TILED    16x16 tiles of C, slices of A and B 64 deep staged in
 *                LDS, each lane one element of C, zero-filled outside the
 *                matrices (same page, sections "Tile concept" and
 *                "Shared-memory tiled GEMM"; page "[AutoMine++] #2 matmul
 *                trial and error", section "Breaking the memory bottleneck:
 *                Tiling").
 *   REGBLOCK_DB  128x128 block tile with an 8x8 register micro-tile per
 *                lane (64x64 with 4x4 when the large tiles are too few),
 *                double-buffered LDS with register prefetch (VALU FMA);
 *                with no more 64x64 tiles than CUs, each tile's workgroup
 *                splits K over 2-4 lane groups.
 *   MFMA         CDNA matrix-core kernel on binary32 inputs
 *                (v_mfma_f32_32x32x2_f32), tile shape chosen from the
 *                problem shape, one tile per workgroup; slices staged
 *                through registers into two LDS buffers, or, on the 64x64
 *                tiles when rows are 16-byte aligned, K is a multiple of 4
 *                and there are at least 13 slices of 16, loaded straight
 *                into a ring of six LDS stages.
 *   MFMA_STREAMK the MFMA kernel with the tile count decoupled from the
 *                workgroup count.  When the tiles do not fill whole waves
 *                of resident workgroups (the tile-size versus occupancy
 *                trade-off of page "Roofline & Tiling notes",
 *                legato-user-group.github.io/tensor2silicon-lab/week04/
 *                researchers/jaehyeong, key points), the tiles of the last
 *                partial wave are split along K, in one of two forms:
 *                "parts", when they fit in half a wave and spread evenly,
 *                each tile cut into up to 8 equal runs of K slices that run
 *                in the same launch as the other tiles; otherwise "runs",
 *                their slices shared out evenly over one wave of
 *                workgroups in a launch of their own, a run crossing tiles
 *                (the stream-K decomposition of Osama et al., "Stream-K:
 *                Work-centric Parallel Decomposition for Dense Matrix-
 *                Matrix Multiplication on the GPU", 2023).  The partial
 *                sums of each split tile are added in K order by a second
 *                kernel, so results are deterministic.  Needs a device
 *                workspace of tra_gemm_workspace_size() bytes; without a
 *                split it runs the MFMA launch.
 *   AUTO         the library's choice for the shape: MFMA, or MFMA_STREAMK
 *                where a split is predicted to pay.
 */
typedef enum tra_gemm_variant {
    TRA_GEMM_AUTO = 0,
    TRA_GEMM_NAIVE = 1,
    TRA_GEMM_LDS_TILED = 2,
    TRA_GEMM_REGBLOCK_DB = 3,
    TRA_GEMM_MFMA = 4,
    TRA_GEMM_MFMA_STREAMK = 5
} tra_gemm_variant;

#define TRA_GEMM_VARIANT_COUNT 6

/*
 * gemm_f32: C = A x B with the library's choice of kernel (TRA_GEMM_AUTO).
 *
 *   M, N, K  sizes; M, N, K >= 0.  M == 0 or N == 0 is a no-op (TRA_OK,
 *            pointers unused).  K == 0 writes C := 0.
 *   A        device pointer to M rows of lda floats, row-major (may be NULL
 *            when K == 0); lda >= K.
 *   B        device pointer to K rows of ldb floats, row-major (may be NULL
 *            when K == 0); ldb >= N.
 *   C        device pointer to M rows of ldc floats, row-major; ldc >= N;
 *            overwritten.  C must not overlap A or B.
 *   stream   hipStream_t on the current device, or NULL.
 *
 * Pointers need only 4-byte alignment; 16-byte aligned bases with
 * leading dimensions divisible by 4 take the vector-load path.
 *
 * Returns TRA_OK, TRA_ERR_INVALID_ARG (negative size, ld too small, NULL
 * pointer where data is needed, C overlapping A or B), TRA_ERR_UNSUPPORTED
 * (the launch grid would exceed 2^31 - 1 workgroups or 2^32 - 1 lanes, or
 * the call needs the library's scratch while `stream` is being captured) or
 * TRA_ERR_HIP (a launch failed, or the library's stream-K workspace could
 * not be allocated).
 */
TRA_API tra_status gemm_f32(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    float *C, int64_t ldc,
                    void *stream);

/*
 * gemm_f32_variant: as gemm_f32 but runs the given rung of the ladder
 * (a tra_gemm_variant value).  An unknown variant is TRA_ERR_INVALID_ARG.
 */
TRA_API tra_status gemm_f32_variant(int variant,
                            int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda,
                            const float *B, int64_t ldb,
                            float *C, int64_t ldc,
                            void *stream);

/*
 * gemm_f32_variant_ws: as gemm_f32_variant, with device scratch supplied by
 * the caller instead of the library's: `workspace` (16-byte aligned device
 * memory on the current device, owned by the caller) of `workspace_bytes`
 * bytes, at least tra_gemm_workspace_size() for the same variant and
 * sizes.  It may be NULL when that size is 0.  Calls that share a workspace
 * must be ordered (e.g. on one stream); it holds no state between calls.
 * Allocates nothing.  A workspace that is too small or NULL when one is
 * needed is TRA_ERR_INVALID_ARG.
 */
TRA_API tra_status gemm_f32_variant_ws(int variant,
                               int64_t M, int64_t N, int64_t K,
                               const float *A, int64_t lda,
                               const float *B, int64_t ldb,
                               float *C, int64_t ldc,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * gemm_f32_variant_noalloc: as gemm_f32_variant, for callers that cannot
 * allocate device memory -- code under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing, on the
 * host or the device: the stream-K split's partial tiles go to a scratch
 * array of TRA_STATIC_SCRATCH_BYTES that is part of the library's code
 * object (one per device, held until the process ends).  A call whose
 * split needs more than that (tra_gemm_workspace_size) is refused with
 * TRA_ERR_UNSUPPORTED before anything is enqueued; such callers pass their
 * own buffer to gemm_f32_variant_ws instead.  Every call on a device
 * shares that device's one array, and a call leaves its partial tiles
 * there: calls that may overlap in time on one device (on different
 * streams, or from threads without ordering) race and must be ordered by
 * the caller, e.g. issued on one stream.  Nothing in the array needs to
 * start at zero.  The first call on each device looks up the array's
 * device address (hipGetSymbolAddress); a caller that captures graphs
 * makes one call on each device before capturing.  Otherwise the same
 * arguments, results and status codes as gemm_f32_variant.
 */
#define TRA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

TRA_API tra_status gemm_f32_variant_noalloc(int variant,
                                    int64_t M, int64_t N, int64_t K,
                                    const float *A, int64_t lda,
                                    const float *B, int64_t ldb,
                                    float *C, int64_t ldc,
                                    void *stream);

/*
 * tra_gemm_workspace_size: device scratch in bytes that gemm_f32_variant_ws
 * needs for this variant and these sizes on the current device (0 for every
 * variant except a stream-K split), written to *bytes.  Returns
 * TRA_ERR_INVALID_ARG for an unknown variant, negative sizes or bytes ==
 * NULL.
 */
TRA_API tra_status tra_gemm_workspace_size(int variant, int64_t M, int64_t N, int64_t K,
                                   size_t *bytes);

/*
 * tra_gemm_describe: writes a one-line, NUL-terminated description of the
 * launch that gemm_f32_variant(variant, M, N, K, ...) would make for
 * 16-byte-aligned operands with lda = K, ldb = N, ldc = N (kernel name, tile
 * shape, grid and block size, the split tiles and the workgroups that run
 * them, the form of the split -- "none", "parts" or "runs", see
 * TRA_GEMM_MFMA_STREAMK -- and workspace bytes) into buf[0 .. len-1].
 * Launches nothing; the split is planned for the current device's CU count
 * and occupancy, or for MI355X's (256 CUs) when no device is present.  Returns TRA_OK, or TRA_ERR_INVALID_ARG for an
 * unknown variant, negative sizes, or buf == NULL with len > 0.
 */
TRA_API tra_status tra_gemm_describe(int variant, int64_t M, int64_t N, int64_t K,
                             char *buf, size_t len);

/*
 * Measurement probes: the two roofs of the roofline model measured on the
 * device (page "Roofline & Tiling notes", legato-user-group.github.io/
 * tensor2silicon-lab/week04/researchers/jaehyeong: performance is bounded
 * by min(peak flops, bandwidth x arithmetic intensity); its section 1 uses a
 * vector add as the example with no reuse).  Each call enqueues one kernel
 * on `stream` and returns; time it with events.  tra_probe_work() gives the
 * work one call does: bytes moved for TRA_PROBE_COPY (amount = n), flops
 * for TRA_PROBE_MFMA and TRA_PROBE_FMA (amount = iters); -1 for an unknown
 * probe or a negative amount.
 *
 *   tra_probe_copy_f32  dst[i] = src[i] for i < n (float4 stream; src and
 *                       dst 16-byte aligned and not overlapping, else
 *                       TRA_ERR_INVALID_ARG).  Use buffers larger than the
 *                       256 MB last-level cache to measure HBM.
 *   tra_probe_mfma_f32  TRA_PROBE_BLOCKS workgroups of 4 waves, each wave
 *                       `iters` rounds of 4 independent FP32 MFMAs
 *                       (v_mfma_f32_32x32x2_f32) from registers.
 *   tra_probe_fma_f32   the same grid, each lane `iters` rounds of 8
 *                       independent v_fma_f32.
 *   tra_probe_launch    `workgroups` workgroups of 256 lanes that do
 *                       nothing (1 <= workgroups, workgroups x 256 <=
 *                       2^32 - 1, else TRA_ERR_INVALID_ARG): timed back to
 *                       back, the cost of a launch that does no work -- the
 *                       floor under any one-launch GEMM's time.
 * The compute probes write TRA_PROBE_SINK_FLOATS floats of no meaning to
 * `sink` (device memory owned by the caller).
 */
typedef enum tra_probe {
    TRA_PROBE_COPY = 0,
    TRA_PROBE_MFMA = 1,
    TRA_PROBE_FMA = 2
} tra_probe;

#define TRA_PROBE_BLOCKS 1024
#define TRA_PROBE_SINK_FLOATS (TRA_PROBE_BLOCKS * 256)

TRA_API double tra_probe_work(int probe, int64_t amount);
TRA_API tra_status tra_probe_copy_f32(int64_t n, const float *src, float *dst, void *stream);
TRA_API tra_status tra_probe_mfma_f32(int64_t iters, float *sink, void *stream);
TRA_API tra_status tra_probe_fma_f32(int64_t iters, float *sink, void *stream);
TRA_API tra_status tra_probe_launch(int64_t workgroups, void *stream);

/*
 * tra_gemm_release_workspaces: frees every workspace that gemm_f32 and
 * gemm_f32_variant allocated (on every device and stream), for a caller
 * about to unload the library or to hand the memory back.  It first waits
 * for all work on each such device (hipDeviceSynchronize), since the
 * streams the buffers served may no longer exist.  Later calls allocate
 * again as needed.  Returns TRA_OK, or TRA_ERR_HIP (kept for
 * tra_last_hip_error()) if a wait or release failed; the current device is
 * restored either way.
 */
TRA_API tra_status tra_gemm_release_workspaces(void);

/* Static strings for a status or variant value ("unknown" otherwise). */
TRA_API const char *tra_status_string(int status);
TRA_API const char *tra_gemm_variant_name(int variant);

/*
 * The hipError_t of the last call on this thread that returned TRA_ERR_HIP
 * (0 if none).  Not cleared by later successful calls.
 */
TRA_API int tra_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TRA_GEMM_H */
