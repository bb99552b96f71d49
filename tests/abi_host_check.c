/*
 * Host-only exercise of the C ABI (include/tra_gemm.h), built and run under
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_sanitizers.py.  Every call here is answered on the host:
 * names, plans (tra_gemm_describe into buffers of every small length),
 * workspace sizes, calls rejected by the argument checks, and the release
 * of workspaces when none was allocated.  Nothing is
 * launched, so no GPU is needed.  Exits 0 and prints "ok" when every
 * result is as the header documents.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tra_gemm.h"

#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

int main(void) {
    static const int64_t shapes[][3] = {
        {1, 1, 1},       {1024, 1024, 1024}, {4096, 4096, 4096}, {3000, 2049, 1531},
        {16384, 64, 16384}, {0, 5, 5},      {5, 0, 5},          {5, 5, 0},
        {200, 300, 4100}, {64, 64, 100000}, {100000, 100000, 1000},
        {(int64_t)1 << 31, 64, 64},
    };
    const int nshapes = (int)(sizeof shapes / sizeof shapes[0]);
    static const size_t lens[] = {1, 2, 7, 16, 64, 200, 512};
    char buf[600];

    for (int s = -3; s < 8; ++s) CHECK(tra_status_string(s) != NULL);
    for (int v = -3; v < 9; ++v) CHECK(tra_gemm_variant_name(v) != NULL);

    for (int v = 0; v <= TRA_GEMM_MFMA_STREAMK; ++v) {
        for (int i = 0; i < nshapes; ++i) {
            const int64_t M = shapes[i][0], N = shapes[i][1], K = shapes[i][2];
            for (size_t l = 0; l < sizeof lens / sizeof lens[0]; ++l) {
                memset(buf, 'x', sizeof buf);
                CHECK(tra_gemm_describe(v, M, N, K, buf, lens[l]) == TRA_OK);
                CHECK(memchr(buf, 0, lens[l]) != NULL);   /* NUL-terminated in range */
                CHECK(buf[lens[l]] == 'x');                 /* nothing past len */
            }
            size_t bytes = 12345;
            CHECK(tra_gemm_workspace_size(v, M, N, K, &bytes) == TRA_OK);
            CHECK(v == TRA_GEMM_MFMA_STREAMK || v == TRA_GEMM_AUTO || bytes == 0);
        }
        CHECK(tra_gemm_describe(v, 4, 4, 4, NULL, 0) == TRA_OK);
        CHECK(tra_gemm_describe(v, 4, 4, 4, NULL, 8) == TRA_ERR_INVALID_ARG);
        CHECK(tra_gemm_describe(v, -1, 4, 4, buf, sizeof buf) == TRA_ERR_INVALID_ARG);
        CHECK(tra_gemm_workspace_size(v, 4, 4, -4, &(size_t){0}) == TRA_ERR_INVALID_ARG);
        CHECK(tra_gemm_workspace_size(v, 4, 4, 4, NULL) == TRA_ERR_INVALID_ARG);
    }
    CHECK(tra_gemm_describe(99, 4, 4, 4, buf, sizeof buf) == TRA_ERR_INVALID_ARG);

    /* rejected before any HIP call: fake, never-dereferenced addresses */
    const float *A = (const float *)(uintptr_t)0x10000000;
    const float *B = (const float *)(uintptr_t)0x20000000;
    float *C = (float *)(uintptr_t)0x30000000;
    CHECK(gemm_f32(-1, 4, 4, A, 4, B, 4, C, 4, NULL) == TRA_ERR_INVALID_ARG);
    CHECK(gemm_f32(4, 4, 4, NULL, 4, B, 4, C, 4, NULL) == TRA_ERR_INVALID_ARG);
    CHECK(gemm_f32(4, 4, 8, A, 7, B, 4, C, 4, NULL) == TRA_ERR_INVALID_ARG);
    CHECK(gemm_f32(4, 8, 4, A, 4, B, 7, C, 8, NULL) == TRA_ERR_INVALID_ARG);
    CHECK(gemm_f32(4, 4, 4, A, 4, B, 4, (float *)A + 4, 4, NULL) == TRA_ERR_INVALID_ARG);
    CHECK(gemm_f32_variant(42, 4, 4, 4, A, 4, B, 4, C, 4, NULL) == TRA_ERR_INVALID_ARG);
    CHECK(gemm_f32_variant_ws(TRA_GEMM_MFMA_STREAMK, 3000, 2049, 1531, A, 1531, B, 2049, C,
                              2049, NULL, 1, NULL) == TRA_ERR_INVALID_ARG);
    /* 2^24 workgroups of 256 lanes: 2^32 lanes, past HIP's limit */
    CHECK(gemm_f32_variant(TRA_GEMM_NAIVE, (int64_t)1 << 26, 64, 0, NULL, 0, NULL, 64, C, 64,
                           NULL) == TRA_ERR_UNSUPPORTED);
    /* the no-alloc entry point: a split past its static scratch is refused */
    CHECK(gemm_f32_variant_noalloc(TRA_GEMM_MFMA_STREAMK, 4608, 4608, 4096, A, 4096, B, 4608, C,
                                   4608, NULL) == TRA_ERR_UNSUPPORTED);
    CHECK(gemm_f32_variant_noalloc(42, 4, 4, 4, A, 4, B, 4, C, 4, NULL) == TRA_ERR_INVALID_ARG);
    /* nothing to compute: OK, no launch */
    CHECK(gemm_f32(0, 4, 4, NULL, 4, NULL, 4, NULL, 4, NULL) == TRA_OK);
    /* no workspace was allocated: nothing to release */
    CHECK(tra_gemm_release_workspaces() == TRA_OK);
    printf("ok\n");
    return 0;
}
