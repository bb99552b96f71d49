// Host-only check of the workgroup -> tile maps in gemm_internal.h, built
// and run by tests/test_tile_maps.py (no GPU): the 32-bit maps equal the
// 64-bit ones, xcd_remap is a bijection on [0, n), and grouped_tile visits
// every (tile row, tile column) exactly once.  Prints "ok" and exits 0.
#include <cstdio>
#include <vector>

#include "gemm_internal.h"

int main() {
    const int dims[] = {1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 33, 64, 100, 257};
    for (int tm_n : dims) {
        for (int tn_n : dims) {
            const int n = tm_n * tn_n;
            std::vector<int> seen_id(n, 0), seen_tile(n, 0), seen4(n, 0);
            for (int b = 0; b < n; ++b) {
                const int id = tra::xcd_remap32(b, n);
                if (id != tra::xcd_remap(b, n) || id < 0 || id >= n || seen_id[id]++) {
                    std::printf("xcd_remap32 wrong: n=%d b=%d id=%d\n", n, b, id);
                    return 1;
                }
                int tm, tn;
                int64_t tm64, tn64;
                tra::grouped_tile32<8>(id, tm_n, tn_n, tm, tn);
                tra::grouped_tile(id, tm_n, tn_n, 8, tm64, tn64);
                int tm4, tn4;
                int64_t tm4_64, tn4_64;
                tra::grouped_tile32<4>(id, tm_n, tn_n, tm4, tn4);
                tra::grouped_tile(id, tm_n, tn_n, 4, tm4_64, tn4_64);
                if (tm4 != tm4_64 || tn4 != tn4_64 || tm4 < 0 || tm4 >= tm_n || tn4 < 0 ||
                    tn4 >= tn_n || seen4[tm4 * tn_n + tn4]++) {
                    std::printf("grouped_tile32<4> wrong: %dx%d id=%d\n", tm_n, tn_n, id);
                    return 1;
                }
                if (tm != tm64 || tn != tn64 || tm < 0 || tm >= tm_n || tn < 0 || tn >= tn_n ||
                    seen_tile[tm * tn_n + tn]++) {
                    std::printf("grouped_tile32 wrong: %dx%d id=%d -> %d,%d (%lld,%lld)\n", tm_n,
                                tn_n, id, tm, tn, (long long)tm64, (long long)tn64);
                    return 1;
                }
            }
        }
    }
    // the largest grid the host accepts for 256-lane workgroups: 2^24 tiles
    const int big_m = 1 << 12, big_n = 1 << 12, big = big_m * big_n;
    for (int b : {0, 1, 7, 8, big / 2 + 3, big - 9, big - 1}) {
        const int id = tra::xcd_remap32(b, big);
        int tm, tn;
        int64_t tm64, tn64;
        tra::grouped_tile32<8>(id, big_m, big_n, tm, tn);
        tra::grouped_tile(id, big_m, big_n, 8, tm64, tn64);
        if (id != tra::xcd_remap(b, big) || tm != tm64 || tn != tn64) {
            std::printf("large grid mismatch at b=%d\n", b);
            return 1;
        }
    }
    std::printf("ok\n");
    return 0;
}
