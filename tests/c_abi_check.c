/* The public header, compiled as C11, against the built library: layouts,
 * enum values, and the entry points that make no HIP call (plan, ring
 * bounds, argument errors, status strings).  Built and run by
 * tests/test_abi_cpu.py; needs no GPU. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ptored.h"

#define CHECK(c)                                                  \
    do {                                                          \
        if (!(c)) {                                               \
            printf("FAIL line %d: %s\n", __LINE__, #c);           \
            return 1;                                             \
        }                                                         \
    } while (0)

int main(void) {
    CHECK(ptored_abi_version() == PTORED_ABI_VERSION);
    CHECK(ptored_max_ranks() == PTORED_MAX_RANKS);
    CHECK(sizeof(ptored_tuning) == 16 && offsetof(ptored_tuning, max_launch_bytes) == 8);
    CHECK(sizeof(ptored_plan_info) == 40 && offsetof(ptored_plan_info, wgs_per_cu) == 32);
    CHECK(PTORED_F32 == 0 && PTORED_BF16 == 1 && PTORED_F16 == 2 && PTORED_I32 == 3);
    CHECK(PTORED_SUM == 0 && PTORED_MAX == 1 && PTORED_MIN == 2 && PTORED_PROD == 3);

    /* plans on made-up device addresses: planning makes no HIP call */
    const void* srcs[17];
    for (int r = 0; r < 17; ++r) srcs[r] = (const void*)(uintptr_t)(0x100000000ull * (r + 1));
    void* dst = (void*)(uintptr_t)0x7000000000ull;
    ptored_plan_info info;
    memset(&info, 0xAB, sizeof info);
    CHECK(ptored_treduce_plan(srcs, 16, 0, dst, 4096, 4096, 4096, 4096, 4096, PTORED_I32,
                              PTORED_SUM, NULL, &info) == PTORED_OK);
    CHECK(info.path == PTORED_PATH_VEC_FIXED && info.rows_mode == 0 && info.launches == 1);
    CHECK(info.vec_elems == 4 && info.slots == 4096 * 1024 && info.wgs_per_cu == 6);
    CHECK(info.lead == 0);
    ptored_tuning t = {PTORED_FORCE_RUNTIME_N | PTORED_FULL_OCCUPANCY, 0, 0};
    CHECK(ptored_treduce_plan(srcs, 17, 3, dst, 8191, 12287, 12288, 8191, 12287, PTORED_F16,
                              PTORED_MAX, &t, &info) == PTORED_OK);
    CHECK(info.path == PTORED_PATH_VEC_RUNTIME && info.rows_mode == 1 && info.wgs_per_cu == 0);

    /* argument errors come back before any HIP call */
    CHECK(ptored_treduce(srcs, 0, 0, dst, 1, 1, 1, 1, 1, PTORED_F32, PTORED_SUM, NULL) ==
          PTORED_ERR_INVALID_ARG);
    CHECK(ptored_treduce(srcs, 2, 2, dst, 1, 1, 1, 1, 1, PTORED_F32, PTORED_SUM, NULL) ==
          PTORED_ERR_INVALID_ARG);
    CHECK(ptored_treduce(srcs, 2, 0, dst, 1, 1, 1, 1, 1, 9, PTORED_SUM, NULL) ==
          PTORED_ERR_UNSUPPORTED);
    CHECK(ptored_treduce(srcs, 2, 0, (char*)srcs[0] + 4, 4, 4, 4, 4, 4, PTORED_F32, PTORED_SUM,
                         NULL) == PTORED_ERR_OVERLAP);
    CHECK(ptored_allreduce((void* const*)srcs, 2, 0, 2, 3, 2, 2, 2, PTORED_F32, PTORED_SUM,
                           NULL, NULL) == PTORED_ERR_INVALID_ARG); /* cols > ld */

    int64_t b[5];
    CHECK(ptored_ring_bounds(100, 4, PTORED_F32, b) == PTORED_OK);
    CHECK(b[0] == 0 && b[1] == 25 && b[2] == 50 && b[3] == 75 && b[4] == 100);
    CHECK(ptored_ring_bounds(100, 4, PTORED_BF16, b) == PTORED_OK);
    CHECK(b[1] == 32 && b[2] == 64 && b[3] == 80 && b[4] == 100);
    CHECK(strncmp(ptored_status_string(PTORED_ERR_OVERLAP), "PTORED_ERR_OVERLAP", 18) == 0);
    printf("c abi ok\n");
    return 0;
}
