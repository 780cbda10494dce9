/* host_launches.c -- drives the library's host code (checks, plans, launch
 * splitting) through the C ABI with made-up device addresses, linked against
 * tests/sanitize/hip_stub.cpp instead of the HIP runtime and kernels.  Built
 * with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitize_cpu.py; needs no GPU.
 *
 * For every call the stub records the byte window [base, base + extent) of
 * every buffer each launch would address.  The checks: every window lies
 * within its buffer's span (less the at most 1 KiB the slot origin may sit
 * before the pointer), every extent fits 32-bit buffer offsets, and the
 * windows of each buffer cover every valid row.  Shapes include calls past
 * 2 GiB (several launches), rows longer than one launch, misaligned
 * pointers, odd pitches, every forced kernel family and walk, the in-place
 * allreduce, the ring reduce-scatter and push-with-add. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ptored.h"

long stub_take_record(long* bad_launches, uintptr_t* lo, uintptr_t* hi, long cap, long* nwin);

#define MAXWIN 200000
static uintptr_t wlo[MAXWIN], whi[MAXWIN];
static int failures = 0;

#define FAIL(...)                                   \
    do {                                            \
        printf("FAIL %s: ", label);                 \
        printf(__VA_ARGS__);                        \
        printf("\n");                               \
        ++failures;                                 \
        return;                                     \
    } while (0)

static int esize(int dt) { return (dt == PTORED_F32 || dt == PTORED_I32) ? 4 : 2; }

/* Fake device address of buffer k: 64 GiB apart, plus a byte offset. */
static uintptr_t fake(int k, int off) { return ((uintptr_t)(k + 1) << 36) + (uintptr_t)off; }

/* Is [lo, hi) covered by the union of the windows that start inside
 * [blo, bhi) (the windows of one buffer)? */
static int covered(long nwin, uintptr_t blo, uintptr_t bhi, uintptr_t lo, uintptr_t hi) {
    uintptr_t at = lo;
    int moved = 1;
    while (at < hi && moved) {
        moved = 0;
        for (long k = 0; k < nwin; ++k)
            if (wlo[k] >= blo && wlo[k] < bhi && wlo[k] <= at && whi[k] > at) {
                at = whi[k];
                moved = 1;
            }
    }
    return at >= hi;
}

/* Check the record of one call against the buffers it was given: `bufs`
 * (nbuf of them) with `span` bytes each from the pointer, rows of the valid
 * rectangle at pitch `ldb` bytes, `vrow` bytes valid per row; the first
 * `ncover` buffers must have every valid row addressable. */
static void check_record(const char* label, const uintptr_t* bufs, int nbuf, int ncover,
                         int64_t span, int64_t vr, int64_t ldb, int64_t vrow,
                         long want_launches) {
    long bad = 0, nwin = 0;
    const long launches = stub_take_record(&bad, wlo, whi, MAXWIN, &nwin);
    if (bad) FAIL("%ld launches flagged by the stub", bad);
    if (nwin > MAXWIN) FAIL("too many windows (%ld)", nwin);
    if (want_launches >= 0 && launches != want_launches)
        FAIL("%ld launches, expected %ld", launches, want_launches);
    for (long k = 0; k < nwin; ++k) {
        int inside = 0;
        for (int b = 0; b < nbuf && !inside; ++b)
            inside = wlo[k] + 1024 > bufs[b] && whi[k] <= bufs[b] + (uintptr_t)span &&
                     wlo[k] <= whi[k];
        if (!inside)
            FAIL("window [%#lx, %#lx) outside every buffer", (unsigned long)wlo[k],
                 (unsigned long)whi[k]);
    }
    if (vr == 0 || vrow == 0) {
        if (launches != 0) FAIL("an empty region launched %ld kernels", launches);
        return;
    }
    /* first, middle and last valid rows of every buffer are addressable */
    const int64_t rows_to_check[3] = {0, vr / 2, vr - 1};
    for (int b = 0; b < ncover; ++b)
        for (int k = 0; k < 3; ++k) {
            const uintptr_t lo = bufs[b] + (uintptr_t)(rows_to_check[k] * ldb);
            if (!covered(nwin, bufs[b] - 1024, bufs[b] + (uintptr_t)span, lo,
                         lo + (uintptr_t)vrow))
                FAIL("buffer %d row %lld not covered", b, (long long)rows_to_check[k]);
        }
}

static void reduce_case(const char* label, int n, int dt, int64_t rows, int64_t cols, int64_t ld,
                        int64_t vr, int64_t vc, uint32_t flags, const int* offs, int dst_off,
                        long want_launches) {
    uintptr_t bufs[PTORED_MAX_RANKS + 1];
    const void* srcs[PTORED_MAX_RANKS];
    for (int r = 0; r < n; ++r) {
        bufs[r] = fake(r, offs ? offs[r] : 0);
        srcs[r] = (const void*)bufs[r];
    }
    bufs[n] = fake(n, dst_off);
    const ptored_tuning t = {flags, 0, 0};
    const int es = esize(dt);
    const int st = ptored_treduce_ex(srcs, n, n / 2, (void*)bufs[n], rows, cols, ld, vr, vc, dt,
                                     PTORED_SUM, &t, 0);
    if (st != PTORED_OK) {
        long bad, nwin;
        stub_take_record(&bad, wlo, whi, 0, &nwin);
        FAIL("status %d", st);
    }
    const int64_t span = vr && vc ? ((vr - 1) * ld + vc) * es : 0;
    check_record(label, bufs, n + 1, n + 1, span, vr, ld * es, vc * es, want_launches);
}

static void expect_status(const char* label, int got, int want) {
    long bad, nwin;
    const long launches = stub_take_record(&bad, wlo, whi, 0, &nwin);
    if (got != want) FAIL("status %d, expected %d", got, want);
    if (launches != 0) FAIL("a rejected call launched %ld kernels", launches);
}

int main(void) {
    const int64_t G = (int64_t)1 << 30;
    int offs[PTORED_MAX_RANKS];

    /* the five workloads' shapes */
    reduce_case("n2 f32 16x16", 2, PTORED_F32, 16, 16, 16, 16, 16, 0, NULL, 0, 1);
    reduce_case("n4 f32 1000x1000 in 1024^2", 4, PTORED_F32, 1024, 1024, 1024, 1000, 1000, 0,
                NULL, 0, 1);
    reduce_case("n8 bf16 8192^2", 8, PTORED_BF16, 8192, 8192, 8192, 8192, 8192, 0, NULL, 0, 1);
    reduce_case("n16 i32 4096^2", 16, PTORED_I32, 4096, 4096, 4096, 4096, 4096, 0, NULL, 0, 1);
    reduce_case("n8 f16 ragged", 8, PTORED_F16, 8192, 12288, 12288, 8191, 12287, 0, NULL, 0, 1);
    reduce_case("n8 bf16 8192^2 row tiles", 8, PTORED_BF16, 8192, 8192, 8192, 8192, 8192,
                PTORED_FORCE_ROWS | PTORED_ROW_TILES, NULL, 0, 1);
    reduce_case("n8 f16 ragged flat", 8, PTORED_F16, 8192, 12288, 12288, 8191, 12287,
                PTORED_FORCE_ROWS | PTORED_FLAT_WALK, NULL, 0, 1);
    reduce_case("n8 f16 ragged lds", 8, PTORED_F16, 8192, 12288, 12288, 8191, 12287,
                PTORED_LDS_PINGPONG, NULL, 0, 1);
    reduce_case("n8 f16 ragged elementwise", 8, PTORED_F16, 8192, 12288, 12288, 8191, 12287,
                PTORED_FORCE_ELEMENTWISE, NULL, 0, 1);
    reduce_case("n40 i32 runtime loop", 40, PTORED_I32, 512, 1000, 1024, 500, 999, 0, NULL, 0, 1);
    reduce_case("n3 i32 runtime forced", 3, PTORED_I32, 64, 64, 64, 64, 64,
                PTORED_FORCE_RUNTIME_N, NULL, 0, 1);
    /* empty and single-rank */
    reduce_case("empty rows", 4, PTORED_F32, 16, 16, 16, 0, 16, 0, NULL, 0, 0);
    reduce_case("empty cols", 4, PTORED_F32, 16, 16, 16, 16, 0, 0, NULL, 0, 0);
    reduce_case("n1 copy", 1, PTORED_F16, 300, 301, 305, 299, 300, 0, NULL, 0, -1);
    /* misaligned pointers: a common offset, then differing offsets */
    for (int r = 0; r < 8; ++r) offs[r] = 6;
    reduce_case("n8 f16 common offset 6", 8, PTORED_F16, 257, 1000, 1024, 257, 999, 0, offs, 6,
                -1);
    for (int r = 0; r < 8; ++r) offs[r] = 2 * (r % 8);
    reduce_case("n8 f16 mixed offsets", 8, PTORED_F16, 257, 1000, 1024, 257, 999, 0, offs, 4, -1);
    for (int r = 0; r < 8; ++r) offs[r] = 1000;
    reduce_case("n8 f32 offset 1000", 8, PTORED_F32, 100, 3000, 3000, 100, 3000, 0, offs, 1000,
                -1);
    /* pitch off the 16-byte grid */
    reduce_case("n5 f16 odd pitch", 5, PTORED_F16, 301, 201, 203, 300, 201, 0, NULL, 0, -1);
    reduce_case("n5 f32 pitch 3 mod 4", 5, PTORED_F32, 301, 201, 203, 300, 199, 0, NULL, 0, -1);
    /* past 2 GiB: contiguous spans, row bands, rows longer than one launch */
    reduce_case("n2 f32 3 GiB contiguous", 2, PTORED_F32, 3 * 16384, 16384, 16384, 3 * 16384,
                16384, 0, NULL, 0, 2);
    reduce_case("n2 bf16 5 GiB row bands", 2, PTORED_BF16, 40000, 60000, 65536, 40000, 59999, 0,
                NULL, 0, -1);
    reduce_case("n2 f32 rows of 2.5 GiB", 2, PTORED_F32, 3, 700000000, 700000000, 3, 699999999,
                0, NULL, 0, 6);
    for (int r = 0; r < 3; ++r) offs[r] = 12;
    reduce_case("n3 i32 3 GiB at offset 12", 3, PTORED_I32, 24576, 32768, 32768, 24576, 32768, 0,
                offs, 12, -1);
    reduce_case("n2 f16 3 GiB elementwise", 2, PTORED_F16, 3 * 32768, 16384, 16384, 3 * 32768,
                16384, PTORED_FORCE_ELEMENTWISE, NULL, 0, -1);

    /* in-place allreduce */
    {
        const char* label = "allreduce n8 f16 ragged";
        uintptr_t bufs[8];
        void* p[8];
        for (int r = 0; r < 8; ++r) p[r] = (void*)(bufs[r] = fake(r, 0));
        const int st = ptored_allreduce(p, 8, 0, 8192, 12288, 12288, 8191, 12287, PTORED_F16,
                                        PTORED_SUM, NULL, 0);
        if (st != PTORED_OK) {
            printf("FAIL %s: status %d\n", label, st);
            ++failures;
        }
        check_record(label, bufs, 8, 8, (8190LL * 12288 + 12287) * 2, 8191, 12288 * 2,
                     12287 * 2, 1);
    }
    /* ring reduce-scatter: one window, several windows (3 GiB streams), ragged */
    {
        const int64_t counts[3] = {(int64_t)4096 * 4096, 3 * G / 4 + 7, 1000003};
        const int dts[3] = {PTORED_I32, PTORED_F32, PTORED_F16};
        const int ns[3] = {16, 4, 7};
        for (int c = 0; c < 3; ++c) {
            char label[64];
            snprintf(label, sizeof label, "ring n%d count %lld", ns[c], (long long)counts[c]);
            uintptr_t bufs[2 * PTORED_MAX_RANKS];
            const void* s[PTORED_MAX_RANKS];
            void* d[PTORED_MAX_RANKS];
            for (int r = 0; r < ns[c]; ++r) {
                s[r] = (const void*)(bufs[r] = fake(r, 0));
                d[r] = (void*)(bufs[ns[c] + r] = fake(ns[c] + r, 0));
            }
            const int st = ptored_reduce_scatter_ring(s, ns[c], d, counts[c], dts[c], PTORED_SUM,
                                                      NULL, 0);
            if (st != PTORED_OK) {
                printf("FAIL %s: status %d\n", label, st);
                ++failures;
            }
            const int64_t span = counts[c] * esize(dts[c]);
            /* the sources carry the whole stream; dst s gets segment s only */
            long bad = 0, nwin = 0;
            stub_take_record(&bad, wlo, whi, MAXWIN, &nwin);
            int64_t bounds[PTORED_MAX_RANKS + 1];
            ptored_ring_bounds(counts[c], ns[c], dts[c], bounds);
            for (int k = 0; k < ns[c]; ++k) {
                const uintptr_t d0 = bufs[ns[c] + k];
                const uintptr_t lo = d0 + (uintptr_t)(bounds[k] * esize(dts[c]));
                const uintptr_t hi = d0 + (uintptr_t)(bounds[k + 1] * esize(dts[c]));
                if (!covered(nwin, d0, d0 + (uintptr_t)span, lo, hi)) {
                    printf("FAIL %s: segment %d not covered in its dst\n", label, k);
                    ++failures;
                }
                if (k + 1 < ns[c] && covered(nwin, d0, d0 + (uintptr_t)span, hi, hi + 1) &&
                    bounds[k + 1] < counts[c]) {
                    printf("FAIL %s: dst %d addressed past its segment\n", label, k);
                    ++failures;
                }
            }
            /* replay the call for the window and coverage checks */
            ptored_reduce_scatter_ring(s, ns[c], d, counts[c], dts[c], PTORED_SUM, NULL, 0);
            check_record(label, bufs, 2 * ns[c], ns[c], span, 1, span, span, -1);
        }
    }
    /* push-with-add: aligned, odd pitch */
    {
        const char* label = "accumulate n8 bf16 odd pitch";
        uintptr_t bufs[9];
        const void* s[8];
        for (int r = 0; r < 8; ++r) s[r] = (const void*)(bufs[r] = fake(r, 0));
        bufs[8] = fake(8, 2);
        const int st = ptored_accumulate_add(s, 8, (void*)bufs[8], 4096, 8192, 8193, 4096, 8191,
                                             PTORED_BF16, NULL, 0);
        if (st != PTORED_OK) {
            printf("FAIL %s: status %d\n", label, st);
            ++failures;
        }
        check_record(label, bufs, 9, 9, (4095LL * 8193 + 8191) * 2, 4096, 8193 * 2, 8191 * 2,
                     -1);
    }
    /* rejected calls launch nothing */
    {
        const void* s[3] = {(const void*)fake(0, 0), (const void*)fake(1, 0), NULL};
        expect_status("null source", ptored_treduce(s, 3, 0, (void*)fake(3, 0), 4, 4, 4, 4, 4,
                                                    PTORED_F32, PTORED_SUM, 0),
                      PTORED_ERR_INVALID_ARG);
        expect_status("root out of range", ptored_treduce(s, 2, 2, (void*)fake(3, 0), 4, 4, 4, 4,
                                                          4, PTORED_F32, PTORED_SUM, 0),
                      PTORED_ERR_INVALID_ARG);
        expect_status("partial overlap", ptored_treduce(s, 2, 0, (void*)(fake(0, 0) + 4), 4, 4, 4,
                                                        4, 4, PTORED_F32, PTORED_SUM, 0),
                      PTORED_ERR_OVERLAP);
        expect_status("unknown op", ptored_treduce(s, 2, 0, (void*)fake(3, 0), 4, 4, 4, 4, 4,
                                                   PTORED_F32, 9, 0),
                      PTORED_ERR_UNSUPPORTED);
        expect_status("extent overflow", ptored_treduce(s, 2, 0, (void*)fake(3, 0),
                                                        (int64_t)1 << 40, 1 << 30, 1 << 30, 1, 1,
                                                        PTORED_F32, PTORED_SUM, 0),
                      PTORED_ERR_INVALID_ARG);
        int64_t bounds[5];
        expect_status("ring bounds negative count", ptored_ring_bounds(-1, 4, PTORED_F32, bounds),
                      PTORED_ERR_INVALID_ARG);
    }
    if (failures) {
        printf("%d failure(s)\n", failures);
        return 1;
    }
    printf("host launches ok\n");
    return 0;
}
