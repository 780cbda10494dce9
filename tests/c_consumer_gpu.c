/* A plain C11 program using the library the way a C caller would: device
 * buffers from hipMalloc, the C ABI, a HIP stream, no torch anywhere in the
 * process.  Each call is checked byte for byte (NaN by NaN-ness) against the
 * CPU oracle, linked here as a C library.  Built and run by
 * tests/test_c_consumer_gpu.py; prints the case before every GPU step. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ptored.h"

/* the oracle (oracle/treduce_oracle.c) */
int oracle_treduce(const void* const* srcs, int nranks, int root, void* dst, int64_t rows,
                   int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols, int dtype,
                   int op);
int oracle_allreduce_inplace(void* const* bufs, int nranks, int root, void* scratch,
                             int64_t rows, int64_t cols, int64_t ld, int64_t valid_rows,
                             int64_t valid_cols, int dtype, int op);
int oracle_reduce_scatter_ring(const void* const* srcs, int nranks, void* const* dsts,
                               int64_t count, int dtype, int op);
int oracle_accumulate_add(const void* const* srcs, int nranks, void* dst, int64_t rows,
                          int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols,
                          int dtype, double* exact, double* absum);
void oracle_combine_bits(int dtype, int op, const uint32_t* a, const uint32_t* b, uint32_t* out,
                         int64_t n);

#define MAXN 16
#define PAD 64 /* bytes before and after every device buffer */

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            printf("HIP error %d at line %d\n", (int)e_, __LINE__);            \
            exit(2);                                                           \
        }                                                                      \
    } while (0)

static uint64_t rng_state;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int esize(int dtype) { return (dtype == PTORED_BF16 || dtype == PTORED_F16) ? 2 : 4; }

/* Finite values with a few zeros: exponents near 1 so products of 16 stay
 * mostly in range; i32 takes any bits. */
static void fill(int dtype, unsigned char* p, int64_t n) {
    for (int64_t k = 0; k < n; ++k) {
        uint64_t r = next_u64();
        uint32_t v;
        if (dtype == PTORED_I32) {
            v = (uint32_t)r;
        } else if (dtype == PTORED_F16) {
            uint32_t exp = 9u + (uint32_t)((r >> 16) % 13u);
            v = ((uint32_t)(r >> 40) & 0x8000u) | (exp << 10) | ((uint32_t)r & 0x3FFu);
        } else {
            uint32_t exp = 119u + (uint32_t)((r >> 24) % 17u);
            v = ((uint32_t)(r >> 40) & 0x80000000u) | (exp << 23) | ((uint32_t)r & 0x7FFFFFu);
            if (dtype == PTORED_BF16) v >>= 16;
        }
        if ((r >> 58) == 0) v &= (dtype == PTORED_F32 || dtype == PTORED_I32) ? 0x80000000u
                                                                              : 0x8000u;
        memcpy(p + k * esize(dtype), &v, (size_t)esize(dtype));
    }
}

static int is_nan(int dtype, uint32_t v) {
    switch (dtype) {
    case PTORED_F32: return (v & 0x7F800000u) == 0x7F800000u && (v & 0x7FFFFFu);
    case PTORED_BF16: return (v & 0x7F80u) == 0x7F80u && (v & 0x7Fu);
    case PTORED_F16: return (v & 0x7C00u) == 0x7C00u && (v & 0x3FFu);
    default: return 0;
    }
}

/* Byte-for-byte equality of two buffers, NaN matched by NaN-ness. */
static int same(int dtype, const unsigned char* got, const unsigned char* want, int64_t bytes,
                const char* what) {
    const int es = esize(dtype);
    for (int64_t b = 0; b < bytes; b += es) {
        uint32_t g = 0, w = 0;
        memcpy(&g, got + b, (size_t)es);
        memcpy(&w, want + b, (size_t)es);
        if (g != w && !(is_nan(dtype, g) && is_nan(dtype, w))) {
            printf("MISMATCH %s at byte %lld: got %08x want %08x\n", what, (long long)b, g, w);
            return 0;
        }
    }
    return 1;
}

typedef struct {
    unsigned char* base; /* hipMalloc'd, PAD guard bytes on each side */
    unsigned char* p;    /* base + PAD + lead */
} dbuf;

static dbuf dalloc(int64_t bytes, int lead) {
    dbuf d;
    HIP_OK(hipMalloc((void**)&d.base, (size_t)(bytes + 2 * PAD)));
    HIP_OK(hipMemset(d.base, 0xA5, (size_t)(bytes + 2 * PAD)));
    d.p = d.base + PAD + lead;
    return d;
}

static int guards_ok(dbuf d, int64_t bytes, int lead) {
    unsigned char g[2 * PAD + 16];
    HIP_OK(hipMemcpy(g, d.base, PAD + lead, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g + PAD + lead, d.p + bytes, PAD - lead, hipMemcpyDeviceToHost));
    for (int k = 0; k < 2 * PAD; ++k)
        if (g[k] != 0xA5) return 0;
    return 1;
}

typedef struct {
    int64_t rows, cols, ld, vr, vc;
} shape;

static const shape SHAPES[] = {
    {37, 1000, 1024, 35, 997}, /* 2-D: ragged row ends, a short last band */
    {1, 70001, 70001, 1, 70001}, /* one contiguous span with a ragged tail */
};

static int cases_run = 0;

/* One treduce call; offs[r] = byte offset of source r (dst at offs[n]). */
static int check_treduce(int dtype, int op, int n, int root, shape s, const int* offs,
                         hipStream_t st) {
    const int es = esize(dtype);
    const int64_t size = (s.rows - 1) * s.ld + s.cols, bytes = size * es;
    unsigned char* h[MAXN];
    const void* hp[MAXN];
    const void* dp[MAXN];
    dbuf d[MAXN + 1];
    for (int r = 0; r < n; ++r) {
        h[r] = malloc((size_t)bytes);
        fill(dtype, h[r], size);
        hp[r] = h[r];
        d[r] = dalloc(bytes, offs[r]);
        HIP_OK(hipMemcpy(d[r].p, h[r], (size_t)bytes, hipMemcpyHostToDevice));
        dp[r] = d[r].p;
    }
    d[n] = dalloc(bytes, offs[n]);
    HIP_OK(hipMemset(d[n].p, 0xFF, (size_t)bytes));
    unsigned char* want = malloc((size_t)bytes);
    unsigned char* got = malloc((size_t)bytes);
    memset(want, 0xFF, (size_t)bytes);
    printf("treduce dtype %d op %d n %d root %d shape %lldx%lld lead %d\n", dtype, op, n, root,
           (long long)s.rows, (long long)s.cols, offs[0]);
    fflush(stdout);
    int st_ = ptored_treduce(dp, n, root, d[n].p, s.rows, s.cols, s.ld, s.vr, s.vc, dtype, op,
                             st);
    if (st_ != PTORED_OK) {
        printf("status %s\n", ptored_status_string(st_));
        return 0;
    }
    HIP_OK(hipStreamSynchronize(st));
    HIP_OK(hipMemcpy(got, d[n].p, (size_t)bytes, hipMemcpyDeviceToHost));
    if (oracle_treduce(hp, n, root, want, s.rows, s.cols, s.ld, s.vr, s.vc, dtype, op) != 0)
        return 0;
    int ok = same(dtype, got, want, bytes, "treduce") && guards_ok(d[n], bytes, offs[n]);
    for (int r = 0; r < n && ok; ++r) { /* sources unchanged */
        HIP_OK(hipMemcpy(got, d[r].p, (size_t)bytes, hipMemcpyDeviceToHost));
        ok = memcmp(got, h[r], (size_t)bytes) == 0;
    }
    for (int r = 0; r <= n; ++r) HIP_OK(hipFree(d[r].base));
    for (int r = 0; r < n; ++r) free(h[r]);
    free(want);
    free(got);
    ++cases_run;
    return ok;
}

static int check_allreduce(int dtype, int op, int n, int root, shape s, hipStream_t st) {
    const int es = esize(dtype);
    const int64_t size = (s.rows - 1) * s.ld + s.cols, bytes = size * es;
    unsigned char* h[MAXN];
    void* hp[MAXN];
    void* dp[MAXN];
    dbuf d[MAXN];
    for (int r = 0; r < n; ++r) {
        h[r] = malloc((size_t)bytes);
        fill(dtype, h[r], size);
        hp[r] = h[r];
        d[r] = dalloc(bytes, 0);
        HIP_OK(hipMemcpy(d[r].p, h[r], (size_t)bytes, hipMemcpyHostToDevice));
        dp[r] = d[r].p;
    }
    unsigned char* scratch = malloc((size_t)bytes);
    unsigned char* got = malloc((size_t)bytes);
    printf("allreduce dtype %d op %d n %d root %d shape %lldx%lld\n", dtype, op, n, root,
           (long long)s.rows, (long long)s.cols);
    fflush(stdout);
    int st_ = ptored_allreduce(dp, n, root, s.rows, s.cols, s.ld, s.vr, s.vc, dtype, op, NULL,
                               st);
    if (st_ != PTORED_OK) {
        printf("status %s\n", ptored_status_string(st_));
        return 0;
    }
    HIP_OK(hipStreamSynchronize(st));
    if (oracle_allreduce_inplace(hp, n, root, scratch, s.rows, s.cols, s.ld, s.vr, s.vc, dtype,
                                 op) != 0)
        return 0;
    int ok = 1;
    for (int r = 0; r < n && ok; ++r) {
        HIP_OK(hipMemcpy(got, d[r].p, (size_t)bytes, hipMemcpyDeviceToHost));
        ok = same(dtype, got, h[r], bytes, "allreduce") && guards_ok(d[r], bytes, 0);
    }
    for (int r = 0; r < n; ++r) {
        HIP_OK(hipFree(d[r].base));
        free(h[r]);
    }
    free(scratch);
    free(got);
    ++cases_run;
    return ok;
}

static int check_ring(int dtype, int op, int n, int64_t count, hipStream_t st) {
    const int es = esize(dtype);
    const int64_t bytes = count * es;
    unsigned char *h[MAXN], *w[MAXN];
    const void *hp[MAXN], *dp[MAXN];
    void *wp[MAXN], *ddp[MAXN];
    dbuf d[MAXN], o[MAXN];
    for (int r = 0; r < n; ++r) {
        h[r] = malloc((size_t)bytes);
        fill(dtype, h[r], count);
        hp[r] = h[r];
        w[r] = malloc((size_t)bytes);
        memset(w[r], 0xFF, (size_t)bytes);
        wp[r] = w[r];
        d[r] = dalloc(bytes, 0);
        HIP_OK(hipMemcpy(d[r].p, h[r], (size_t)bytes, hipMemcpyHostToDevice));
        dp[r] = d[r].p;
        o[r] = dalloc(bytes, 0);
        HIP_OK(hipMemset(o[r].p, 0xFF, (size_t)bytes));
        ddp[r] = o[r].p;
    }
    unsigned char* got = malloc((size_t)bytes);
    printf("ring dtype %d op %d n %d count %lld\n", dtype, op, n, (long long)count);
    fflush(stdout);
    int st_ = ptored_reduce_scatter_ring(dp, n, ddp, count, dtype, op, NULL, st);
    if (st_ != PTORED_OK) {
        printf("status %s\n", ptored_status_string(st_));
        return 0;
    }
    HIP_OK(hipStreamSynchronize(st));
    if (oracle_reduce_scatter_ring(hp, n, wp, count, dtype, op) != 0) return 0;
    int ok = 1;
    for (int r = 0; r < n && ok; ++r) {
        HIP_OK(hipMemcpy(got, o[r].p, (size_t)bytes, hipMemcpyDeviceToHost));
        ok = same(dtype, got, w[r], bytes, "ring") && guards_ok(o[r], bytes, 0);
    }
    for (int r = 0; r < n; ++r) {
        HIP_OK(hipFree(d[r].base));
        HIP_OK(hipFree(o[r].base));
        free(h[r]);
        free(w[r]);
    }
    free(got);
    ++cases_run;
    return ok;
}

/* push-with-add.  Default (the call's sources folded first): with no other
 * push landing meanwhile, dst becomes dst + fold(srcs) rounded once -- the
 * oracle's fold with root 0, then its one combine step -- byte for byte.
 * Per rank (i32 only here): wrapping integer sums, exact in any order. */
static int check_accumulate(int dtype, int n, shape s, int per_rank, hipStream_t st) {
    const int es = esize(dtype);
    const int64_t size = (s.rows - 1) * s.ld + s.cols, bytes = size * es;
    unsigned char* h[MAXN];
    const void *hp[MAXN], *dp[MAXN];
    dbuf d[MAXN];
    for (int r = 0; r < n; ++r) {
        h[r] = malloc((size_t)bytes);
        fill(dtype, h[r], size);
        hp[r] = h[r];
        d[r] = dalloc(bytes, 0);
        HIP_OK(hipMemcpy(d[r].p, h[r], (size_t)bytes, hipMemcpyHostToDevice));
        dp[r] = d[r].p;
    }
    unsigned char* want = malloc((size_t)bytes);
    unsigned char* got = malloc((size_t)bytes);
    fill(dtype, want, size);
    dbuf dd = dalloc(bytes, 0);
    HIP_OK(hipMemcpy(dd.p, want, (size_t)bytes, hipMemcpyHostToDevice));
    printf("accumulate_add dtype %d %s n %d shape %lldx%lld\n", dtype,
           per_rank ? "per rank" : "folded", n, (long long)s.rows, (long long)s.cols);
    fflush(stdout);
    const ptored_tuning t = {per_rank ? PTORED_ACC_PER_RANK : 0u, 0, 0};
    int st_ = ptored_accumulate_add(dp, n, dd.p, s.rows, s.cols, s.ld, s.vr, s.vc, dtype, &t, st);
    if (st_ != PTORED_OK) {
        printf("status %s\n", ptored_status_string(st_));
        return 0;
    }
    HIP_OK(hipStreamSynchronize(st));
    if (per_rank) {
        double* ex = malloc(sizeof(double) * (size_t)(s.vr * s.vc));
        double* ab = malloc(sizeof(double) * (size_t)(s.vr * s.vc));
        if (oracle_accumulate_add(hp, n, want, s.rows, s.cols, s.ld, s.vr, s.vc, dtype, ex, ab) !=
            0)
            return 0;
        free(ex);
        free(ab);
    } else {
        unsigned char* fold = calloc(1, (size_t)bytes);
        if (oracle_treduce(hp, n, 0, fold, s.rows, s.cols, s.ld, s.vr, s.vc, dtype, PTORED_SUM) !=
            0)
            return 0;
        const int64_t cnt = s.vr * s.vc;
        uint32_t* a = calloc((size_t)cnt, sizeof(uint32_t));
        uint32_t* b = calloc((size_t)cnt, sizeof(uint32_t));
        uint32_t* o = calloc((size_t)cnt, sizeof(uint32_t));
        for (int64_t i = 0, k = 0; i < s.vr; ++i)
            for (int64_t j = 0; j < s.vc; ++j, ++k) {
                memcpy(&a[k], want + (i * s.ld + j) * es, (size_t)es);
                memcpy(&b[k], fold + (i * s.ld + j) * es, (size_t)es);
            }
        oracle_combine_bits(dtype, PTORED_SUM, a, b, o, cnt);
        for (int64_t i = 0, k = 0; i < s.vr; ++i)
            for (int64_t j = 0; j < s.vc; ++j, ++k)
                memcpy(want + (i * s.ld + j) * es, &o[k], (size_t)es);
        free(fold);
        free(a);
        free(b);
        free(o);
    }
    HIP_OK(hipMemcpy(got, dd.p, (size_t)bytes, hipMemcpyDeviceToHost));
    int ok = same(dtype, got, want, bytes, "accumulate_add") && guards_ok(dd, bytes, 0);
    for (int r = 0; r < n; ++r) {
        HIP_OK(hipFree(d[r].base));
        free(h[r]);
    }
    HIP_OK(hipFree(dd.base));
    free(want);
    free(got);
    ++cases_run;
    return ok;
}

int main(void) {
    rng_state = 0x5EEDC0DEull;
    int ndev = 0;
    HIP_OK(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        printf("no GPU\n");
        return 3;
    }
    HIP_OK(hipSetDevice(0));
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    const int dts[4] = {PTORED_F32, PTORED_BF16, PTORED_F16, PTORED_I32};
    for (int t = 0; t < 4; ++t) {
        const int dt = dts[t], es = esize(dt);
        for (int op = PTORED_SUM; op <= PTORED_PROD; ++op) {
            for (int k = 0; k < 2; ++k) {
                const int n = k ? 16 : 3, root = k ? 11 : 1;
                int offs[MAXN + 1] = {0};
                if (!check_treduce(dt, op, n, root, SHAPES[k], offs, st)) return 1;
            }
        }
        /* every buffer at one odd offset (the head path), then each at its own
         * offset (element-wise) */
        int offs[MAXN + 1];
        for (int r = 0; r <= MAXN; ++r) offs[r] = 3 * es;
        if (!check_treduce(dt, PTORED_SUM, 5, 2, SHAPES[0], offs, st)) return 1;
        for (int r = 0; r <= MAXN; ++r) offs[r] = (r % 8) * es;
        if (!check_treduce(dt, PTORED_MAX, 5, 0, SHAPES[1], offs, st)) return 1;
        if (!check_allreduce(dt, PTORED_SUM, 8, 3, SHAPES[0], st)) return 1;
        if (!check_ring(dt, PTORED_MIN, 6, 100003, st)) return 1;
        for (int k = 0; k < 2; ++k)
            if (!check_accumulate(dt, 7, SHAPES[k], 0, st)) return 1;
    }
    if (!check_accumulate(PTORED_I32, 7, SHAPES[0], 1, st)) return 1;
    HIP_OK(hipStreamDestroy(st));
    printf("c consumer ok: %d calls\n", cases_run);
    return 0;
}
