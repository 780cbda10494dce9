/*
 * treduce_oracle.c -- plain, slow CPU oracle for the N-way TREDUCE reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU path is compared against.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call it; the product library
 * never links, loads or calls anything here.  It shares no code, header,
 * table or constant with the GPU path.
 *
 * Sources (cited by title and section):
 *   [TREDUCE]  "CANN PTO-ISA TREDUCE instruction explained: principle,
 *              constraints and practice of multi-NPU cross-card Reduce"
 *              (lpnh.cn news article on pto-isa).
 *   [N6]       "Distributed Operators (N6)", PyPTO developer documentation.
 *
 * What is computed ([TREDUCE] §1.1 math definition, §4.3 simple-path loop):
 *   for every (i, j) in the valid rectangle [0,valid_rows) x [0,valid_cols):
 *       acc = src[root][i, j]
 *       for r = 0 .. N-1, skipping r == root:  acc = acc (+) src[r][i, j]
 *       dst[i, j] = acc
 *   Element (i, j) of every buffer sits at element offset i*ld + j.
 *   Nothing outside the valid rectangle is read from dst or written to it.
 *   N == 1 copies the root's bits unchanged ([TREDUCE] §4.3, single-rank case).
 *   An empty rectangle writes nothing ([TREDUCE] §4.1 empty short-circuit).
 *
 * The combine (+) ([TREDUCE] §1.3 ReduceTiles: TADD / TMAX / TMIN into the
 * accumulator tile, which has the element type; [N6] ReduceOp enum adds Prod):
 *   Sum, Prod on f32 / bf16 / f16: the exact sum or product of the two operands
 *     rounded once to the element type, round-to-nearest-ties-to-even,
 *     subnormals kept, overflow to +-Inf.  The exact value is formed in double:
 *     the product of two such values is exact in double; the sum is rounded
 *     once to double, and rounding that to the narrower type gives the same
 *     result as rounding the exact sum (53 >= 2p+2 for p = 24, 11 and 8).
 *     A NaN result is the quiet NaN with the sign of the double result.
 *   Sum, Prod on i32: two's-complement wrap-around modulo 2^32.
 *   Max, Min on i32: signed comparison.
 *   Max, Min on floats: if either operand is a NaN the result is the quiet
 *     NaN; otherwise the extremum under IEEE-754 totalOrder restricted to
 *     non-NaN values, which orders -0 below +0.
 *
 * Built with gcc -O2 -ffp-contract=off and without fast-math, on x86-64 where
 * float and double arithmetic are IEEE binary32 / binary64.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* dtype and op codes of the C ABI, restated here so this file stands alone. */
enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2, OR_I32 = 3 };
enum { OR_SUM = 0, OR_MAX = 1, OR_MIN = 2, OR_PROD = 3 };
enum { OR_MAX_RANKS = 1024 };

/* ------------------------------------------------------------------------ */
/* binary16 and bfloat16 <-> double, written from the IEEE-754 formats.      */
/* ------------------------------------------------------------------------ */

/* Decode a p-bit-significand format with `ebits` exponent bits and `mbits`
 * stored mantissa bits; bias = 2^(ebits-1) - 1.  Exact in double for both
 * formats used here. */
static double decode_small(uint32_t bits, int ebits, int mbits) {
    const uint32_t sign = (bits >> (ebits + mbits)) & 1u;
    const uint32_t e = (bits >> mbits) & ((1u << ebits) - 1u);
    const uint32_t m = bits & ((1u << mbits) - 1u);
    const int bias = (1 << (ebits - 1)) - 1;
    double v;
    if (e == (1u << ebits) - 1u) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        /* subnormal: m * 2^(1 - bias - mbits) */
        v = ldexp((double)m, 1 - bias - mbits);
    } else {
        v = ldexp((double)((1u << mbits) | m), (int)e - bias - mbits);
    }
    return sign ? -v : v;
}

/* Round a double to the nearest value of the small format, ties to even.
 * The significand is scaled to an integer grid by an exact power of two and
 * rounded with nearbyint(), which rounds to nearest-even in the default
 * floating-point environment. */
static uint32_t encode_small(double x, int ebits, int mbits) {
    const int bias = (1 << (ebits - 1)) - 1;
    const uint32_t emax_field = (1u << ebits) - 1u; /* all-ones exponent */
    const uint32_t sign = signbit(x) ? 1u : 0u;
    const uint32_t sbit = sign << (ebits + mbits);
    if (isnan(x)) {
        return sbit | (emax_field << mbits) | (1u << (mbits - 1));
    }
    double a = fabs(x);
    if (isinf(a)) {
        return sbit | (emax_field << mbits);
    }
    const int emin = 1 - bias; /* exponent of the smallest normal */
    int E;
    frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1; /* a in [2^e, 2^(e+1)) */
    if (a == 0.0 || e < emin) {
        /* subnormal range: grid spacing 2^(emin - mbits) */
        double q = nearbyint(ldexp(a, mbits - emin));
        /* q == 2^mbits lands exactly on the smallest normal: the encoding
         * (exponent field 1, mantissa 0) equals the integer q. */
        return sbit | (uint32_t)q;
    }
    double q = nearbyint(ldexp(a, mbits - e)); /* in [2^mbits, 2^(mbits+1)] */
    if (q == ldexp(1.0, mbits + 1)) {
        q = ldexp(1.0, mbits);
        e += 1;
    }
    if (e > bias) { /* beyond the largest finite exponent */
        return sbit | (emax_field << mbits);
    }
    const uint32_t field = (uint32_t)(e + bias);
    return sbit | (field << mbits) | ((uint32_t)q - (1u << mbits));
}

static double f16_to_double(uint16_t h) { return decode_small(h, 5, 10); }
static double bf16_to_double(uint16_t b) { return decode_small(b, 8, 7); }
static uint16_t double_to_f16(double x) { return (uint16_t)encode_small(x, 5, 10); }
static uint16_t double_to_bf16(double x) { return (uint16_t)encode_small(x, 8, 7); }

static double f32_to_double(uint32_t bits) {
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}
static uint32_t double_to_f32(double x) {
    /* The C conversion rounds to nearest-even (SSE2, default environment). */
    float f = (float)x;
    uint32_t bits;
    if (isnan(x)) {
        return (signbit(x) ? 0x80000000u : 0u) | 0x7FC00000u;
    }
    memcpy(&bits, &f, 4);
    return bits;
}

/* element bits <-> double for the three float types */
static double to_double(int dtype, uint32_t bits) {
    switch (dtype) {
    case OR_F32: return f32_to_double(bits);
    case OR_BF16: return bf16_to_double((uint16_t)bits);
    default: return f16_to_double((uint16_t)bits);
    }
}
static uint32_t from_double(int dtype, double x) {
    switch (dtype) {
    case OR_F32: return double_to_f32(x);
    case OR_BF16: return double_to_bf16(x);
    default: return double_to_f16(x);
    }
}
static uint32_t quiet_nan(int dtype) {
    switch (dtype) {
    case OR_F32: return 0x7FC00000u;
    case OR_BF16: return 0x7FC0u;
    default: return 0x7E00u;
    }
}

/* ------------------------------------------------------------------------ */
/* The combine step  acc = acc (+) x  on raw element bits.                   */
/* ------------------------------------------------------------------------ */

/* -0 < +0 < ... : for two non-NaN doubles, is a below b in totalOrder? */
static int total_less(double a, double b) {
    if (a < b) return 1;
    if (a > b) return 0;
    return signbit(a) && !signbit(b); /* equal: only -0 vs +0 differ */
}

static uint32_t combine(int dtype, int op, uint32_t acc, uint32_t x) {
    if (dtype == OR_I32) {
        const int32_t a = (int32_t)acc, b = (int32_t)x;
        switch (op) {
        case OR_SUM: return acc + x;          /* wraps modulo 2^32 */
        case OR_PROD: return acc * x;         /* wraps modulo 2^32 */
        case OR_MAX: return (uint32_t)(b > a ? b : a);
        default: return (uint32_t)(b < a ? b : a);
        }
    }
    const double a = to_double(dtype, acc), b = to_double(dtype, x);
    switch (op) {
    case OR_SUM: return from_double(dtype, a + b);
    case OR_PROD: return from_double(dtype, a * b);
    case OR_MAX:
        if (isnan(a) || isnan(b)) return quiet_nan(dtype);
        return total_less(a, b) ? x : acc;
    default:
        if (isnan(a) || isnan(b)) return quiet_nan(dtype);
        return total_less(b, a) ? x : acc;
    }
}

static int esize_of(int dtype) { return (dtype == OR_F32 || dtype == OR_I32) ? 4 : 2; }

static uint32_t load_bits(const void* base, int64_t idx, int es) {
    if (es == 4) {
        uint32_t v;
        memcpy(&v, (const char*)base + idx * 4, 4);
        return v;
    }
    uint16_t v;
    memcpy(&v, (const char*)base + idx * 2, 2);
    return v;
}
static void store_bits(void* base, int64_t idx, int es, uint32_t v) {
    if (es == 4) {
        memcpy((char*)base + idx * 4, &v, 4);
    } else {
        uint16_t h = (uint16_t)v;
        memcpy((char*)base + idx * 2, &h, 2);
    }
}

/* Argument rules of the operation ([TREDUCE] §3.3: group size > 0, root in
 * range; shape rules of a valid rectangle inside a rows x cols view). */
static int check_args(const void* const* srcs, int nranks, int root, const void* dst,
                      int64_t rows, int64_t cols, int64_t ld, int64_t valid_rows,
                      int64_t valid_cols, int dtype, int op) {
    if (nranks < 1 || nranks > OR_MAX_RANKS) return -1;
    if (root < 0 || root >= nranks) return -1;
    if (!srcs || !dst) return -1;
    for (int r = 0; r < nranks; ++r)
        if (!srcs[r]) return -1;
    if (rows < 0 || cols < 0 || ld < 0 || valid_rows < 0 || valid_cols < 0) return -1;
    if (cols > ld || valid_rows > rows || valid_cols > cols) return -1;
    if (dtype < OR_F32 || dtype > OR_I32) return -2;
    if (op < OR_SUM || op > OR_PROD) return -2;
    return 0;
}

/* The reduction itself, in the order of [TREDUCE] §4.3. */
int oracle_treduce(const void* const* srcs, int nranks, int root, void* dst, int64_t rows,
                   int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols,
                   int dtype, int op) {
    int rc = check_args(srcs, nranks, root, dst, rows, cols, ld, valid_rows, valid_cols, dtype,
                        op);
    if (rc) return rc;
    const int es = esize_of(dtype);
    for (int64_t i = 0; i < valid_rows; ++i) {
        for (int64_t j = 0; j < valid_cols; ++j) {
            const int64_t idx = i * ld + j;
            uint32_t acc = load_bits(srcs[root], idx, es);
            for (int r = 0; r < nranks; ++r) {
                if (r == root) continue;
                acc = combine(dtype, op, acc, load_bits(srcs[r], idx, es));
            }
            store_bits(dst, idx, es, acc);
        }
    }
    return 0;
}

/* In-place allreduce on one device ([N6] pld.tensor.allreduce: every rank's
 * slice is reduced in place, so after the call every slice holds the same
 * reduced value).  Computes the reduction of [TREDUCE] §4.3 into `scratch`
 * (a caller buffer of the same layout) and then writes it to all N buffers
 * over the valid rectangle. */
int oracle_allreduce_inplace(void* const* bufs, int nranks, int root, void* scratch, int64_t rows,
                             int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols,
                             int dtype, int op) {
    int rc = oracle_treduce((const void* const*)bufs, nranks, root, scratch, rows, cols, ld,
                            valid_rows, valid_cols, dtype, op);
    if (rc) return rc;
    const int es = esize_of(dtype);
    for (int r = 0; r < nranks; ++r)
        for (int64_t i = 0; i < valid_rows; ++i)
            for (int64_t j = 0; j < valid_cols; ++j)
                store_bits(bufs[r], i * ld + j, es, load_bits(scratch, i * ld + j, es));
    return 0;
}

/* Segment boundaries of the ring schedule ([N6] pld.tensor.allreduce, ring
 * mode): a stream of `count` elements is cut into `nranks` segments at the
 * balanced boundaries floor(i * count / nranks); for 2-byte elements every
 * interior boundary is then rounded up to a multiple of 16 elements (32
 * bytes) and capped at `count`, so short streams may have empty segments.
 * bounds[0] = 0, bounds[nranks] = count. */
int oracle_ring_bounds(int64_t count, int nranks, int dtype, int64_t* bounds) {
    if (count < 0 || nranks < 1 || nranks > OR_MAX_RANKS || !bounds) return -1;
    if (dtype < OR_F32 || dtype > OR_I32) return -2;
    bounds[0] = 0;
    for (int i = 1; i < nranks; ++i) {
        int64_t b = (int64_t)((__int128)i * count / nranks);
        if (esize_of(dtype) == 2) {
            b = (b + 15) / 16 * 16;
            if (b > count) b = count;
        }
        bounds[i] = b;
    }
    bounds[nranks] = count;
    return 0;
}

/* The reduce-scatter share of the ring schedule on one device: segment s of
 * the stream is reduced over all ranks and written to dsts[s] (same element
 * positions).  The partial result of a ring reduce-scatter for segment s
 * starts at rank s+1 and travels round the ring, each rank folding in its own
 * value, until it reaches rank s, which folds its value last: the fold order
 * is s+1, s+2, ..., s+N-1, s (ranks mod N). */
int oracle_reduce_scatter_ring(const void* const* srcs, int nranks, void* const* dsts,
                               int64_t count, int dtype, int op) {
    if (nranks < 1 || nranks > OR_MAX_RANKS || !srcs || !dsts || count < 0) return -1;
    if (dtype < OR_F32 || dtype > OR_I32 || op < OR_SUM || op > OR_PROD) return -2;
    int64_t bounds[OR_MAX_RANKS + 1];
    int rc = oracle_ring_bounds(count, nranks, dtype, bounds);
    if (rc) return rc;
    const int es = esize_of(dtype);
    for (int s = 0; s < nranks; ++s) {
        for (int64_t j = bounds[s]; j < bounds[s + 1]; ++j) {
            uint32_t acc = load_bits(srcs[(s + 1) % nranks], j, es);
            for (int k = 2; k <= nranks; ++k)
                acc = combine(dtype, op, acc, load_bits(srcs[(s + k) % nranks], j, es));
            store_bits(dsts[s], j, es, acc);
        }
    }
    return 0;
}

/* Push-with-add ([N6] pld.tensor.put / remote_store with atomic = kAdd: the
 * pushed data is added into the peer's slice).  With N ranks pushing into
 * one slice, dst[i, j] becomes dst[i, j] + src_0[i, j] + ... + src_{N-1}[i, j]
 * with the additions in an unspecified order.  This reference applies them in
 * rank order, each addition rounded to the element type (i32 wraps), and
 * also returns, for the float types, the exact sum (in `exact`, doubles, one
 * per element of the valid rectangle, row-major) and the sum of absolute
 * values (in `absum`), from which a test bounds any other order's result. */
int oracle_accumulate_add(const void* const* srcs, int nranks, void* dst, int64_t rows,
                          int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols,
                          int dtype, double* exact, double* absum) {
    int rc = check_args(srcs, nranks, 0, dst, rows, cols, ld, valid_rows, valid_cols, dtype,
                        OR_SUM);
    if (rc) return rc;
    const int es = esize_of(dtype);
    int64_t k = 0;
    for (int64_t i = 0; i < valid_rows; ++i) {
        for (int64_t j = 0; j < valid_cols; ++j, ++k) {
            const int64_t idx = i * ld + j;
            uint32_t acc = load_bits(dst, idx, es);
            double ex = 0.0, ab = 0.0;
            if (dtype != OR_I32) {
                ex = to_double(dtype, acc);
                ab = fabs(ex);
            }
            for (int r = 0; r < nranks; ++r) {
                const uint32_t x = load_bits(srcs[r], idx, es);
                acc = combine(dtype, OR_SUM, acc, x);
                if (dtype != OR_I32) {
                    /* summed in double: its own error, at most (N+1) * 2^-53 of
                     * the absolute sum, is far below any element rounding */
                    ex += to_double(dtype, x);
                    ab += fabs(to_double(dtype, x));
                }
            }
            store_bits(dst, idx, es, acc);
            if (exact) exact[k] = ex;
            if (absum) absum[k] = ab;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Exported single steps, so tests can pin the arithmetic on its own.        */
/* ------------------------------------------------------------------------ */

/* out[k] = combine(a[k], b[k]) for k < n, on raw bits (u32 holding the element). */
void oracle_combine_bits(int dtype, int op, const uint32_t* a, const uint32_t* b, uint32_t* out,
                         int64_t n) {
    for (int64_t k = 0; k < n; ++k) out[k] = combine(dtype, op, a[k], b[k]);
}

/* out[k] = nearest element of `dtype` to x[k], ties to even (float types). */
void oracle_round_from_double(int dtype, const double* x, uint32_t* out, int64_t n) {
    for (int64_t k = 0; k < n; ++k) out[k] = from_double(dtype, x[k]);
}

/* out[k] = exact value of the element bits b[k] (float types). */
void oracle_to_double(int dtype, const uint32_t* b, double* out, int64_t n) {
    for (int64_t k = 0; k < n; ++k) out[k] = to_double(dtype, b[k]);
}

int oracle_max_ranks(void) { return OR_MAX_RANKS; }
