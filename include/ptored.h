/*
 * ptored.h -- C ABI of the N-way cross-rank reduction on one MI355X (gfx950).
 *
 * Sources (cited by title and section):
 *   [TREDUCE]  "CANN PTO-ISA TREDUCE instruction explained: principle,
 *              constraints and practice of multi-NPU cross-card Reduce"
 *              (lpnh.cn news article on pto-isa).
 *   [N6]       "Distributed Operators (N6)", PyPTO developer documentation.
 *
 * The operation ([TREDUCE] §1.1): for every element (i, j) of a valid
 * rectangle, dst[i, j] = src_0[i, j] (+) src_1[i, j] (+) ... (+) src_{N-1}[i, j].
 * The N sources are the N ranks' window slices ([N6] overview); on one GPU
 * they are N separate device buffers.  The fold starts from the root's value
 * and then takes every other rank in ascending order ([TREDUCE] §4.3), and
 * every step rounds to the element type (the accumulator tile has the element
 * type, [TREDUCE] §1.3 and §3.1).
 *
 * Layout shared by every buffer (all sources and dst have the same shape and
 * strides, [TREDUCE] §3.3): row-major, `rows` rows of `ld` elements, of which
 * the first `cols` are the tensor's columns; element (i, j) is at element
 * offset i*ld + j.  The valid rectangle [0, valid_rows) x [0, valid_cols) is
 * anchored at (0, 0) ([N6] pld.tensor.allreduce, valid_shape).  A buffer must
 * hold at least ((rows-1)*ld + cols) elements.
 *
 * All values of the enums are append-only: new values are only ever added at
 * the end, so an integer keeps its meaning ([N6] "ABI enums").
 *
 * All functions are thread-safe.  No function allocates device memory; the
 * library keeps no state besides a per-device cache of the compute-unit count
 * and LDS sizes.
 */
#ifndef PTORED_H
#define PTORED_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PTORED_ABI_VERSION 3
/* Largest number of ranks (source buffers) one call accepts. */
#define PTORED_MAX_RANKS 64
/* Threads in one workgroup of the library's kernels: one 64-wide wave.
 * Informative; the plan's resident-workgroup counts are in these units. */
#define PTORED_WORKGROUP_THREADS 64

/* Element type.  One type for every source and for dst ([TREDUCE] §3.1). */
typedef enum ptored_dtype {
    PTORED_F32 = 0,  /* IEEE binary32 */
    PTORED_BF16 = 1, /* bfloat16 (upper half of a binary32) */
    PTORED_F16 = 2,  /* IEEE binary16 */
    PTORED_I32 = 3   /* two's-complement int32 */
} ptored_dtype;

/* Reduction ([TREDUCE] §1.3 ReduceOp; [N6] ReduceOp enum, same values).
 *   SUM  float: exact sum rounded to the element type (nearest, ties to
 *        even, subnormals kept); i32: wraps modulo 2^32.
 *   MAX / MIN  i32: signed.  float: a NaN operand gives NaN; otherwise the
 *        extremum with -0 ordered below +0 (IEEE-754 maximum / minimum).
 *   PROD float: exact product rounded to the element type; i32: wraps. */
typedef enum ptored_op {
    PTORED_SUM = 0,
    PTORED_MAX = 1,
    PTORED_MIN = 2,
    PTORED_PROD = 3
} ptored_op;

/* Status codes; every function returns one of these (never throws). */
typedef enum ptored_status {
    PTORED_OK = 0,
    PTORED_ERR_INVALID_ARG = -1, /* bad count, root, pointer or shape */
    PTORED_ERR_UNSUPPORTED = -2, /* unknown dtype or op */
    PTORED_ERR_OVERLAP = -3,     /* dst partially overlaps a source */
    PTORED_ERR_HIP = -4          /* the HIP runtime reported an error */
} ptored_status;

/*
 * ptored_treduce -- dst = fold of the N sources over the valid rectangle.
 *
 * srcs        HOST array of `nranks` DEVICE pointers; srcs[r] is rank r's
 *             buffer.  The array is read during the call only and may be
 *             freed when the call returns.
 * nranks      N, 1 <= N <= PTORED_MAX_RANKS ([TREDUCE] §3.3: group size > 0).
 * root        0 <= root < N ([TREDUCE] §3.3).  The fold starts from the
 *             root's value (the root's buffer is the reference, §3.3 and
 *             §4.3); with N == 1 the call is a bitwise copy (§4.3).
 * dst         DEVICE pointer to the output buffer.  Only elements inside the
 *             valid rectangle are written; dst is never read, and every
 *             other byte is left unchanged.  dst may be exactly one of the
 *             sources (in-place, as the allreduce of [N6] does); any other
 *             overlap of dst with a source's span is rejected.
 * rows, cols, ld              buffer shape (elements), cols <= ld.
 * valid_rows, valid_cols      valid rectangle, <= rows and <= cols.  An empty
 *             rectangle returns PTORED_OK and launches nothing ([TREDUCE]
 *             §4.1 empty short-circuit).
 * dtype, op   ptored_dtype and ptored_op values.
 * stream      HIP stream of the current device (0 = null stream).  The call
 *             only enqueues work and returns; it never synchronises.  Every
 *             buffer must stay valid and unmodified until that work is done
 *             ([TREDUCE] §3.2).
 *
 * Errors are checked before any HIP call, in this order: INVALID_ARG (N or
 * root out of range, a null pointer, a negative size, cols > ld,
 * valid_rows > rows, valid_cols > cols, a size whose byte extent overflows),
 * UNSUPPORTED (dtype or op outside the enums), INVALID_ARG (a pointer not
 * aligned to the element size), OVERLAP.  ERR_HIP is returned when the
 * launch fails.  Pointers or row pitches that are not 16-byte aligned are
 * not errors: the 16-byte vector kernels run on any alignment.  When every
 * buffer starts at the same offset within a 16-byte block and the pitch is
 * a multiple of 16 bytes, every access is aligned (each row's bytes before
 * the next 16-byte boundary folded as a head), and buffers that also share
 * their offset within 1 KiB (or a 128-byte line) are walked in aligned 1 KiB
 * runs (or whole lines) whatever that offset.  Buffers at different offsets
 * keep dst aligned the same way and read the sources with unaligned 16-byte
 * loads; a pitch that is not a multiple of 16 bytes numbers each row's
 * slots from the row's start, every access unaligned.  A valid row (or
 * span) that does not reach the 16-byte boundary it starts before, the
 * PTORED_LDS_PINGPONG variant on misaligned data and PTORED_FORCE_ELEMENTWISE
 * take an element-wise kernel (and push-with-add with an odd pitch).
 */
int ptored_treduce(const void* const* srcs, int nranks, int root, void* dst, int64_t rows,
                   int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols,
                   int dtype, int op, hipStream_t stream);

/* Forcing flags of ptored_treduce_ex (for tests and tuning; 0 = automatic). */
#define PTORED_FORCE_ELEMENTWISE 0x1u /* element-wise kernel even when 16-B aligned */
#define PTORED_FORCE_ROWS 0x2u        /* 2-D row walk even for a contiguous region */
#define PTORED_FORCE_RUNTIME_N 0x4u   /* rank-count loop instead of an unrolled N */
#define PTORED_NO_XCD_REMAP 0x8u      /* persistent grid: plain block order, not per-XCD bands */
#define PTORED_ROW_TILES 0x10u        /* 2-D region: tiles of one row's column chunk (the pages'
                                         2-D sliding chunk walk, the default when a row's
                                         slots fill its chunks well) even when they do not */
#define PTORED_LDS_PINGPONG 0x20u     /* stage the sources through a ring of LDS buffers with
                                         direct buffer-to-LDS loads (the pages' ping/pong
                                         tiles) instead of registers; N >= 2, 16-byte data */
#define PTORED_SEGMENT_LAUNCHES 0x40u /* reduce-scatter: one launch per ring segment instead of
                                         one launch over every segment */
#define PTORED_FLAT_WALK 0x100u       /* 2-D region: slots numbered straight through the rows
                                         instead of row tiles */
#define PTORED_ACC_PER_RANK 0x200u    /* push-with-add: add every source's elements into dst with
                                         atomics of their own (N atomics per dst word, as N
                                         ranks' remote stores land) instead of folding the
                                         call's sources first and adding the fold (one) */
#define PTORED_FULL_OCCUPANCY 0x80u   /* let every CU hold as many workgroups as fit, instead of
                                         the 3-16 per CU the automatic launch keeps resident
                                         by reserving LDS it does not use -- a reservation
                                         that also keeps kernels running concurrently on
                                         other streams off those CUs' LDS; set this when the
                                         reduction overlaps such kernels */

/* Launch choices of ptored_treduce_ex. */
typedef struct ptored_tuning {
    uint32_t flags;          /* PTORED_FORCE_* and PTORED_NO_XCD_REMAP bits */
    int32_t blocks_per_cu;   /* 0 = one workgroup (one wave) per tile (default; 3-16 resident
                                per compute unit, by rank count); > 0 = persistent
                                grid of that many workgroups per compute unit, in per-XCD
                                bands; < 0 = persistent grid at the kernel's occupancy */
    int64_t max_launch_bytes; /* split a call into launches that touch at most this many
                                 bytes of each buffer; 0 = auto (2^31) */
} ptored_tuning;

/* ptored_treduce with explicit launch choices; `tuning` may be NULL (= all
 * automatic).  Results are identical for every choice. */
int ptored_treduce_ex(const void* const* srcs, int nranks, int root, void* dst, int64_t rows,
                      int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols,
                      int dtype, int op, const ptored_tuning* tuning, hipStream_t stream);

/* Kernel family the automatic choice would take (no HIP call, no launch). */
#define PTORED_PATH_NONE 0        /* empty rectangle: nothing launched */
#define PTORED_PATH_COPY 1        /* N == 1 copy */
#define PTORED_PATH_VEC_FIXED 2   /* 16-B vectors, N unrolled at compile time */
#define PTORED_PATH_VEC_RUNTIME 3 /* 16-B vectors, rank-count loop */
#define PTORED_PATH_ELEMENTWISE 4 /* one element per slot (forced, rows shorter than their
                                     first 16-byte block, misaligned data through the LDS
                                     variant, or push-with-add with an odd pitch) */

typedef struct ptored_plan_info {
    int32_t path;          /* PTORED_PATH_* */
    int32_t rows_mode;     /* 1: 2-D row walk; 0: one contiguous span */
    int32_t vec_elems;     /* elements per slot */
    int32_t slots_per_thread; /* slots one thread handles per tile */
    int64_t slots;         /* slots in the whole call */
    int64_t launches;      /* kernel launches the call is split into */
    int32_t wgs_per_cu;    /* workgroups kept resident per CU by one-tile-per-block
                              launches large enough to fill them; 0 = as many as fit */
    int32_t lead;          /* vector path: bytes past the slot origin at which every buffer
                              starts -- the coarsest of a 1 KiB, 128-byte or 16-byte
                              boundary at which every buffer (and, for rows, the pitch)
                              has the same offset; with none, dst's offset past the
                              coarsest such boundary the pitch keeps, or 0 (slots from
                              each row's start) for a pitch off the 16-byte grid; a row
                              starting inside a 16-byte block begins with a head */
} ptored_plan_info;

/* Validate like ptored_treduce_ex and describe the launch it would make,
 * without any HIP call.  Returns the same status codes. */
int ptored_treduce_plan(const void* const* srcs, int nranks, int root, const void* dst,
                        int64_t rows, int64_t cols, int64_t ld, int64_t valid_rows,
                        int64_t valid_cols, int dtype, int op, const ptored_tuning* tuning,
                        ptored_plan_info* info);

/*
 * ptored_allreduce -- the in-place allreduce of one device's share
 * ([N6] pld.tensor.allreduce: every participating rank's window slice is
 * reduced in place).  Every buffer's valid rectangle is replaced by the fold
 * of all N buffers (same fold order and arithmetic as ptored_treduce with
 * the same root); everything outside the valid rectangle is left unchanged.
 *
 * bufs        HOST array of N DEVICE pointers, each read and written.  Two
 *             entries may be the same buffer; partially overlapping buffers
 *             are rejected (PTORED_ERR_OVERLAP).  N == 1 changes nothing.
 * Other arguments and errors as ptored_treduce_ex (tuning may be NULL).
 * Bytes moved: N reads and N writes of the valid rectangle.
 */
int ptored_allreduce(void* const* bufs, int nranks, int root, int64_t rows, int64_t cols,
                     int64_t ld, int64_t valid_rows, int64_t valid_cols, int dtype, int op,
                     const ptored_tuning* tuning, hipStream_t stream);

/*
 * ptored_ring_bounds -- segment boundaries of the ring schedule ([N6]
 * pld.tensor.allreduce, ring mode): a stream of `count` elements is cut at
 * floor(i * count / N); for 2-byte element types every interior boundary is
 * then rounded up to a multiple of 16 elements (32 bytes) and capped at
 * `count`, so short streams can have empty segments.  `bounds` (HOST, N + 1
 * entries) receives 0, b_1, ..., b_{N-1}, count.  No HIP call.
 */
int ptored_ring_bounds(int64_t count, int nranks, int dtype, int64_t* bounds);

/*
 * ptored_reduce_scatter_ring -- the reduce-scatter half of the ring schedule
 * on one device.  Segment s ([b_s, b_{s+1}) of ptored_ring_bounds) of the
 * N source streams is folded in ring order -- ranks s+1, s+2, ..., s (mod N),
 * the order in which a ring passes the partial result from rank s+1 round
 * to its owner s -- and written to dsts[s] at the same element positions.
 * Nothing else of any dst is written.
 *
 * srcs, dsts  HOST arrays of N DEVICE pointers to streams of `count`
 *             elements.  dsts[s] may be srcs[s] (in place into the owner's
 *             window), any other source or another dst; partial overlaps are
 *             rejected.
 * Errors as ptored_treduce_ex.  When the 16-byte kernels apply (at any
 * alignment, as for ptored_treduce), one launch covers every segment (a
 * window of at most max_launch_bytes per launch): each workgroup takes one
 * segment's tile and folds it in that segment's ring order, and one more
 * tile per segment folds its elements outside whole 16-byte slots.
 * Otherwise, or with PTORED_SEGMENT_LAUNCHES, one launch per non-empty
 * segment.
 */
int ptored_reduce_scatter_ring(const void* const* srcs, int nranks, void* const* dsts,
                               int64_t count, int dtype, int op, const ptored_tuning* tuning,
                               hipStream_t stream);

/*
 * ptored_accumulate_add -- push-with-add into one slice ([N6]
 * pld.tensor.put / remote_store with atomic = kAdd, the pushed data added
 * into the peer's slice): dst[i, j] += src_0[i, j] + ... + src_{N-1}[i, j]
 * over the valid rectangle, with device-scope atomic adds, so pushes from
 * other calls, streams or kernels into the same dst may land at the same
 * time.
 *
 * By default the call's N sources are first folded in rank order exactly as
 * ptored_treduce folds them with root 0 (element-type rounding after every
 * step), and the fold f is added into dst with one atomic per 32-bit word:
 * with no concurrent push, dst[i, j] becomes dst[i, j] + f[i, j] rounded
 * once to the element type (i32: wrapping).  With PTORED_ACC_PER_RANK in
 * tuning->flags every source's elements are added with atomics of their
 * own (N per element, as N ranks' remote stores land), in an order that
 * varies from run to run: float results then agree with any fixed order
 * only within the rounding of N additions; i32 stays exact.
 *
 * f32 atomics add two binary32 values and round to nearest-even; bf16 and
 * f16 elements are added two per word by packed atomics.  A 16-bit element
 * that does not fill its aligned 32-bit word is added by a compare-and-swap
 * on that word which rewrites only its own half.  dst must be device memory
 * of this GPU and must not overlap any source (not even exactly).  The
 * 16-byte kernel keeps dst aligned (sources at other offsets are read
 * unaligned) and needs a pitch on the 16-byte grid, so that its atomics stay
 * on naturally aligned words; with an odd pitch the sources are added
 * element by element.  Other arguments and errors as ptored_treduce_ex.
 * Bytes moved: N reads of the valid rectangle and one atomic read-modify-
 * write of dst (N with PTORED_ACC_PER_RANK).
 */
int ptored_accumulate_add(const void* const* srcs, int nranks, void* dst, int64_t rows,
                          int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols,
                          int dtype, const ptored_tuning* tuning, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* ptored_status_string(int status);

/* PTORED_ABI_VERSION of the built library. */
int ptored_abi_version(void);

/* PTORED_MAX_RANKS of the built library. */
int ptored_max_ranks(void);

#ifdef __cplusplus
}
#endif

#endif /* PTORED_H */
