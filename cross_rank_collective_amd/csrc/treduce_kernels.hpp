// treduce_kernels.hpp -- gfx950 kernels of the N-way reduction.
//
// Sources (cited by title and section):
//   [TREDUCE]  "CANN PTO-ISA TREDUCE instruction explained" (lpnh.cn article
//              on pto-isa): §1.1 definition, §1.3 ReduceTiles op mapping,
//              §4.1 dispatch, §4.2 2-D sliding chunk walk with row/column
//              masks, §4.3 load-root / fold-the-others / store order, §4.4
//              ping-pong loads.
//   [N6]       "Distributed Operators (N6)", PyPTO docs: pld.tensor.allreduce
//              (ragged last chunk keeps its width with a smaller valid
//              extent) and "Host multi-core AllReduce" (block-cyclic tile
//              ownership).
//
// Work decomposition.  The valid rectangle is cut into slots: a slot is a
// run of VEC consecutive elements of one row (16 bytes on the vector path,
// one element on the element-wise path).  A tile is BLOCK * U slots, walked
// in one of three ways:
//   contiguous  the valid rows follow each other without a gap: one span,
//               tiles of consecutive slots;
//   row tiles   the pages' 2-D sliding chunk walk: tile (r, c) is column
//               chunk c of row r, the last chunk of a row masked (or, when
//               it would be at most half full, left to the tail tiles) --
//               used when rows are wide enough to keep the threads busy;
//   flattened   narrow rows: slots numbered row-major straight through the
//               rectangle, the row found by a multiply-high division.
// Block b takes tiles b, b+G, b+2G, ... of a grid of G blocks (the pages'
// block-cyclic walk).  By default G equals the tile count -- one tile per
// block, handed out in order by the hardware dispatcher, round-robin over
// the XCDs, as blocks retire -- and the host keeps only 3-16 blocks resident
// per CU (an LDS reservation, by rank count), so the tiles in
// flight cover a compact window of every buffer; a smaller persistent grid
// can be requested.  A block is one wave: its U * 64 slots are consecutive
// and lane l takes slots l, l+64, ..., so every wave instruction moves
// 1 KiB of one buffer.
//
// Per slot a thread issues the loads of all N sources before it combines
// anything -- the many waves in flight on a CU take the place of the pages'
// ping-pong recv tiles -- then folds them in the fixed order (root first,
// then ascending rank; the host passes the pointers already in that order),
// rounding to the element type after every step, and stores the result.
// Elements outside the valid rectangle are never read or written.
//
// Memory path.  Every access is a buffer instruction against a resource
// whose record count is the byte extent this launch may touch, so the
// hardware drops any access past it (loads return zero, stores are
// discarded): slots past the end of the work are given an offset beyond
// the extent instead of a branch.  Source loads are non-temporal (the data
// is used once); stores of dst are non-temporal, or device-scope (sc1: written
// through the XCD's L2) at one and four ranks, whichever measured faster on
// MI355X for a dst that goes to HBM on every call; the in-place allreduce's
// N store-backs take sc1 | nt.  Push-with-add replaces the store by device-scope
// atomic adds on naturally aligned 32-bit words (through global addresses,
// so those offsets are checked against the work, not the extent).
//
// Ragged edges.  Full 16-byte slots form the main tiles.  They are numbered
// from an aligned origin below the data (1 KiB, 128 bytes or 16 bytes, the
// coarsest at which every buffer has the same offset), so every wave's run
// is aligned; the slots before the data are skipped.  Buffers with no offset
// in common take dst's origin, and rows whose pitch is off the 16-byte grid
// number their slots from each row's start: every access is a byte offset
// from each buffer's own base, so the other buffers' accesses are simply
// unaligned, which the hardware serves in the unaligned access mode the HSA
// ABI enables.  Separate tail tiles
// -- placed before the main tiles in the grid, so their scattered accesses
// overlap the streaming -- carry, one item per thread: a row's valid bytes
// after its last full slot (fewer than 16, at most two exact-size accesses
// per buffer, e.g. 12 + 2 bytes for seven 16-bit elements), a row's head
// (its bytes before the first 16-byte boundary when the data starts inside
// a slot, at most three aligned accesses), and a row's last few full slots
// when they would fill at most half of a row tile.  Nothing outside the
// valid rectangle is touched, and the main tiles are branch-free.  The
// element-wise path (forced, rows that never reach their first 16-byte
// boundary, misaligned data through the LDS variant, or push-with-add with
// a pitch off the 16-byte grid)
// has no main tiles: its tail tiles carry every element of the rectangle,
// one element per access.
//
// Combines on gfx950 (element type kept after every step):
//   f32  sum v_add_f32, prod v_mul_f32, max/min v_maximum3_f32 / v_minimum3_f32
//   f16  sum v_pk_add_f16, prod v_pk_mul_f16, max/min v_pk_maximum3_f16 / ...
//   bf16 sum/prod: widen both halves to f32 (exact), add/mul, round back to
//        bf16 with v_cvt_pk_bf16_f32 (nearest-even); max/min: widen and use
//        v_maximum3_f32 / v_minimum3_f32, whose result is one of the
//        operands, then take the upper halves back.
//   i32  v_add_u32 / v_mul_lo_u32 (wrap), v_max3_i32 / v_min3_i32.
// Rounding an f32 sum of two bf16 (or the f16 hardware add) to the element
// type gives the same bits as rounding the exact sum once, since binary32
// carries at least 2p+2 significand bits for p = 8 and p = 11; an f32 product
// of two bf16 values is exact or, in the subnormal range, exact to a grid
// fine enough that the second rounding cannot meet a false tie.
// IEEE-754 maximum/minimum order -0 below +0 and turn any NaN into a NaN,
// which is the extremum rule of the reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treduce_plan.h"

namespace ptored {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------
// Combine on one 32-bit word: one f32 / i32 element, or two bf16 / f16
// elements (lane 0 in the low half).  Acc<DT, OP> holds the running value;
// add(x) performs acc = acc (+) x, add2(x, y) performs two steps in order.
// ------------------------------------------------------------------------

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u(h2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float bf_lo(uint32_t u) { return as_f(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return as_f(u & 0xFFFF0000u); }
// Two f32 values rounded to bf16 (nearest-even) and packed, lo in bits 0..15.
__device__ __forceinline__ uint32_t bf_pack_rne(float lo, float hi) {
    f2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
}
// Upper halves of two f32 values whose low halves are zero (exact bf16).
__device__ __forceinline__ uint32_t bf_pack_exact(float lo, float hi) {
    return __builtin_amdgcn_perm(as_u(hi), as_u(lo), 0x07060302u);
}

template <int DT, int OP>
struct Acc;

// f32 -------------------------------------------------------------------
template <>
struct Acc<PTORED_F32, PTORED_SUM> {
    float v;
    __device__ __forceinline__ void init(uint32_t x) { v = as_f(x); }
    __device__ __forceinline__ void add(uint32_t x) { v = v + as_f(x); }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) { add(x); add(y); }
    __device__ __forceinline__ uint32_t get() const { return as_u(v); }
};
template <>
struct Acc<PTORED_F32, PTORED_PROD> {
    float v;
    __device__ __forceinline__ void init(uint32_t x) { v = as_f(x); }
    __device__ __forceinline__ void add(uint32_t x) { v = v * as_f(x); }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) { add(x); add(y); }
    __device__ __forceinline__ uint32_t get() const { return as_u(v); }
};
template <>
struct Acc<PTORED_F32, PTORED_MAX> {
    float v;
    __device__ __forceinline__ void init(uint32_t x) { v = as_f(x); }
    __device__ __forceinline__ void add(uint32_t x) {
        v = __builtin_elementwise_maximum(v, as_f(x));
    }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) {
        v = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v, as_f(x)), as_f(y));
    }
    __device__ __forceinline__ uint32_t get() const { return as_u(v); }
};
template <>
struct Acc<PTORED_F32, PTORED_MIN> {
    float v;
    __device__ __forceinline__ void init(uint32_t x) { v = as_f(x); }
    __device__ __forceinline__ void add(uint32_t x) {
        v = __builtin_elementwise_minimum(v, as_f(x));
    }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) {
        v = __builtin_elementwise_minimum(__builtin_elementwise_minimum(v, as_f(x)), as_f(y));
    }
    __device__ __forceinline__ uint32_t get() const { return as_u(v); }
};

// i32 -------------------------------------------------------------------
template <>
struct Acc<PTORED_I32, PTORED_SUM> {
    uint32_t v;
    __device__ __forceinline__ void init(uint32_t x) { v = x; }
    __device__ __forceinline__ void add(uint32_t x) { v = v + x; }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) { v = v + x + y; }
    __device__ __forceinline__ uint32_t get() const { return v; }
};
template <>
struct Acc<PTORED_I32, PTORED_PROD> {
    uint32_t v;
    __device__ __forceinline__ void init(uint32_t x) { v = x; }
    __device__ __forceinline__ void add(uint32_t x) { v = v * x; }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) { add(x); add(y); }
    __device__ __forceinline__ uint32_t get() const { return v; }
};
template <>
struct Acc<PTORED_I32, PTORED_MAX> {
    int32_t v;
    __device__ __forceinline__ void init(uint32_t x) { v = (int32_t)x; }
    __device__ __forceinline__ void add(uint32_t x) { v = max(v, (int32_t)x); }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) {
        v = max(max(v, (int32_t)x), (int32_t)y);
    }
    __device__ __forceinline__ uint32_t get() const { return (uint32_t)v; }
};
template <>
struct Acc<PTORED_I32, PTORED_MIN> {
    int32_t v;
    __device__ __forceinline__ void init(uint32_t x) { v = (int32_t)x; }
    __device__ __forceinline__ void add(uint32_t x) { v = min(v, (int32_t)x); }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) {
        v = min(min(v, (int32_t)x), (int32_t)y);
    }
    __device__ __forceinline__ uint32_t get() const { return (uint32_t)v; }
};

// f16 (two lanes per word) ----------------------------------------------
template <>
struct Acc<PTORED_F16, PTORED_SUM> {
    h2 v;
    __device__ __forceinline__ void init(uint32_t x) { v = as_h2(x); }
    __device__ __forceinline__ void add(uint32_t x) { v = v + as_h2(x); }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) { add(x); add(y); }
    __device__ __forceinline__ uint32_t get() const { return as_u(v); }
};
template <>
struct Acc<PTORED_F16, PTORED_PROD> {
    h2 v;
    __device__ __forceinline__ void init(uint32_t x) { v = as_h2(x); }
    __device__ __forceinline__ void add(uint32_t x) { v = v * as_h2(x); }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) { add(x); add(y); }
    __device__ __forceinline__ uint32_t get() const { return as_u(v); }
};
template <>
struct Acc<PTORED_F16, PTORED_MAX> {
    h2 v;
    __device__ __forceinline__ void init(uint32_t x) { v = as_h2(x); }
    __device__ __forceinline__ void add(uint32_t x) {
        v = __builtin_elementwise_maximum(v, as_h2(x));
    }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) {
        v = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v, as_h2(x)), as_h2(y));
    }
    __device__ __forceinline__ uint32_t get() const { return as_u(v); }
};
template <>
struct Acc<PTORED_F16, PTORED_MIN> {
    h2 v;
    __device__ __forceinline__ void init(uint32_t x) { v = as_h2(x); }
    __device__ __forceinline__ void add(uint32_t x) {
        v = __builtin_elementwise_minimum(v, as_h2(x));
    }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) {
        v = __builtin_elementwise_minimum(__builtin_elementwise_minimum(v, as_h2(x)), as_h2(y));
    }
    __device__ __forceinline__ uint32_t get() const { return as_u(v); }
};

// bf16 (two lanes per word, kept widened to f32 between steps) -----------
template <>
struct Acc<PTORED_BF16, PTORED_SUM> {
    float lo, hi;
    uint32_t packed;
    __device__ __forceinline__ void init(uint32_t x) {
        packed = x;
        lo = bf_lo(x);
        hi = bf_hi(x);
    }
    __device__ __forceinline__ void add(uint32_t x) {
        packed = bf_pack_rne(lo + bf_lo(x), hi + bf_hi(x));
        lo = bf_lo(packed);
        hi = bf_hi(packed);
    }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) { add(x); add(y); }
    __device__ __forceinline__ uint32_t get() const { return packed; }
};
template <>
struct Acc<PTORED_BF16, PTORED_PROD> {
    float lo, hi;
    uint32_t packed;
    __device__ __forceinline__ void init(uint32_t x) {
        packed = x;
        lo = bf_lo(x);
        hi = bf_hi(x);
    }
    __device__ __forceinline__ void add(uint32_t x) {
        packed = bf_pack_rne(lo * bf_lo(x), hi * bf_hi(x));
        lo = bf_lo(packed);
        hi = bf_hi(packed);
    }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) { add(x); add(y); }
    __device__ __forceinline__ uint32_t get() const { return packed; }
};
template <>
struct Acc<PTORED_BF16, PTORED_MAX> {
    float lo, hi;
    __device__ __forceinline__ void init(uint32_t x) { lo = bf_lo(x); hi = bf_hi(x); }
    __device__ __forceinline__ void add(uint32_t x) {
        lo = __builtin_elementwise_maximum(lo, bf_lo(x));
        hi = __builtin_elementwise_maximum(hi, bf_hi(x));
    }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) {
        lo = __builtin_elementwise_maximum(__builtin_elementwise_maximum(lo, bf_lo(x)), bf_lo(y));
        hi = __builtin_elementwise_maximum(__builtin_elementwise_maximum(hi, bf_hi(x)), bf_hi(y));
    }
    __device__ __forceinline__ uint32_t get() const { return bf_pack_exact(lo, hi); }
};
template <>
struct Acc<PTORED_BF16, PTORED_MIN> {
    float lo, hi;
    __device__ __forceinline__ void init(uint32_t x) { lo = bf_lo(x); hi = bf_hi(x); }
    __device__ __forceinline__ void add(uint32_t x) {
        lo = __builtin_elementwise_minimum(lo, bf_lo(x));
        hi = __builtin_elementwise_minimum(hi, bf_hi(x));
    }
    __device__ __forceinline__ void add2(uint32_t x, uint32_t y) {
        lo = __builtin_elementwise_minimum(__builtin_elementwise_minimum(lo, bf_lo(x)), bf_lo(y));
        hi = __builtin_elementwise_minimum(__builtin_elementwise_minimum(hi, bf_hi(x)), bf_hi(y));
    }
    __device__ __forceinline__ uint32_t get() const { return bf_pack_exact(lo, hi); }
};

// ------------------------------------------------------------------------
// Memory access: buffer instructions with a per-launch record count.
// ------------------------------------------------------------------------

// Word 3 of a raw buffer resource: 32-bit data format, no swizzle, stride 0.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy bits of the buffer instructions (gfx950): nt (2) for loads;
// for stores of dst, nt or sc1 (16: device scope, write-through of the XCD's
// L2) by rank count, and sc1 | nt for the in-place allreduce's store-backs.
// Measured on MI355X with dst written to HBM on every call: nt stores ahead
// by 1-4% from 5 ranks on (and at 2), sc1 ahead at 1 and 4 ranks; the
// allreduce's sc1 | nt ahead of nt alone.  (A dst rewritten back to back,
// which stays in the Infinity Cache, favours sc1 throughout.)
constexpr int kLoadPolicy = 2;
constexpr int kStoreNt = 2;
constexpr int kStoreSc1 = 16;
constexpr int kStoreAllPolicy = 18;
// Store policy of dst for NR ranks (NR == 0: a runtime count, above 16).
constexpr int store_policy_for(int nr) { return (nr == 1 || nr == 4) ? kStoreSc1 : kStoreNt; }
// An offset no launch extent reaches (extents are capped at 2^31 bytes).
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t extent) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)extent,
                                             kRsrcWord3);
}
__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadPolicy);
}
template <int POL>
__device__ __forceinline__ void store16(rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POL);
}
// One element of ES bytes, zero-extended into a word (lane 0).
template <int ES>
__device__ __forceinline__ uint32_t load_elem(rsrc_t r, uint32_t off) {
    if constexpr (ES == 4) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kLoadPolicy);
    } else {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kLoadPolicy);
    }
}
template <int ES, int POL>
__device__ __forceinline__ void store_elem(rsrc_t r, uint32_t off, uint32_t v) {
    if constexpr (ES == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, POL);
    } else {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, POL);
    }
}

// Bytes [0, TB) of a 16-byte slot, TB < 16 and a multiple of 2, as at most
// two accesses (12, 8 or 4 bytes, then 2), into the low words of a vector;
// the words past TB are zero.
template <int TB>
__device__ __forceinline__ u32x4 load_partial(rsrc_t r, uint32_t off) {
    u32x4 v = {0u, 0u, 0u, 0u};
    constexpr int big = TB >= 12 ? 12 : (TB >= 8 ? 8 : (TB >= 4 ? 4 : 0));
    if constexpr (big == 12) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, kLoadPolicy);
        v[0] = w[0]; v[1] = w[1]; v[2] = w[2];
    } else if constexpr (big == 8) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadPolicy);
        v[0] = w[0]; v[1] = w[1];
    } else if constexpr (big == 4) {
        v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kLoadPolicy);
    }
    if constexpr (TB - big == 2) {
        v[big / 4] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off + big, 0, kLoadPolicy);
    }
    return v;
}
template <int TB, int POL>
__device__ __forceinline__ void store_partial(rsrc_t r, uint32_t off, u32x4 v) {
    constexpr int big = TB >= 12 ? 12 : (TB >= 8 ? 8 : (TB >= 4 ? 4 : 0));
    if constexpr (big == 12) {
        typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
        const u32x3 w = {v[0], v[1], v[2]};
        __builtin_amdgcn_raw_buffer_store_b96(w, r, off, 0, POL);
    } else if constexpr (big == 8) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = {v[0], v[1]};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, POL);
    } else if constexpr (big == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(v[0], r, off, 0, POL);
    }
    if constexpr (TB - big == 2) {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v[big / 4], r, off + big, 0,
                                             POL);
    }
}

// Bytes [LO, 16) of a 16-byte slot (LO a multiple of 2, 0 < LO < 16) in
// pieces aligned from the slot's start -- 2 bytes at LO when LO is 2 mod 4,
// then 4 bytes to reach an 8-byte boundary, then 8 -- into the same words of
// a vector as a whole slot would fill; the bytes before LO are zero.
template <int LO>
__device__ __forceinline__ u32x4 load_head(rsrc_t r, uint32_t off) {
    static_assert(LO > 0 && LO < 16 && LO % 2 == 0, "head range");
    u32x4 v = {0u, 0u, 0u, 0u};
    constexpr int A = (LO + 3) / 4 * 4;  // first 4-byte boundary at or after LO
    if constexpr (LO % 4 == 2) {
        v[LO / 4] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off + LO, 0, kLoadPolicy)
                    << 16;
    }
    if constexpr (A == 4 || A == 12) {
        v[A / 4] = __builtin_amdgcn_raw_buffer_load_b32(r, off + A, 0, kLoadPolicy);
    }
    if constexpr (A <= 8) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8, 0, kLoadPolicy);
        v[2] = w[0];
        v[3] = w[1];
    }
    return v;
}
template <int LO, int POL>
__device__ __forceinline__ void store_head(rsrc_t r, uint32_t off, u32x4 v) {
    constexpr int A = (LO + 3) / 4 * 4;
    if constexpr (LO % 4 == 2) {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(v[LO / 4] >> 16), r, off + LO, 0,
                                             POL);
    }
    if constexpr (A == 4 || A == 12) {
        __builtin_amdgcn_raw_buffer_store_b32(v[A / 4], r, off + A, 0, POL);
    }
    if constexpr (A <= 8) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = {v[2], v[3]};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, off + 8, 0, POL);
    }
}

// Quotient by a per-launch constant without a divide: the multiply-high
// method of Granlund and Montgomery ("Division by invariant integers using
// multiplication", PLDI 1994, Fig. 4.1), exact for every 32-bit dividend.
__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& d) {
    const uint32_t t = __umulhi(n, d.mul);
    return (t + ((n - t) >> d.sh1)) >> d.sh2;
}

// Block index remapped so that the blocks the hardware places on one XCD
// (it deals consecutive workgroups round-robin over the 8 XCDs) get one
// contiguous range of logical indices (persistent grids only).
__device__ __forceinline__ uint32_t logical_block(uint32_t b, uint32_t grid, bool remap) {
    if (!remap || (grid & 7u) != 0u) return b;
    return (b & 7u) * (grid >> 3) + (b >> 3);
}

// Byte offset of numbered slot s (16 bytes) in the contiguous and flattened
// walks, or kOutOfRange past the end and for the skipped slots before a
// row's (or the span's) first full slot.
template <int WALK>
__device__ __forceinline__ uint32_t slot_offset(const KArgs& a, uint32_t s) {
    if (s >= a.nslots) return kOutOfRange;
    if constexpr (WALK == kWalkFlat) {
        const uint32_t row = fast_div(s, a.div_slots);
        const uint32_t v = s - row * a.slots_per_row;
        return v >= a.slot_skip ? row * a.ld_bytes + v * 16u : kOutOfRange;
    } else {
        return s >= a.slot_skip ? s * 16u : kOutOfRange;
    }
}

// Byte offset of element q of the element-wise path, or kOutOfRange past the end.
template <int WALK, int ES>
__device__ __forceinline__ uint32_t tail_offset(const KArgs& a, uint32_t q) {
    if (q >= a.ntail) return kOutOfRange;
    if constexpr (WALK != kWalkContig) {
        const uint32_t row = fast_div(q, a.div_tail);
        return row * a.ld_bytes + a.tail_col_bytes + (q - row * a.tail_per_row) * (uint32_t)ES;
    } else {
        return a.tail_col_bytes + q * (uint32_t)ES;
    }
}

// ------------------------------------------------------------------------
// Atomic adds into dst (push-with-add, [N6] pld.tensor.put / remote_store
// with atomic = kAdd): device-scope, one 32-bit word per atomic --
// global_atomic_add_f32, global_atomic_pk_add_f16, global_atomic_pk_add_bf16
// (two 16-bit elements per word) and global_atomic_add_u32.  On gfx950
// every such atomic is performed past the XCD's L2, at the memory side
// (measured: WRITE_SIZE counts 4 bytes per atomic), so concurrent pushes
// from any XCD, stream or kernel into the same words all land.
// ------------------------------------------------------------------------

typedef short s16x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ void atomic_add_word(char* p, uint32_t bits) {
    if constexpr (DT == PTORED_F32) {
        __hip_atomic_fetch_add(reinterpret_cast<float*>(p), as_f(bits), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (DT == PTORED_I32) {
        __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(p), bits, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (DT == PTORED_F16) {
        __builtin_amdgcn_global_atomic_fadd_v2f16((__attribute__((address_space(1))) h2*)p,
                                                  as_h2(bits));
    } else {
        __builtin_amdgcn_global_atomic_fadd_v2bf16((__attribute__((address_space(1))) s16x2*)p,
                                                   __builtin_bit_cast(s16x2, bits));
    }
}

// a + b for one 16-bit element, rounded to the element type.
template <int DT>
__device__ __forceinline__ uint32_t add16(uint32_t a, uint32_t b) {
    if constexpr (DT == PTORED_F16) {
        return as_u(as_h2(a) + as_h2(b)) & 0xFFFFu;
    } else {
        return bf_pack_rne(bf_lo(a) + bf_lo(b), 0.0f) & 0xFFFFu;
    }
}

// Add one element at p (ES bytes; low bits of `bits`) atomically.  A 16-bit
// element takes a compare-and-swap loop on its aligned 32-bit word that
// rewrites only its own half, so the neighbouring half keeps its bits.
template <int DT, int ES>
__device__ __forceinline__ void atomic_add_elem(char* p, uint32_t bits) {
    if constexpr (ES == 4) {
        atomic_add_word<DT>(p, bits);
    } else {
        const uintptr_t addr = reinterpret_cast<uintptr_t>(p);
        uint32_t* w = reinterpret_cast<uint32_t*>(addr & ~uintptr_t(3));
        const uint32_t shift = (addr & 2u) ? 16u : 0u;
        uint32_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (;;) {
            const uint32_t sum = add16<DT>((old >> shift) & 0xFFFFu, bits & 0xFFFFu);
            const uint32_t desired = (old & ~(0xFFFFu << shift)) | (sum << shift);
            if (__hip_atomic_compare_exchange_strong(w, &old, desired, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                break;
        }
    }
}

// Element-wise push: lane l adds element v[u] at dst byte offset off[u]
// (kOutOfRange: none), where off[u] is element base + u * 64 + l of a run
// of consecutive elements.  For 16-bit types, a lane whose element opens a
// 32-bit word and whose right neighbour -- the next lane, or lane 0 of the
// next slice for lane 63 -- holds the word's other half adds both with one
// packed atomic; every other element takes the half-word compare-and-swap.
// The shuffles run on every lane, before any branch.
template <int DT, int ES, int TU>
__device__ __forceinline__ void push_elements(char* d, const uint32_t (&off)[TU],
                                              const uint32_t (&v)[TU]) {
    if constexpr (ES == 4) {
#pragma unroll
        for (int u = 0; u < TU; ++u)
            if (off[u] != kOutOfRange) atomic_add_word<DT>(d + off[u], v[u]);
    } else {
        const uint32_t lane = threadIdx.x;
#pragma unroll
        for (int u = 0; u < TU; ++u) {
            const bool valid = off[u] != kOutOfRange;
            uint32_t next_off = (uint32_t)__shfl_down((int)off[u], 1, kBlock);
            uint32_t next_v = (uint32_t)__shfl_down((int)v[u], 1, kBlock);
            uint32_t prev_off = (uint32_t)__shfl_up((int)off[u], 1, kBlock);
            if (u + 1 < TU) {
                const uint32_t o = (uint32_t)__shfl((int)off[u + 1], 0, kBlock);
                const uint32_t x = (uint32_t)__shfl((int)v[u + 1], 0, kBlock);
                if (lane == (uint32_t)kBlock - 1u) {
                    next_off = o;
                    next_v = x;
                }
            } else if (lane == (uint32_t)kBlock - 1u) {
                next_off = kOutOfRange;
            }
            if (u > 0) {
                const uint32_t o = (uint32_t)__shfl((int)off[u - 1], kBlock - 1, kBlock);
                if (lane == 0u) prev_off = o;
            } else if (lane == 0u) {
                prev_off = kOutOfRange;
            }
            const bool opens = (reinterpret_cast<uintptr_t>(d + off[u]) & 3u) == 0u;
            const bool leads = valid && opens && next_off == off[u] + 2u;
            const bool led = valid && !opens && prev_off + 2u == off[u];
            if (leads) {
                atomic_add_word<DT>(d + off[u], (v[u] & 0xFFFFu) | (next_v << 16));
            } else if (valid && !led) {
                atomic_add_elem<DT, ES>(d + off[u], v[u]);
            }
        }
    }
}

// Store one finished slot: to dst; back into every source (the in-place
// allreduce of [N6] pld.tensor.allreduce -- each slot is read from every
// buffer by the thread that later writes it, so the write never races a
// read); or added into dst, one atomic per word (push-with-add; dst's slots
// are 16-byte aligned on this path).
template <int DT, int SM, int NR>
__device__ __forceinline__ void store_result(const KArgs& a, rsrc_t rd, uint32_t off, u32x4 v) {
    if constexpr (SM == kStoreAll) {
        for (uint32_t k = 0; k < a.nranks; ++k)
            store16<kStoreAllPolicy>(make_rsrc(a.src[k], a.extent), off, v);
    } else if constexpr (SM == kStoreAdd) {
        if (off != kOutOfRange) {
            char* const p = static_cast<char*>(a.dst) + off;
#pragma unroll
            for (int w = 0; w < 4; ++w) atomic_add_word<DT>(p + 4 * w, v[w]);
        }
    } else {
        store16<store_policy_for(NR)>(rd, off, v);
    }
}

// Fold of one word from NR (compile-time) loaded values, in order.
template <int DT, int OP, int NR, int U>
__device__ __forceinline__ uint32_t fold_word(const u32x4 (&x)[NR][U], int u, int w) {
    Acc<DT, OP> acc;
    acc.init(x[0][u][w]);
#pragma unroll
    for (int k = 1; k + 1 < NR; k += 2) acc.add2(x[k][u][w], x[k + 1][u][w]);
    if constexpr (NR > 1 && (NR - 1) % 2 == 1) acc.add(x[NR - 1][u][w]);
    return acc.get();
}

// Load U slots at byte offsets off[] from NR sources (NR == 0: n at run
// time), source k through src(k), and fold them in order k = 0, 1, ...
// into out[].  Every load of a slot is issued before its fold starts.
template <int DT, int OP, int NR, int U, class SrcFn>
__device__ __forceinline__ void fold_slots(SrcFn src, uint32_t n, const uint32_t (&off)[U],
                                           u32x4 (&out)[U]) {
    if constexpr (NR > 0) {
        u32x4 x[NR][U];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const rsrc_t r = src((uint32_t)k);
#pragma unroll
            for (int u = 0; u < U; ++u) x[k][u] = load16(r, off[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) out[u][w] = fold_word<DT, OP, NR, U>(x, u, w);
    } else {
        // Runtime rank count: groups of four sources in flight, then the
        // remainder one at a time, always in order.
        Acc<DT, OP> acc[U][4];
        {
            const rsrc_t r = src(0u);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const u32x4 x0 = load16(r, off[u]);
#pragma unroll
                for (int w = 0; w < 4; ++w) acc[u][w].init(x0[w]);
            }
        }
        uint32_t k = 1;
        for (; k + 4 <= n; k += 4) {
            u32x4 x[4][U];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const rsrc_t r = src(k + (uint32_t)g);
#pragma unroll
                for (int u = 0; u < U; ++u) x[g][u] = load16(r, off[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    acc[u][w].add2(x[0][u][w], x[1][u][w]);
                    acc[u][w].add2(x[2][u][w], x[3][u][w]);
                }
        }
        for (; k < n; ++k) {
            const rsrc_t r = src(k);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const u32x4 x = load16(r, off[u]);
#pragma unroll
                for (int w = 0; w < 4; ++w) acc[u][w].add(x[w]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) out[u][w] = acc[u][w].get();
    }
}

// Byte offsets of the U slots a lane folds in main tile t (kOutOfRange for
// slots past a row's end or before its first full slot).  Row tiles: tile t
// is column chunk c of row r (t = r * tiles_per_row + c, split on the scalar
// unit), so every wave's 1 KiB run starts a whole number of KiB past the
// row's slot origin and never shares a cache line with another wave; the
// other walks number the slots straight through.
template <int U, int WALK>
__device__ __forceinline__ void main_tile_offsets(const KArgs& a, uint32_t t,
                                                  uint32_t (&off)[U]) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t in_tile = wave * (uint32_t)(64 * U) + lane;
    if constexpr (WALK == kWalkRowTiles) {
        const uint32_t row = fast_div(t, a.div_tiles);
        const uint32_t v0 = (t - row * a.tiles_per_row) * (uint32_t)(kBlock * U) + in_tile;
        const uint32_t row_off = row * a.ld_bytes;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t v = v0 + (uint32_t)(u * 64);
            off[u] = v < a.slots_per_row && v >= a.slot_skip ? row_off + v * 16u : kOutOfRange;
        }
    } else {
        const uint32_t base = t * (uint32_t)(kBlock * U) + in_tile;
#pragma unroll
        for (int u = 0; u < U; ++u) off[u] = slot_offset<WALK>(a, base + (uint32_t)(u * 64));
    }
}

// Byte offset of slot s (0 <= s < 64 U) of main tile t, as main_tile_offsets
// gives it to the lane that folds it.
template <int U, int WALK>
__device__ __forceinline__ uint32_t tile_slot_offset(const KArgs& a, uint32_t t, uint32_t s) {
    if constexpr (WALK == kWalkRowTiles) {
        const uint32_t row = fast_div(t, a.div_tiles);
        const uint32_t v = (t - row * a.tiles_per_row) * (uint32_t)(kBlock * U) + s;
        return v < a.slots_per_row && v >= a.slot_skip ? row * a.ld_bytes + v * 16u
                                                       : kOutOfRange;
    } else {
        return slot_offset<WALK>(a, t * (uint32_t)(kBlock * U) + s);
    }
}

// Push-with-add of one main tile's folded slots.  Lane l holds slot
// 64 u + l; the slots pass through LDS so that word j of each 1 KiB run is
// added by lane j % 64 in step j / 64: every atomic instruction of the wave
// covers 256 contiguous bytes (two cache lines).  A lane adding its own
// slot's four words would spread each instruction over eight lines -- on
// MI355X four times slower at the memory side, where the atomics are done.
template <int DT, int U, int WALK>
__device__ __forceinline__ void push_tile(const KArgs& a, uint32_t t, const u32x4 (&out)[U]) {
    __shared__ uint32_t xpose[U][256];
    const uint32_t lane = threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) *reinterpret_cast<u32x4*>(&xpose[u][lane * 4u]) = out[u];
    __syncthreads();
    char* const d = static_cast<char*>(a.dst);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t s = (uint32_t)(u * 64 + k * 16) + (lane >> 2);
            const uint32_t off = tile_slot_offset<U, WALK>(a, t, s);
            const uint32_t v = xpose[u][k * 64 + lane];
            if (off != kOutOfRange) atomic_add_word<DT>(d + off + 4u * (lane & 3u), v);
        }
    __syncthreads();  // the next tile of a persistent grid rewrites xpose
}

// One main tile: U full 16-byte slots per thread, NR sources.
template <int DT, int OP, int NR, int U, int WALK, int SM>
__device__ __forceinline__ void main_tile(const KArgs& a, uint32_t t) {
    uint32_t off[U];
    main_tile_offsets<U, WALK>(a, t, off);
    const rsrc_t rd = make_rsrc(a.dst, a.extent);
    u32x4 out[U];
    fold_slots<DT, OP, NR, U>([&](uint32_t k) { return make_rsrc(a.src[k], a.extent); },
                              a.nranks, off, out);
    if constexpr (SM == kStoreAdd) {
        push_tile<DT, U, WALK>(a, t, out);
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) store_result<DT, SM, NR>(a, rd, off[u], out[u]);
    }
}

// ------------------------------------------------------------------------
// LDS ping-pong variant (the pages' ping/pong recv tiles, [TREDUCE] §2.2 and
// §4.4): every wave streams the sources through a ring of S 1-KiB LDS stages
// with gfx950's direct buffer-to-LDS loads, folding stage k while the loads
// of ranks k+1 .. k+S-1 are in flight.  Each lane reads back exactly the 16
// bytes it loaded (the load writes lane l's data at stage + 16 l), so the
// stages are private to the wave and need no barrier.  The compiler does not
// order an LDS read after the load that fills it, so the waits are explicit:
// s_waitcnt vmcnt(n) before a stage is read (n = loads issued after it); the
// read itself waits lgkmcnt(0) before the stage is refilled.
// ------------------------------------------------------------------------

// s_waitcnt immediates (gfx9 encoding): wait for vmcnt <= n only / lgkmcnt == 0 only.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}
// wait until at most n (0 <= n < S) vector loads of this wave are outstanding
template <int S>
__device__ __forceinline__ void wait_vmcnt_upto(uint32_t n) {
    if constexpr (S > 1) {
        if (n >= (uint32_t)(S - 1)) {
            wait_vmcnt<S - 1>();
            return;
        }
        wait_vmcnt_upto<S - 1>(n);
    } else {
        wait_vmcnt<0>();
    }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Read 16 bytes of LDS and wait for them.  Written as one asm block so the
// compiler, which cannot tell which in-flight LDS load this read depends on,
// does not add a wait for all of them; the caller's vmcnt wait orders it.
__device__ __forceinline__ u32x4 lds_read16(const uint32_t* p) {
    u32x4 v;
    const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

template <int S>
struct LdsStages {
    // [wave][stage][64 lanes x 16 bytes]
    uint32_t words[kBlock / 64][S][256];
};

template <int DT, int OP, int S, int WALK>
__device__ __forceinline__ void main_tile_lds(const KArgs& a, uint32_t t, LdsStages<S>& st) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    uint32_t offs[1];
    main_tile_offsets<1, WALK>(a, t, offs);
    const uint32_t off = offs[0];
    const uint32_t n = a.nranks;
    // prologue: the first min(S, N) ranks
#pragma unroll
    for (int k = 0; k < S; ++k) {
        if ((uint32_t)k < n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(a.src[k], a.extent),
                                                     (lds_ptr_t)&st.words[wave][k][0], 16, off,
                                                     0, 0, kLoadPolicy);
    }
    Acc<DT, OP> acc[4];
    for (uint32_t k = 0; k < n; ++k) {
        const uint32_t after = min((uint32_t)(S - 1), n - 1 - k);  // loads issued after k
        wait_vmcnt_upto<S>(after);
        const uint32_t slot = k % (uint32_t)S;
        const u32x4 x = lds_read16(&st.words[wave][slot][lane * 4]);
        if (k + S < n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(a.src[k + S], a.extent),
                                                     (lds_ptr_t)&st.words[wave][slot][0], 16,
                                                     off, 0, 0, kLoadPolicy);
        if (k == 0) {
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[w].init(x[w]);
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[w].add(x[w]);
        }
    }
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) out[w] = acc[w].get();
    store16<store_policy_for(0)>(make_rsrc(a.dst, a.extent), off, out);
}

// One tail tile of the element-wise path: kElemUnroll elements per thread,
// element by element.
template <int DT, int OP, int ES, int NR, int WALK, int SM>
__device__ __forceinline__ void element_tile(const KArgs& a, uint32_t t) {
    constexpr int TU = kElemUnroll;
    const uint32_t base = t * (uint32_t)(kBlock * TU) + threadIdx.x;
    uint32_t off[TU];
#pragma unroll
    for (int u = 0; u < TU; ++u) off[u] = tail_offset<WALK, ES>(a, base + (uint32_t)(u * kBlock));
    const rsrc_t rd = make_rsrc(a.dst, a.extent);
    Acc<DT, OP> acc[TU];
    {
        const rsrc_t r = make_rsrc(a.src[0], a.extent);
#pragma unroll
        for (int u = 0; u < TU; ++u) acc[u].init(load_elem<ES>(r, off[u]));
    }
    const uint32_t n = NR > 0 ? (uint32_t)NR : a.nranks;
    for (uint32_t k = 1; k < n; ++k) {
        const rsrc_t r = make_rsrc(a.src[k], a.extent);
        uint32_t x[TU];
#pragma unroll
        for (int u = 0; u < TU; ++u) x[u] = load_elem<ES>(r, off[u]);
#pragma unroll
        for (int u = 0; u < TU; ++u) acc[u].add(x[u]);
    }
    if constexpr (SM == kStoreAdd) {
        uint32_t v[TU];
#pragma unroll
        for (int u = 0; u < TU; ++u) v[u] = ES == 4 ? acc[u].get() : acc[u].get() & 0xFFFFu;
        push_elements<DT, ES, TU>(static_cast<char*>(a.dst), off, v);
        return;
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
        if constexpr (SM == kStoreAll) {
            for (uint32_t k = 0; k < n; ++k)
                store_elem<ES, kStoreAllPolicy>(make_rsrc(a.src[k], a.extent), off[u],
                                                acc[u].get());
        } else {
            store_elem<ES, store_policy_for(NR)>(rd, off[u], acc[u].get());
        }
    }
}

// One row remainder of TB bytes (the pages' partial column chunk with a
// dynamic valid extent): loaded from every source, folded lane-wise in the
// same order as the main tiles, stored with the same two exact accesses.
template <int DT, int OP, int ES, int NR, int TB, int SM>
__device__ __forceinline__ void row_tail(const KArgs& a, uint32_t off) {
    const rsrc_t rd = make_rsrc(a.dst, a.extent);
    Acc<DT, OP> acc[4];
    {
        const u32x4 x0 = load_partial<TB>(make_rsrc(a.src[0], a.extent), off);
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w].init(x0[w]);
    }
    const uint32_t n = NR > 0 ? (uint32_t)NR : a.nranks;
    for (uint32_t k = 1; k < n; ++k) {
        const u32x4 x = load_partial<TB>(make_rsrc(a.src[k], a.extent), off);
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w].add(x[w]);
    }
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) out[w] = acc[w].get();
    if constexpr (SM == kStoreAll) {
        for (uint32_t k = 0; k < n; ++k)
            store_partial<TB, kStoreAllPolicy>(make_rsrc(a.src[k], a.extent), off, out);
    } else if constexpr (SM == kStoreAdd) {
        // whole words, then a lone 16-bit element (the low half of its word)
        char* const p = static_cast<char*>(a.dst) + off;
#pragma unroll
        for (int e = 0; e + 4 <= TB; e += 4) atomic_add_word<DT>(p + e, out[e / 4]);
        if constexpr (TB % 4 == 2)
            atomic_add_elem<DT, ES>(p + (TB - 2), out[(TB - 2) / 4] & 0xFFFFu);
    } else {
        store_partial<TB, store_policy_for(NR)>(rd, off, out);
    }
}

// One row head: bytes [LO, 16) of the slot at `off`, loaded from every
// source with the pieces of load_head, folded word-wise in the same order
// as the main tiles (the zero bytes before LO fold among themselves and are
// never stored), stored with the same pieces.
template <int DT, int OP, int ES, int NR, int LO, int SM>
__device__ __forceinline__ void row_head(const KArgs& a, uint32_t off) {
    Acc<DT, OP> acc[4];
    {
        const u32x4 x0 = load_head<LO>(make_rsrc(a.src[0], a.extent), off);
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w].init(x0[w]);
    }
    const uint32_t n = NR > 0 ? (uint32_t)NR : a.nranks;
    for (uint32_t k = 1; k < n; ++k) {
        const u32x4 x = load_head<LO>(make_rsrc(a.src[k], a.extent), off);
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w].add(x[w]);
    }
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) out[w] = acc[w].get();
    if constexpr (SM == kStoreAll) {
        for (uint32_t k = 0; k < n; ++k)
            store_head<LO, kStoreAllPolicy>(make_rsrc(a.src[k], a.extent), off, out);
    } else if constexpr (SM == kStoreAdd) {
        // a lone 16-bit element at LO (the high half of its word), then whole words
        char* const p = static_cast<char*>(a.dst) + off;
        constexpr int A = (LO + 3) / 4 * 4;
        if constexpr (LO % 4 == 2) atomic_add_elem<DT, ES>(p + LO, out[LO / 4] >> 16);
#pragma unroll
        for (int e = A; e < 16; e += 4) atomic_add_word<DT>(p + e, out[e / 4]);
    } else {
        store_head<LO, store_policy_for(NR)>(make_rsrc(a.dst, a.extent), off, out);
    }
}

// One tail tile of the vector path: kBlock items, one per thread -- row
// remainders (items [0, ntail)), row heads (the next nhead), then spill
// slots (the next nspill): the last few whole slots of every row when they
// would fill less than half of a row tile of their own, so each lane folds
// one slot of a different row instead of most lanes of a tile idling.
template <int DT, int OP, int ES, int NR, int SM>
__device__ __forceinline__ void row_tail_tile(const KArgs& a, uint32_t t) {
    const uint32_t q = t * (uint32_t)kBlock + threadIdx.x;
    if (q >= a.ntail) {
        const uint32_t h = q - a.ntail;
        if (h >= a.nhead) {
            const uint32_t k = h - a.nhead;
            if (k >= a.nspill) return;
            const uint32_t row = fast_div(k, a.div_spill);
            const uint32_t v = a.spill_v0 + (k - row * a.spill_per_row);
            const uint32_t off[1] = {row * a.ld_bytes + v * 16u};
            u32x4 out[1];
            fold_slots<DT, OP, NR, 1>([&](uint32_t r) { return make_rsrc(a.src[r], a.extent); },
                                      a.nranks, off, out);
            store_result<DT, SM, NR>(a, make_rsrc(a.dst, a.extent), off[0], out[0]);
            return;
        }
        const uint32_t off = h * a.ld_bytes + a.head_off;
        switch (a.head_lo) {  // uniform over the launch
        case 2: if constexpr (ES == 2) row_head<DT, OP, ES, NR, 2, SM>(a, off); break;
        case 4: row_head<DT, OP, ES, NR, 4, SM>(a, off); break;
        case 6: if constexpr (ES == 2) row_head<DT, OP, ES, NR, 6, SM>(a, off); break;
        case 8: row_head<DT, OP, ES, NR, 8, SM>(a, off); break;
        case 10: if constexpr (ES == 2) row_head<DT, OP, ES, NR, 10, SM>(a, off); break;
        case 12: row_head<DT, OP, ES, NR, 12, SM>(a, off); break;
        case 14: if constexpr (ES == 2) row_head<DT, OP, ES, NR, 14, SM>(a, off); break;
        default: break;
        }
        return;
    }
    const uint32_t off = q * a.ld_bytes + a.tail_col_bytes;
    switch (a.tail_bytes) {  // uniform over the launch
    case 2: if constexpr (ES == 2) row_tail<DT, OP, ES, NR, 2, SM>(a, off); break;
    case 4: row_tail<DT, OP, ES, NR, 4, SM>(a, off); break;
    case 6: if constexpr (ES == 2) row_tail<DT, OP, ES, NR, 6, SM>(a, off); break;
    case 8: row_tail<DT, OP, ES, NR, 8, SM>(a, off); break;
    case 10: if constexpr (ES == 2) row_tail<DT, OP, ES, NR, 10, SM>(a, off); break;
    case 12: row_tail<DT, OP, ES, NR, 12, SM>(a, off); break;
    case 14: if constexpr (ES == 2) row_tail<DT, OP, ES, NR, 14, SM>(a, off); break;
    default: break;
    }
}

// One tile of the reduction kernel: a main tile of 16-byte slots, or a tail
// tile (row remainders, heads, spill slots); element tiles without VEC.
template <int DT, int OP, int ES, int NR, int U, int WALK, bool VEC, int SM>
__device__ __forceinline__ void any_tile(const KArgs& a, uint32_t t) {
    if constexpr (VEC) {
        const uint32_t tails = a.total_tiles - a.main_tiles;
        if (t >= tails) {
            main_tile<DT, OP, NR, U, WALK, SM>(a, t - tails);
        } else {
            row_tail_tile<DT, OP, ES, NR, SM>(a, t);
        }
    } else {
        element_tile<DT, OP, ES, NR, WALK, SM>(a, t);
    }
}

// The reduction kernel.  The first total_tiles - main_tiles tiles are tail
// tiles (row remainders), the rest main tiles: issued first, the scattered
// remainder accesses overlap the main tiles' streaming instead of forming a
// serial phase at the end (measured 3-4% on ragged rows).  Block b takes
// tiles b, b + G, ... (one tile per block when G equals the tile count).
// The host launches at most one block per tile and never a launch without
// tiles, so every block's first tile exists: it is taken without a check,
// which lets the compiler issue every load of the kernel arguments the tile
// needs in one batch (with the check in front, the source pointers came in
// a second round after it; measured 3-5% off the kernel time of 1-20 MB
// calls, level on large ones).
// NR == 0: runtime rank count.  VEC: 16-byte main tiles with row-remainder
// and row-head tail tiles; otherwise element tiles only.
// WALK: kWalkContig, kWalkRowTiles or kWalkFlat.  SM: the StoreMode --
// into dst, into every source buffer (in-place allreduce), or added into
// dst with atomics (push-with-add, Sum only).
template <int DT, int OP, int ES, int NR, int U, int WALK, bool VEC, int SM>
__global__ __launch_bounds__(kBlock) void treduce_kernel(const KArgs a) {
    const uint32_t grid = gridDim.x;
    uint32_t t = logical_block(blockIdx.x, grid, a.xcd_remap != 0u);
    do {
        any_tile<DT, OP, ES, NR, U, WALK, VEC, SM>(a, t);
        t += grid;
    } while (t < a.total_tiles);
}

// The LDS ping-pong kernel: main tiles through LDS stages (one slot per
// thread, any walk), tail tiles (first) as in treduce_kernel.  Runtime rank
// count.
template <int DT, int OP, int ES, int WALK, int S>
__global__ __launch_bounds__(kBlock) void treduce_lds_kernel(const KArgs a) {
    __shared__ LdsStages<S> stages;
    const uint32_t grid = gridDim.x;
    for (uint32_t t = logical_block(blockIdx.x, grid, a.xcd_remap != 0u); t < a.total_tiles;
         t += grid) {
        const uint32_t tails = a.total_tiles - a.main_tiles;
        if (t >= tails) {
            main_tile_lds<DT, OP, S, WALK>(a, t - tails, stages);
        } else {
            row_tail_tile<DT, OP, ES, 0, kStoreDst>(a, t);
        }
    }
}

}  // namespace ptored
