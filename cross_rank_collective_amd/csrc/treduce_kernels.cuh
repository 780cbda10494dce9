// treduce_kernels.cuh -- gfx950 kernels of the N-way reduction.
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
// one element on the element-wise path).  Row i holds nvec_row slots; the
// last one is partial when valid_cols is not a multiple of VEC and then
// carries only `tail` valid elements -- the analog of the pages' partial
// column chunk with a dynamic valid extent.  Slots are numbered row-major.
// A tile is BLOCK * U consecutive slots, and block b takes tiles b, b+G,
// b+2G, ... of a persistent grid of G blocks (the pages' block-cyclic walk).
// Within a tile, thread t owns slots t, t+BLOCK, ..., so every wave
// instruction moves 64 adjacent 16-byte vectors (1 KiB) of one buffer.
//
// Per slot a thread issues the loads of all N sources before it combines
// anything -- the many waves in flight on a CU take the place of the pages'
// ping-pong recv tiles -- then folds them in the fixed order (root first,
// then ascending rank; the host passes the pointers already in that order),
// rounding to the element type after every step, and stores the result with
// a non-temporal store.  Elements outside the valid rectangle are never read
// or written.
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

#define PTORED_GLOBAL __attribute__((address_space(1)))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;

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
// Memory access helpers (global address space, 32-bit byte offsets so the
// loads use one offset VGPR against each source's SGPR base).
// ------------------------------------------------------------------------

template <bool NT>
__device__ __forceinline__ u32x4 load16(const void* base, uint32_t off) {
    const PTORED_GLOBAL u32x4* p =
        (const PTORED_GLOBAL u32x4*)((const PTORED_GLOBAL char*)base + off);
    if constexpr (NT) {
        return __builtin_nontemporal_load(p);
    } else {
        return *p;
    }
}
__device__ __forceinline__ void store16(void* base, uint32_t off, u32x4 v) {
    PTORED_GLOBAL u32x4* p = (PTORED_GLOBAL u32x4*)((PTORED_GLOBAL char*)base + off);
    __builtin_nontemporal_store(v, p);
}
// One element of ES bytes, zero-extended into a word.
template <int ES>
__device__ __forceinline__ uint32_t load_elem(const void* base, uint32_t off) {
    if constexpr (ES == 4) {
        return *(const PTORED_GLOBAL uint32_t*)((const PTORED_GLOBAL char*)base + off);
    } else {
        return *(const PTORED_GLOBAL uint16_t*)((const PTORED_GLOBAL char*)base + off);
    }
}
template <int ES>
__device__ __forceinline__ void store_elem(void* base, uint32_t off, uint32_t v) {
    if constexpr (ES == 4) {
        *(PTORED_GLOBAL uint32_t*)((PTORED_GLOBAL char*)base + off) = v;
    } else {
        *(PTORED_GLOBAL uint16_t*)((PTORED_GLOBAL char*)base + off) = (uint16_t)v;
    }
}

// Quotient by the slots-per-row count without a divide: the multiply-high
// method of Granlund and Montgomery ("Division by invariant integers using
// multiplication", PLDI 1994, Fig. 4.1), exact for every 32-bit dividend.
__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& d) {
    const uint32_t t = __umulhi(n, d.mul);
    return (t + ((n - t) >> d.sh1)) >> d.sh2;
}

// Block index remapped so that the blocks the hardware places on one XCD
// (it deals consecutive workgroups round-robin over the 8 XCDs) get one
// contiguous range of logical indices: each XCD then sweeps its own band of
// every grid-stride pass instead of every eighth tile.
__device__ __forceinline__ uint32_t logical_block(uint32_t b, uint32_t grid, bool remap) {
    if (!remap || (grid & 7u) != 0u) return b;
    return (b & 7u) * (grid >> 3) + (b >> 3);
}

// Byte offset and valid element count of slot s.
template <bool ROWS, int VEC, int ES>
__device__ __forceinline__ void slot_geometry(const KArgs& a, uint32_t s, uint32_t& off,
                                              uint32_t& cnt) {
    if (s >= a.nslots) {
        off = 0;
        cnt = 0;
        return;
    }
    if constexpr (ROWS) {
        const uint32_t row = fast_div(s, a.div_row);
        const uint32_t v = s - row * a.nvec_row;
        off = row * a.ld_bytes + v * (uint32_t)(VEC * ES);
        cnt = (v + 1u == a.nvec_row) ? a.tail : (uint32_t)VEC;
    } else {
        off = s * (uint32_t)(VEC * ES);
        cnt = (s + 1u == a.nslots) ? a.tail : (uint32_t)VEC;
    }
}

// Fold all ranks of one element (partial-slot path and element-wise
// kernels): the same order and combine as the vector path, one lane.
template <int DT, int OP, int ES>
__device__ __forceinline__ void reduce_one_element(const KArgs& a, uint32_t off) {
    Acc<DT, OP> acc;
    acc.init(load_elem<ES>(a.src[0], off));
    for (uint32_t k = 1; k < a.nranks; ++k) acc.add(load_elem<ES>(a.src[k], off));
    store_elem<ES>(a.dst, off, acc.get());
}

// Fold of NR sources (compile-time count) for U full 16-byte slots.
template <int DT, int OP, int NR, int U, bool NT>
__device__ __forceinline__ void reduce_vec_fixed(const KArgs& a, const uint32_t (&off)[U]) {
    u32x4 x[NR][U];
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) x[k][u] = load16<NT>(a.src[k], off[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            Acc<DT, OP> acc;
            acc.init(x[0][u][w]);
            int k = 1;
#pragma unroll
            for (; k + 1 < NR; k += 2) acc.add2(x[k][u][w], x[k + 1][u][w]);
            if constexpr ((NR - 1) % 2 == 1) acc.add(x[NR - 1][u][w]);
            out[w] = acc.get();
        }
        store16(a.dst, off[u], out);
    }
}

// Fold of a runtime number of sources for one full 16-byte slot: groups of
// four loads in flight, then the remainder one by one, in rank order.
template <int DT, int OP, bool NT>
__device__ __forceinline__ void reduce_vec_runtime(const KArgs& a, uint32_t off) {
    Acc<DT, OP> acc[4];
    {
        const u32x4 x0 = load16<NT>(a.src[0], off);
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w].init(x0[w]);
    }
    uint32_t k = 1;
    for (; k + 4 <= a.nranks; k += 4) {
        u32x4 x[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) x[g] = load16<NT>(a.src[k + g], off);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc[w].add2(x[0][w], x[1][w]);
            acc[w].add2(x[2][w], x[3][w]);
        }
    }
    for (; k < a.nranks; ++k) {
        const u32x4 x = load16<NT>(a.src[k], off);
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w].add(x[w]);
    }
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) out[w] = acc[w].get();
    store16(a.dst, off, out);
}

// Vector kernel: 16-byte slots, NR sources (NR == 0: runtime count).
// ES = element size in bytes, U = slots per thread per tile.
template <int DT, int OP, int ES, int NR, int U, bool ROWS, bool NT>
__global__ __launch_bounds__(kBlock) void treduce_vec_kernel(const KArgs a) {
    constexpr int VEC = 16 / ES;
    const uint32_t grid = gridDim.x;
    const uint32_t lb = logical_block(blockIdx.x, grid, a.xcd_remap != 0u);
    for (uint32_t tile = lb; tile < a.ntiles; tile += grid) {
        const uint32_t s0 = tile * (uint32_t)(kBlock * U) + threadIdx.x;
        uint32_t off[U], cnt[U];
        bool full = true;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            slot_geometry<ROWS, VEC, ES>(a, s0 + (uint32_t)(u * kBlock), off[u], cnt[u]);
            full = full && (cnt[u] == (uint32_t)VEC);
        }
        if (full) {
            if constexpr (NR > 0) {
                reduce_vec_fixed<DT, OP, NR, U, NT>(a, off);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) reduce_vec_runtime<DT, OP, NT>(a, off[u]);
            }
        } else {
            // Ragged edge: the end of the stream or the partial last slot
            // of a row.  Full slots still go 16 bytes at a time; a partial
            // slot goes element by element over its valid elements only.
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (cnt[u] == (uint32_t)VEC) {
                    if constexpr (NR > 0) {
                        const uint32_t one[1] = {off[u]};
                        reduce_vec_fixed<DT, OP, NR, 1, NT>(a, one);
                    } else {
                        reduce_vec_runtime<DT, OP, NT>(a, off[u]);
                    }
                } else {
                    for (uint32_t e = 0; e < cnt[u]; ++e)
                        reduce_one_element<DT, OP, ES>(a, off[u] + e * (uint32_t)ES);
                }
            }
        }
    }
}

// Element-wise kernel for data that is not 16-byte aligned: one element per
// slot, runtime rank count.  U slots per thread per tile.
template <int DT, int OP, int ES, bool ROWS>
__global__ __launch_bounds__(kBlock) void treduce_elem_kernel(const KArgs a) {
    constexpr int U = kElemUnroll;
    const uint32_t grid = gridDim.x;
    const uint32_t lb = logical_block(blockIdx.x, grid, a.xcd_remap != 0u);
    for (uint32_t tile = lb; tile < a.ntiles; tile += grid) {
        const uint32_t s0 = tile * (uint32_t)(kBlock * U) + threadIdx.x;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            uint32_t off, cnt;
            slot_geometry<ROWS, 1, ES>(a, s0 + (uint32_t)(u * kBlock), off, cnt);
            if (cnt) reduce_one_element<DT, OP, ES>(a, off);
        }
    }
}

}  // namespace ptored
