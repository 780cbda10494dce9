// treduce_plan.h -- launch plan shared by the host dispatcher and the kernels.
//
// The host turns one ptored_treduce call into one or more launches of one
// kernel family ("CANN PTO-ISA TREDUCE instruction explained" §4.1: empty
// short-circuit, single-tile path or chunked walk; here: nothing, an N == 1
// copy, the 16-byte vector kernel or the element-wise kernel).
#pragma once

#include <stdint.h>

#include "ptored.h"

namespace ptored {

// Divisor d with its Granlund-Montgomery multiplier: q = (t + ((n - t) >> sh1)) >> sh2,
// t = mulhi(n, mul).
struct FastDiv {
    uint32_t mul;
    uint32_t sh1;
    uint32_t sh2;
};

// Kernel arguments of one launch (passed by value; ~600 bytes of kernarg).
struct KArgs {
    // src[0] is the root's buffer, then the other ranks in ascending order:
    // the kernels fold src[0], src[1], ... in index order.
    const void* src[PTORED_MAX_RANKS];
    void* dst;
    uint32_t nranks;
    uint32_t ntiles;    // tiles of kBlock * U slots
    uint32_t nslots;    // slots in this launch
    uint32_t nvec_row;  // slots per row (row walk)
    uint32_t ld_bytes;  // row pitch in bytes (row walk)
    uint32_t tail;      // valid elements of the last slot of a row / of the stream
    FastDiv div_row;    // division by nvec_row
    uint32_t xcd_remap; // 1: per-XCD contiguous tile bands
};

// Kernel families.
enum Family : int {
    kFamNone = PTORED_PATH_NONE,
    kFamCopy = PTORED_PATH_COPY,
    kFamVecFixed = PTORED_PATH_VEC_FIXED,
    kFamVecRuntime = PTORED_PATH_VEC_RUNTIME,
    kFamElem = PTORED_PATH_ELEMENTWISE,
};

// One kernel selection plus the geometry that every launch of a call shares.
struct Plan {
    int family;
    int dtype;
    int op;
    int nranks;
    int esize;
    int rows_mode;      // 1: 2-D row walk, 0: one contiguous span
    int vec_elems;      // elements per slot
    int unroll;         // slots per thread per tile
    bool nt_loads;
    bool xcd_remap;
    int blocks_per_cu;
    // geometry of the whole call
    int64_t valid_rows;
    int64_t valid_cols;
    int64_t ld;          // elements
    int64_t total_elems; // contiguous mode: elements of the span
    int64_t slots;       // whole call
    int64_t max_launch_bytes;
    int64_t launches;
};

// Unroll (slots per thread per tile) of the fixed-N vector kernel: enough
// 16-byte loads in flight per thread (N * U of them) to cover HBM latency,
// without exhausting VGPRs at large N.
constexpr int unroll_for(int nranks) {
    return nranks <= 2 ? 4 : (nranks <= 4 ? 4 : (nranks <= 8 ? 2 : 1));
}
constexpr int kElemUnroll = 4;
constexpr int kRuntimeUnroll = 2;

// Launch one kernel of the plan's family on `a`, on a persistent grid sized
// for `cu_count` compute units.
// Defined per element type in the kernel translation units.
int launch_f32(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);
int launch_bf16(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);
int launch_f16(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);
int launch_i32(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);

}  // namespace ptored
