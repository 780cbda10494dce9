// treduce_launch.cuh -- kernel selection for one element type.
//
// Included once per element type (treduce_<type>.hip) so the four types
// compile in parallel.  Maps a Plan onto one template instance: the rank
// count N is a compile-time constant for 1 <= N <= 16 (fully unrolled
// loads), larger or forced counts take the runtime rank loop.
#pragma once

#include "treduce_kernels.cuh"

namespace ptored {

// Launch KERNEL over a.ntiles tiles.  The persistent grid holds as many
// blocks as the GPU keeps resident at once for this kernel (occupancy per CU
// times the CU count), so every block is live for the whole sweep and none
// waits for a free slot while others run: a grid larger than that would
// leave a second, partial wave of blocks at the end.  blocks_per_cu > 0
// overrides the occupancy; < 0 launches one block per tile.
template <auto KERNEL>
static void launch(const Plan& p, const KArgs& a, int cu_count, hipStream_t s) {
    static const int occupancy = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERNEL, kBlock, 0) != hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    uint64_t grid;
    if (p.blocks_per_cu < 0) {
        grid = a.ntiles;
    } else {
        const int per_cu = p.blocks_per_cu > 0 ? p.blocks_per_cu : occupancy;
        grid = (uint64_t)cu_count * (uint64_t)per_cu;
        if (grid > a.ntiles) grid = a.ntiles;
    }
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(KERNEL, dim3((uint32_t)grid), dim3(kBlock), 0, s, a);
}

template <int DT, int OP, int ES, int NR, bool ROWS, bool NT>
static void launch_fixed_n(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    constexpr int U = unroll_for(NR);
    launch<treduce_vec_kernel<DT, OP, ES, NR, U, ROWS, NT>>(p, a, cu, s);
}

template <int DT, int OP, int ES, bool ROWS, bool NT>
static int dispatch_fixed(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    switch (p.nranks) {
#define PTORED_CASE(n) \
    case n: launch_fixed_n<DT, OP, ES, n, ROWS, NT>(p, a, cu, s); return 0;
        PTORED_CASE(2) PTORED_CASE(3) PTORED_CASE(4) PTORED_CASE(5) PTORED_CASE(6)
        PTORED_CASE(7) PTORED_CASE(8) PTORED_CASE(9) PTORED_CASE(10) PTORED_CASE(11)
        PTORED_CASE(12) PTORED_CASE(13) PTORED_CASE(14) PTORED_CASE(15) PTORED_CASE(16)
#undef PTORED_CASE
    default: return -1;
    }
}

template <int DT, int OP, int ES>
static int dispatch_op(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    const bool rows = p.rows_mode != 0;
    constexpr int RU = kRuntimeUnroll;
    switch (p.family) {
    case kFamVecFixed:
        if (rows)
            return p.nt_loads ? dispatch_fixed<DT, OP, ES, true, true>(p, a, cu, s)
                              : dispatch_fixed<DT, OP, ES, true, false>(p, a, cu, s);
        return p.nt_loads ? dispatch_fixed<DT, OP, ES, false, true>(p, a, cu, s)
                          : dispatch_fixed<DT, OP, ES, false, false>(p, a, cu, s);
    case kFamVecRuntime:
        if (rows) {
            if (p.nt_loads) launch<treduce_vec_kernel<DT, OP, ES, 0, RU, true, true>>(p, a, cu, s);
            else launch<treduce_vec_kernel<DT, OP, ES, 0, RU, true, false>>(p, a, cu, s);
        } else {
            if (p.nt_loads) launch<treduce_vec_kernel<DT, OP, ES, 0, RU, false, true>>(p, a, cu, s);
            else launch<treduce_vec_kernel<DT, OP, ES, 0, RU, false, false>>(p, a, cu, s);
        }
        return 0;
    case kFamElem:
        if (rows) launch<treduce_elem_kernel<DT, OP, ES, true>>(p, a, cu, s);
        else launch<treduce_elem_kernel<DT, OP, ES, false>>(p, a, cu, s);
        return 0;
    default: return -1;
    }
}

// N == 1: a bitwise copy through the fixed kernel with one source (the
// accumulator only passes the bits through).
template <int DT, int ES>
static int dispatch_copy(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    constexpr int U = unroll_for(1);
    if (p.rows_mode) launch<treduce_vec_kernel<DT, PTORED_SUM, ES, 1, U, true, false>>(p, a, cu, s);
    else launch<treduce_vec_kernel<DT, PTORED_SUM, ES, 1, U, false, false>>(p, a, cu, s);
    return 0;
}

template <int DT, int ES>
static int dispatch_dtype(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    if (p.family == kFamCopy) return dispatch_copy<DT, ES>(p, a, cu, s);
    switch (p.op) {
    case PTORED_SUM: return dispatch_op<DT, PTORED_SUM, ES>(p, a, cu, s);
    case PTORED_MAX: return dispatch_op<DT, PTORED_MAX, ES>(p, a, cu, s);
    case PTORED_MIN: return dispatch_op<DT, PTORED_MIN, ES>(p, a, cu, s);
    case PTORED_PROD: return dispatch_op<DT, PTORED_PROD, ES>(p, a, cu, s);
    default: return -1;
    }
}

}  // namespace ptored
