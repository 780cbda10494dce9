// treduce_launch.hpp -- kernel selection.
//
// Maps a Plan onto one template instance: the rank count N is a
// compile-time constant for 1 <= N <= 16 (fully unrolled loads); larger or
// forced counts and the element-wise path take the runtime rank loop.  The
// reduction and ring kernels of each (element type, operator) pair are
// instantiated in a translation unit of their own (treduce_op.hip, built
// once per pair) and the copy and push-with-add kernels in one per element
// type (treduce_<type>.hip), so the units compile in parallel.
#pragma once

#include "accumulate_kernels.hpp"
#include "ring_kernels.hpp"
#include "treduce_kernels.hpp"

namespace ptored {

// Launch KERNEL over `tiles` tiles.  Default (blocks_per_cu == 0): one
// block per tile, so the dispatcher hands tiles out in order to whichever
// CU frees up first -- on MI355X this beat every persistent grid size
// measured -- with p.wgs_per_cu blocks resident per CU: each block reserves
// p.cap_lds bytes of LDS (its own static LDS included), which it does not
// use, so that no more fit.  blocks_per_cu > 0: a persistent grid of that
// many blocks per CU; blocks_per_cu < 0: a persistent grid at the kernel's
// occupancy.
template <auto KERNEL, class ARGS>
static int launch_grid(const Plan& p, const ARGS& a, uint64_t tiles, int cu_count,
                       hipStream_t s) {
    if (tiles == 0) return kLaunchOk;  // nothing to do: every launched block has a tile
    uint64_t grid = tiles;
    if (p.blocks_per_cu != 0) {
        int per_cu = p.blocks_per_cu;
        if (per_cu < 0) {
            static const int occupancy = [] {
                int n = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERNEL, kBlock, 0) !=
                        hipSuccess ||
                    n < 1)
                    n = 1;
                return n;
            }();
            per_cu = occupancy;
        }
        const uint64_t cap = (uint64_t)cu_count * (uint64_t)per_cu;
        if (grid > cap) grid = cap;
    }
    uint32_t shmem = 0;
    if (p.cap_lds > 0 && tiles >= p.cap_min_tiles) {
        // the kernel's own static LDS counts toward the reservation; when it
        // cannot be read, the launch goes without the limit
        static const int64_t static_lds = [] {
            hipFuncAttributes at{};
            return hipFuncGetAttributes(&at, reinterpret_cast<const void*>(KERNEL)) == hipSuccess
                       ? (int64_t)at.sharedSizeBytes
                       : int64_t(-1);
        }();
        if (static_lds >= 0 && (int64_t)p.cap_lds > static_lds)
            shmem = p.cap_lds - (uint32_t)static_lds;
    }
    // the launch's own status: the caller's last-error state is left alone
    void* args[] = {const_cast<ARGS*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(KERNEL), dim3((uint32_t)grid),
                           dim3(kBlock), args, shmem, s) == hipSuccess
               ? kLaunchOk
               : kLaunchFailed;
}

template <auto KERNEL>
static int launch(const Plan& p, const KArgs& a, int cu_count, hipStream_t s) {
    return launch_grid<KERNEL>(p, a, a.total_tiles, cu_count, s);
}

template <int DT, int OP, int ES, int WALK, int SM>
static int dispatch_n(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    if (p.family == kFamElem) {
        if constexpr (WALK == kWalkRowTiles) {
            return kLaunchNoKernel;  // the element-wise path never takes row tiles
        } else {
            return launch<treduce_kernel<DT, OP, ES, 0, 1, WALK, false, SM>>(p, a, cu, s);
        }
    }
    if constexpr (SM == kStoreAdd) {  // push-with-add of a single source
        if (p.family == kFamVecFixed && p.nranks == 1)
            return launch<treduce_kernel<DT, OP, ES, 1, unroll_for(1), WALK, true, SM>>(p, a, cu,
                                                                                     s);
    }
    switch (p.family == kFamVecFixed ? p.nranks : 0) {
#define PTORED_CASE(n) \
    case n: return launch<treduce_kernel<DT, OP, ES, n, unroll_for(n), WALK, true, SM>>(p, a, cu, s);
        PTORED_CASE(2) PTORED_CASE(3) PTORED_CASE(4) PTORED_CASE(5) PTORED_CASE(6)
        PTORED_CASE(7) PTORED_CASE(8) PTORED_CASE(9) PTORED_CASE(10) PTORED_CASE(11)
        PTORED_CASE(12) PTORED_CASE(13) PTORED_CASE(14) PTORED_CASE(15) PTORED_CASE(16)
#undef PTORED_CASE
    case 0:
        return launch<treduce_kernel<DT, OP, ES, 0, kRuntimeUnroll, WALK, true, SM>>(p, a, cu, s);
    default: return kLaunchNoKernel;
    }
}

template <int DT, int OP, int ES>
static int dispatch_op(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    if (p.store_all) {  // in-place allreduce
        switch (p.rows_mode) {
        case kWalkContig: return dispatch_n<DT, OP, ES, kWalkContig, kStoreAll>(p, a, cu, s);
        case kWalkRowTiles: return dispatch_n<DT, OP, ES, kWalkRowTiles, kStoreAll>(p, a, cu, s);
        case kWalkFlat: return dispatch_n<DT, OP, ES, kWalkFlat, kStoreAll>(p, a, cu, s);
        default: return kLaunchNoKernel;
        }
    }
    if (p.lds_stages) {  // LDS ping-pong variant
        switch (p.rows_mode) {
        case kWalkContig:
            return launch<treduce_lds_kernel<DT, OP, ES, kWalkContig, kLdsStages>>(p, a, cu, s);
        case kWalkRowTiles:
            return launch<treduce_lds_kernel<DT, OP, ES, kWalkRowTiles, kLdsStages>>(p, a, cu,
                                                                                   s);
        case kWalkFlat:
            return launch<treduce_lds_kernel<DT, OP, ES, kWalkFlat, kLdsStages>>(p, a, cu, s);
        default: return kLaunchNoKernel;
        }
    }
    switch (p.rows_mode) {
    case kWalkContig: return dispatch_n<DT, OP, ES, kWalkContig, kStoreDst>(p, a, cu, s);
    case kWalkRowTiles: return dispatch_n<DT, OP, ES, kWalkRowTiles, kStoreDst>(p, a, cu, s);
    default: return dispatch_n<DT, OP, ES, kWalkFlat, kStoreDst>(p, a, cu, s);
    }
}

// Push-with-add, default: the reduction kernel folds the call's sources and
// adds the fold into dst (StoreMode kStoreAdd).
template <int DT, int ES>
static int dispatch_push(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    switch (p.rows_mode) {
    case kWalkContig: return dispatch_n<DT, PTORED_SUM, ES, kWalkContig, kStoreAdd>(p, a, cu, s);
    case kWalkRowTiles:
        return dispatch_n<DT, PTORED_SUM, ES, kWalkRowTiles, kStoreAdd>(p, a, cu, s);
    case kWalkFlat: return dispatch_n<DT, PTORED_SUM, ES, kWalkFlat, kStoreAdd>(p, a, cu, s);
    default: return kLaunchNoKernel;
    }
}

// Push-with-add per rank: a 2-D grid, one row of workgroups per rank.
template <int DT, int ES, int WALK, bool VEC>
static int launch_accumulate(const KArgs& a, hipStream_t s) {
    void* args[] = {const_cast<KArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(accumulate_kernel<DT, ES, WALK, VEC>),
                           dim3(a.total_tiles > 0 ? a.total_tiles : 1, a.nranks), dim3(kBlock),
                           args, 0, s) == hipSuccess
               ? kLaunchOk
               : kLaunchFailed;
}

template <int DT, int ES>
static int dispatch_accumulate(const Plan& p, const KArgs& a, hipStream_t s) {
    const bool vec = p.family != kFamElem;
    switch (p.rows_mode) {
    case kWalkContig:
        return vec ? launch_accumulate<DT, ES, kWalkContig, true>(a, s)
                   : launch_accumulate<DT, ES, kWalkContig, false>(a, s);
    case kWalkFlat:
        return vec ? launch_accumulate<DT, ES, kWalkFlat, true>(a, s)
                   : launch_accumulate<DT, ES, kWalkFlat, false>(a, s);
    case kWalkRowTiles:  // the element-wise path never takes row tiles
        return vec ? launch_accumulate<DT, ES, kWalkRowTiles, true>(a, s) : kLaunchNoKernel;
    default: return kLaunchNoKernel;
    }
}

// N == 1: a bitwise copy through the kernel with one source (the
// accumulator only passes the bits through).
template <int DT, int ES>
static int dispatch_copy(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    constexpr int U = unroll_for(1);
    switch (p.rows_mode) {
    case kWalkContig:
        return launch<treduce_kernel<DT, PTORED_SUM, ES, 1, U, kWalkContig, true, kStoreDst>>(
            p, a, cu, s);
    case kWalkRowTiles:
        return launch<treduce_kernel<DT, PTORED_SUM, ES, 1, U, kWalkRowTiles, true, kStoreDst>>(
            p, a, cu, s);
    default:
        return launch<treduce_kernel<DT, PTORED_SUM, ES, 1, U, kWalkFlat, true, kStoreDst>>(
            p, a, cu, s);
    }
}

// The single-launch ring reduce-scatter: N unrolled for 2 <= N <= 16.
template <int DT, int OP, int ES>
static int dispatch_ring_n(const Plan& p, const RingArgs& a, int cu, hipStream_t s) {
    const uint64_t tiles = (uint64_t)a.nseg * a.tiles_per_seg;
    switch (p.family == kFamVecFixed ? p.nranks : 0) {
#define PTORED_CASE(n) \
    case n: return launch_grid<ring_kernel<DT, OP, ES, n>>(p, a, tiles, cu, s);
        PTORED_CASE(2) PTORED_CASE(3) PTORED_CASE(4) PTORED_CASE(5) PTORED_CASE(6)
        PTORED_CASE(7) PTORED_CASE(8) PTORED_CASE(9) PTORED_CASE(10) PTORED_CASE(11)
        PTORED_CASE(12) PTORED_CASE(13) PTORED_CASE(14) PTORED_CASE(15) PTORED_CASE(16)
#undef PTORED_CASE
    case 0:
        return launch_grid<ring_kernel<DT, OP, ES, 0>>(p, a, tiles, cu, s);
    default: return kLaunchNoKernel;
    }
}

// The reduction and ring launchers of one (element type, operator) pair,
// defined and explicitly instantiated in treduce_op.hip.
template <int DT, int OP>
int launch_op(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);
template <int DT, int OP>
int launch_ring_op(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream);

template <int DT>
static int dispatch_ring(const Plan& p, const RingArgs& a, int cu, hipStream_t s) {
    switch (p.op) {
    case PTORED_SUM: return launch_ring_op<DT, PTORED_SUM>(p, a, cu, s);
    case PTORED_MAX: return launch_ring_op<DT, PTORED_MAX>(p, a, cu, s);
    case PTORED_MIN: return launch_ring_op<DT, PTORED_MIN>(p, a, cu, s);
    case PTORED_PROD: return launch_ring_op<DT, PTORED_PROD>(p, a, cu, s);
    default: return kLaunchNoKernel;
    }
}

template <int DT, int ES>
static int dispatch_dtype(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    if (p.accumulate)
        return p.push_per_rank ? dispatch_accumulate<DT, ES>(p, a, s)
                               : dispatch_push<DT, ES>(p, a, cu, s);
    if (p.family == kFamCopy) return dispatch_copy<DT, ES>(p, a, cu, s);
    switch (p.op) {
    case PTORED_SUM: return launch_op<DT, PTORED_SUM>(p, a, cu, s);
    case PTORED_MAX: return launch_op<DT, PTORED_MAX>(p, a, cu, s);
    case PTORED_MIN: return launch_op<DT, PTORED_MIN>(p, a, cu, s);
    case PTORED_PROD: return launch_op<DT, PTORED_PROD>(p, a, cu, s);
    default: return kLaunchNoKernel;
    }
}

}  // namespace ptored
