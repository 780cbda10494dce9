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

// Kernel arguments of one launch (passed by value; ~630 bytes of kernarg).
// Offsets are bytes from each buffer's launch base.  On the vector path the
// base is the coarsest boundary below the data -- 1 KiB, a 128-byte line or
// 16 bytes -- at which every buffer starts at the same offset (and rows keep
// it): the 16-byte slots of a row (or span) are numbered from that boundary,
// the ones before the data are skipped, and a row that starts inside a slot
// begins with a head -- so every wave's 1 KiB run of slots is one aligned
// KiB, or at least whole cache lines.  With no common offset the base is
// dst's boundary (the sources' accesses unaligned), and with a pitch off the
// 16-byte grid each row's slots start at the row (every access unaligned).
struct KArgs {
    // src[0] is the root's buffer, then the other ranks in ascending order:
    // the kernels fold src[0], src[1], ... in index order.
    const void* src[PTORED_MAX_RANKS];
    void* dst;
    uint32_t nranks;
    uint32_t extent;         // bytes of every buffer this launch may touch (from its base)
    uint32_t main_tiles;     // tiles of full 16-byte slots
    uint32_t total_tiles;    // main tiles, then tail tiles of ragged elements
    uint32_t nslots;         // numbered 16-byte slots (the skipped ones included)
    uint32_t slots_per_row;  // numbered slots per row (row walk)
    uint32_t ld_bytes;       // row pitch in bytes (row walk)
    uint32_t ntail;          // tail items: row remainders (vector path) or elements
    uint32_t tail_per_row;   // elements per row (element-wise row walk)
    uint32_t tail_bytes;     // bytes of every row remainder (vector path), < 16
    uint32_t tail_col_bytes; // byte offset in a row (or the span) of the remainder
    uint32_t tiles_per_row;  // column chunks per row (row tiles)
    uint32_t slot_skip;      // numbered slots of a row (or the span) before its first full slot
    uint32_t nhead;          // head items: a row's bytes before its first full slot
    uint32_t head_off;       // byte offset in a row of the 16-byte block holding its head
    uint32_t head_lo;        // a head covers bytes [head_lo, 16) of that block
    uint32_t nspill;         // spill items: a row's last few slots, folded in tail tiles
    uint32_t spill_per_row;  // spill slots per row (row tiles)
    uint32_t spill_v0;       // numbered slot of a row's first spill slot
    FastDiv div_tiles;       // division by tiles_per_row
    FastDiv div_slots;       // division by slots_per_row
    FastDiv div_tail;        // division by tail_per_row
    FastDiv div_spill;       // division by spill_per_row
    uint32_t xcd_remap;      // 1: per-XCD contiguous tile bands (persistent grids)
};

// Kernel arguments of one launch of the single-launch ring reduce-scatter
// (~1.8 KB of kernarg): a window of the N streams, cut into the ring's
// segments.  Segment s is folded in the order of ranks s+1, s+2, ..., s
// (mod N) and written to dst[s].  The source table holds the N streams
// twice over, so that order is src[s + 1], ..., src[s + N] -- consecutive
// entries from a per-workgroup base, fetched by wide scalar loads.
struct RingArgs {
    const void* src[2 * PTORED_MAX_RANKS]; // src[r] = src[r + N] = rank r's stream
    void* dst[PTORED_MAX_RANKS];         // dst of segment s at the window start
    uint32_t bounds[PTORED_MAX_RANKS + 1]; // byte offset of segment s in the window (clipped)
    uint32_t nranks;
    uint32_t extent;         // bytes of the window
    uint32_t seg0;           // first segment of the launch
    uint32_t nseg;           // segments of the launch
    uint32_t tiles_per_seg;  // main tiles of the largest segment, + 1 with ragged ends
    uint32_t edge;           // 1: the last tile of every segment folds its ragged ends
    FastDiv div_seg;         // division by tiles_per_seg
    uint32_t xcd_remap;      // as KArgs::xcd_remap
};

// Walks of the valid rectangle (values of Plan::walk and ptored_plan_info.rows_mode).
enum Walk : int {
    kWalkContig = 0,    // one contiguous span
    kWalkRowTiles = 1,  // tile = (row, column chunk)
    kWalkFlat = 2,      // slots numbered straight through the rows
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
    int rows_mode;      // Walk
    int vec_elems;      // elements per slot
    int unroll;         // slots per thread per main tile
    bool xcd_remap;
    bool store_all;     // in-place allreduce: the result goes back into every source
    bool accumulate;    // push-with-add: dst += every source, by atomics
    bool push_per_rank; // push-with-add: one atomic per source element (else fold, then one)
    bool lds_stages;    // main tiles staged through LDS (ping-pong variant)
    int lead;           // vector path: bytes every buffer starts past a 16-byte boundary
    int blocks_per_cu;  // 0: one tile per block; > 0: persistent grid; < 0: at occupancy
    int wgs_per_cu;     // one tile per block: workgroups kept resident per CU (0 = no limit)
    uint32_t cap_lds;   // LDS bytes a workgroup reserves to hold that limit (0 = none)
    uint64_t cap_min_tiles; // launches with fewer tiles run without the limit
    // geometry of the whole call
    int64_t valid_rows;
    int64_t valid_cols;
    int64_t ld;          // elements
    int64_t total_elems; // contiguous mode: elements of the span
    int64_t slots;       // whole call
    int64_t max_launch_bytes;
    int64_t launches;
};

// Where a kernel puts a finished slot: into dst, back into every source
// (the in-place allreduce), or added into dst with device-scope atomics
// (push-with-add, after the call's sources are folded).
enum StoreMode : int {
    kStoreDst = 0,
    kStoreAll = 1,
    kStoreAdd = 2,
};

// Result of the per-type launch functions.
enum LaunchStatus : int {
    kLaunchOk = 0,         // the kernel was launched
    kLaunchNoKernel = -1,  // no kernel instance for this plan
    kLaunchFailed = -2,    // the runtime refused the launch
};

// Threads per workgroup: one wave.  A CU slot frees as soon as its one wave
// has stored, so the dispatcher refills each CU wave by wave; measured on
// MI355X at the same waves per CU, one-wave workgroups moved 3-9% more than
// four-wave ones (two-wave ones fell in between) on the large reductions,
// the allreduce, the ring and the element-wise path.
constexpr int kBlock = 64;
static_assert(kBlock == PTORED_WORKGROUP_THREADS, "the header states the workgroup size");

// Unroll (16-byte slots per thread per main tile).  Bandwidth sweeps on
// MI355X over tiles of 1 to 16 slots per thread: the smallest tiles were
// fastest for N >= 3 -- one slot per thread, all N loads of it in flight,
// many small blocks for the dispatcher to balance -- and two slots for N <= 2.
constexpr int unroll_for(int nranks) {
    return nranks <= 2 ? 2 : 1;
}
constexpr int kElemUnroll = 4;     // elements per thread, element-wise path

// Workgroups kept resident per CU for one-tile-per-block launches.  With
// every CU full the chip works on tens of thousands of scattered 1 KiB runs
// at once; keeping a few tiles per CU resident, issued in order by the
// dispatcher, keeps the live window of every buffer compact.  The counts are
// the best of sweeps on MI355X over 4-16 workgroups per CU with dst written
// to HBM on every call (a dst rewritten back to back stays in the 256 MB
// Infinity Cache and favours other counts), rank counts 1-24, four element
// types, the reduction and the ring:
//   reduction, its copy, the ring and push-with-add (folded): by rank count,
//     16 per CU up to 3 ranks down to 8 from 8 ranks on, and 6 from 12 ranks
//     on for 4-byte types
//     (about 48-128 KiB of loads in flight per CU; the 2-byte types, whose
//     slots hold twice the elements to fold, keep 8 there);
//   in-place allreduce, whose stores are half of its bytes: by the bytes a
//     tile moves (2N x 1 KiB), 8 up to 8 KiB, 5 up to 16, 4 beyond;
//   runtime rank loop: 10 (6 for the allreduce) -- it keeps only one group of
//     four ranks' loads in flight per wave, so it wants more waves.
constexpr int wgs_per_cu_reduce(int nranks, int esize) {
    return nranks <= 3 ? 16 : nranks <= 5 ? 12 : nranks <= 7 ? 10 : (nranks >= 12 && esize == 4) ? 6 : 8;
}
constexpr int wgs_per_cu_allreduce(uint64_t tile_bytes) {
    return tile_bytes <= 8u * 1024u ? 8 : (tile_bytes <= 16u * 1024u ? 5 : 4);
}
constexpr int kRuntimeLoopWgs = 10;
constexpr int kRuntimeLoopAllreduceWgs = 6;
// LDS is handed to workgroups in units of 1/128 of a CU's LDS (1280 bytes
// on MI355X): measured, 32768-byte reservations fit 4 workgroups per CU and
// 32000-byte ones 5, and the runtime's occupancy calculator, which assumes a
// finer unit, overcounts.  Reservations are multiples of this unit.
constexpr int kLdsUnitsPerCu = 128;
// A launch needs this many waves of capped workgroups to be worth capping.
constexpr int kCapMinRounds = 4;
constexpr int kLdsStages = 4;      // LDS stages per wave in the ping-pong variant
constexpr int kRuntimeUnroll = 1;  // slots per thread, runtime rank count

// Launch one kernel of the plan's family on `a`, on a persistent grid sized
// for `cu_count` compute units.
// Defined per element type in the kernel translation units.
int launch_f32(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);
int launch_bf16(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);
int launch_f16(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);
int launch_i32(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream);
// The single-launch ring reduce-scatter (vector families only).
int launch_ring_f32(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream);
int launch_ring_bf16(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream);
int launch_ring_f16(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream);
int launch_ring_i32(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream);

}  // namespace ptored
