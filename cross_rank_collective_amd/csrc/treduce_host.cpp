// treduce_host.cpp -- C ABI of the N-way reduction and its collective
// variants: validation, plan, launch.
//
// Sources (cited by title and section):
//   [TREDUCE]  "CANN PTO-ISA TREDUCE instruction explained" (lpnh.cn article
//              on pto-isa): §3.3 group checks (size > 0, root in range,
//              shared shape and strides), §4.1 dispatch (empty region
//              returns at once; data that fits takes the simple path, else
//              the chunked walk), §4.3 fold order and the single-rank copy.
//   [N6]       "Distributed Operators (N6)", PyPTO docs: append-only ABI
//              enums; pld.tensor.allreduce works in place on the window,
//              its ring mode cuts the stream into per-rank segments;
//              pld.tensor.put / remote_store with atomic = kAdd push-adds.
//
// Every argument check runs before the first HIP call, so every error status
// is reachable without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>

#include "ptored.h"
#include "treduce_plan.h"

namespace ptored {
namespace {

int esize_of(int dtype) { return (dtype == PTORED_F32 || dtype == PTORED_I32) ? 4 : 2; }

constexpr int64_t kDefaultLaunchBytes = int64_t(1) << 31;
constexpr int64_t kMaxElems = int64_t(1) << 60;

// Byte extent [p, p + span) that the valid rectangle touches in one buffer.
int64_t valid_span_bytes(int64_t vr, int64_t vc, int64_t ld, int es) {
    if (vr == 0 || vc == 0) return 0;
    return ((vr - 1) * ld + vc) * es;
}

// Checks shared by every entry point: rank count, pointers, shape, codes,
// element alignment ([TREDUCE] §3.3 group checks; a valid rectangle inside a
// rows x cols view).  `ptrs` holds every buffer the call touches.
int validate_common(const void* const* ptrs, int nptrs, int nranks, int64_t rows, int64_t cols,
                    int64_t ld, int64_t valid_rows, int64_t valid_cols, int dtype, int op) {
    if (nranks < 1 || nranks > PTORED_MAX_RANKS) return PTORED_ERR_INVALID_ARG;
    if (ptrs == nullptr) return PTORED_ERR_INVALID_ARG;
    for (int r = 0; r < nptrs; ++r)
        if (ptrs[r] == nullptr) return PTORED_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0 || ld < 0 || valid_rows < 0 || valid_cols < 0)
        return PTORED_ERR_INVALID_ARG;
    if (cols > ld || valid_rows > rows || valid_cols > cols) return PTORED_ERR_INVALID_ARG;
    if (rows > 0 && ld > 0 && rows > kMaxElems / ld) return PTORED_ERR_INVALID_ARG;
    if (dtype < PTORED_F32 || dtype > PTORED_I32) return PTORED_ERR_UNSUPPORTED;
    if (op < PTORED_SUM || op > PTORED_PROD) return PTORED_ERR_UNSUPPORTED;
    // Every pointer holds whole elements (natural alignment of the type).
    const uintptr_t amask = (uintptr_t)esize_of(dtype) - 1u;
    for (int r = 0; r < nptrs; ++r)
        if ((reinterpret_cast<uintptr_t>(ptrs[r]) & amask) != 0) return PTORED_ERR_INVALID_ARG;
    return PTORED_OK;
}

bool spans_overlap(const void* a, const void* b, int64_t span) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)span && y < x + (uintptr_t)span;
}

// Every pair of buffers is either the same buffer (when `alias_ok`) or
// disjoint over the `span` bytes the call touches.
int check_pairs(const void* const* a, int na, const void* const* b, int nb, int64_t span,
                bool alias_ok) {
    if (span <= 0) return PTORED_OK;
    for (int i = 0; i < na; ++i)
        for (int j = 0; j < nb; ++j) {
            if (a[i] == b[j] && alias_ok) continue;
            if (spans_overlap(a[i], b[j], span)) return PTORED_ERR_OVERLAP;
        }
    return PTORED_OK;
}

enum Mode { kModeReduce, kModeAllreduce, kModeAccumulate };

// Row tiles of a row of `numbered` slots, `per_tile` slots per tile: whole
// tiles, and a last partial tile when it would be at least half full; a
// smaller remainder (the spill) is folded in tail tiles instead, one slot
// per lane across rows, so that no tile runs with most of its lanes idle.
struct RowSplit {
    int64_t tiles;  // row tiles per row
    int64_t spill;  // slots per row left to the tail tiles
};
// Per-rank push-with-add (`no_spill`) keeps every slot in its row tiles.
RowSplit row_split(int64_t numbered, int64_t per_tile, bool no_spill = false) {
    const int64_t whole = numbered / per_tile, rem = numbered % per_tile;
    if (!no_spill && whole >= 1 && rem > 0 && rem * 2 <= per_tile) return {whole, rem};
    return {(numbered + per_tile - 1) / per_tile, 0};
}

// Choose the kernel family and the slot geometry ([TREDUCE] §4.1 analog) for
// already validated arguments.  `ptrs` holds every buffer the kernels touch
// (all sources, and dst when there is one).
int make_plan(const void* const* ptrs, int nptrs, int nranks, int64_t valid_rows,
              int64_t valid_cols, int64_t ld, int dtype, int op, const ptored_tuning* tuning,
              Mode mode, Plan& p) {
    const uint32_t flags = tuning ? tuning->flags : 0u;
    p = Plan{};
    p.dtype = dtype;
    p.op = op;
    p.nranks = nranks;
    p.esize = esize_of(dtype);
    p.valid_rows = valid_rows;
    p.valid_cols = valid_cols;
    p.ld = ld;
    p.blocks_per_cu = tuning ? tuning->blocks_per_cu : 0;
    // per-XCD bands only for persistent grids: with one tile per block the
    // dispatcher's round-robin over the XCDs keeps the live tiles contiguous
    p.xcd_remap = (flags & PTORED_NO_XCD_REMAP) == 0 && p.blocks_per_cu != 0;
    p.store_all = mode == kModeAllreduce;
    p.accumulate = mode == kModeAccumulate;
    p.push_per_rank = p.accumulate && (flags & PTORED_ACC_PER_RANK) != 0;
    int64_t mlb = (tuning && tuning->max_launch_bytes > 0) ? tuning->max_launch_bytes
                                                           : kDefaultLaunchBytes;
    mlb = std::min<int64_t>(mlb, kDefaultLaunchBytes);
    mlb = std::max<int64_t>(mlb & ~int64_t(15), 16);
    p.max_launch_bytes = mlb;

    if (valid_rows == 0 || valid_cols == 0) {
        p.family = kFamNone;
        p.launches = 0;
        return PTORED_OK;
    }
    // One contiguous span when the valid rows follow each other with no gap.
    const bool contiguous =
        (valid_cols == ld || valid_rows == 1) && (flags & PTORED_FORCE_ROWS) == 0;
    p.rows_mode = contiguous ? 0 : 1;
    p.total_elems = contiguous ? (valid_rows == 1 ? valid_cols : valid_rows * ld) : 0;

    // The 16-byte vector path numbers slots from an origin shared by every
    // buffer (byte offsets are taken from each buffer's own base, so slot k
    // holds the same elements everywhere); `lead` is the offset of element 0
    // past that origin, and a row or span starting inside a 16-byte block
    // begins with a head of element-wise items.  When every buffer starts at
    // the same offset within a 16-byte block and every row start keeps it
    // (pitch a multiple of 16 bytes), slots are numbered from the coarsest
    // boundary at which every buffer (and row) has the same offset: 1 KiB, so
    // that each wave's 1 KiB run is one aligned KiB (measured 3-4% faster than
    // runs at 128-512 bytes past it), else a 128-byte line, so that it covers 8
    // whole lines (12% faster than runs straddling lines), else 16 bytes.
    // Otherwise the slots keep one buffer aligned and the others take
    // unaligned 16-byte accesses, which gfx9 and later serve in the unaligned
    // access mode the HSA ABI enables: buffers at different offsets take the
    // last pointer's alignment (dst for the reduction); rows whose pitch is
    // not a multiple of 16 bytes number their slots from each row's start.
    // Measured on MI355X against one element per slot: +14-23% for 2-byte
    // types and odd pitches, level for 4-byte types at N = 16.  Push-with-add
    // takes dst's alignment too (only its source loads go unaligned; its
    // atomics stay on aligned words) but not odd pitches, which would move
    // its atomics off their words; the LDS variant (whose loads go straight
    // to LDS) keeps the shared-offset rule.
    bool use_vec = (flags & PTORED_FORCE_ELEMENTWISE) == 0;
    auto common_offset = [&](uintptr_t align) {
        const uintptr_t off = reinterpret_cast<uintptr_t>(ptrs[0]) & (align - 1u);
        for (int r = 1; r < nptrs; ++r)
            if ((reinterpret_cast<uintptr_t>(ptrs[r]) & (align - 1u)) != off) return -1;
        if (p.rows_mode && ((ld * p.esize) & (int64_t)(align - 1u)) != 0) return -1;
        return (int)off;
    };
    // offset of the last pointer past an `align` boundary, if every row keeps it
    auto anchor_offset = [&](uintptr_t align) {
        if (p.rows_mode && ((ld * p.esize) & (int64_t)(align - 1u)) != 0) return -1;
        return (int)(reinterpret_cast<uintptr_t>(ptrs[nptrs - 1]) & (align - 1u));
    };
    const bool lds = (flags & PTORED_LDS_PINGPONG) != 0 && mode == kModeReduce && nranks > 1;
    const bool odd_pitch = p.rows_mode && ((ld * p.esize) & 15) != 0;
    const bool unaligned_ok = !lds && !(mode == kModeAccumulate && odd_pitch);
    int lead = use_vec ? common_offset(16) : -1;
    if (lead >= 0) {
        const int kib = common_offset(1024), line = common_offset(128);
        if (kib >= 0) {
            lead = kib;
        } else if (line >= 0) {
            lead = line;
        }
    } else if (use_vec && unaligned_ok) {
        if (odd_pitch) {
            lead = 0;  // slots from each row's start
        } else {
            const int kib = anchor_offset(1024), line = anchor_offset(128);
            lead = kib >= 0 ? kib : (line >= 0 ? line : anchor_offset(16));
        }
    } else {
        use_vec = false;
    }
    if (use_vec) {
        const int64_t row_bytes = (contiguous ? p.total_elems : valid_cols) * p.esize;
        if (lead % 16 != 0 && lead % 16 + row_bytes < 16) use_vec = false;
    }
    p.lead = use_vec ? lead : 0;

    if (use_vec) {
        p.vec_elems = 16 / p.esize;
        if (p.push_per_rank) {
            p.family = kFamVecRuntime;  // one source per workgroup row; U = 1
            p.unroll = 1;
        } else if (nranks == 1 && mode != kModeAccumulate) {
            p.family = kFamCopy;
            p.unroll = unroll_for(1);
        } else if ((flags & PTORED_LDS_PINGPONG) != 0 && mode == kModeReduce) {
            p.family = kFamVecRuntime;  // runtime rank count through LDS stages
            p.lds_stages = true;
            p.unroll = 1;
        } else if (nranks <= 16 && (flags & PTORED_FORCE_RUNTIME_N) == 0) {
            p.family = kFamVecFixed;
            p.unroll = unroll_for(nranks);
        } else {
            p.family = kFamVecRuntime;
            p.unroll = kRuntimeUnroll;
        }
    } else {
        p.family = kFamElem;
        p.vec_elems = 1;
        p.unroll = kElemUnroll;
    }
    // Resident workgroups per CU for one-tile-per-block launches of the
    // 16-byte kernels (not per-rank push-with-add, which is bound by its
    // atomics; the folding one moves the reduction's streams).
    if (p.family != kFamElem && !p.push_per_rank && p.blocks_per_cu == 0 &&
        (flags & PTORED_FULL_OCCUPANCY) == 0) {
        const bool runtime_loop =
            p.family == kFamVecRuntime && (!p.lds_stages || nranks > 16);
        if (runtime_loop) {
            p.wgs_per_cu = mode == kModeAllreduce ? kRuntimeLoopAllreduceWgs : kRuntimeLoopWgs;
        } else if (mode == kModeAllreduce) {
            p.wgs_per_cu = wgs_per_cu_allreduce(2u * (uint64_t)nranks * kBlock * 16u *
                                                (uint64_t)p.unroll);
        } else {
            p.wgs_per_cu = wgs_per_cu_reduce(p.family == kFamCopy ? 1 : nranks, p.esize);
        }
    }
    const int64_t vec = p.vec_elems;
    if (p.rows_mode) {
        p.slots = valid_rows * ((valid_cols + vec - 1) / vec);
        // Row tiles when a row's full slots fill its column chunks well (at
        // least 7/8 of the threads busy, or 8+ chunks per row), else the
        // flattened walk.  Row tiles keep every wave's 1 KiB run inside one
        // row and cache-line aligned, so no line is fetched twice; with
        // few workgroups resident per CU they measured 3-4% faster than the
        // flattened walk on ragged rows.
        p.rows_mode = kWalkFlat;
        if (p.family != kFamElem && (flags & PTORED_FLAT_WALK) == 0) {
            const int64_t numbered = (p.lead + valid_cols * p.esize) / 16;
            const int64_t full = numbered - (p.lead + 15) / 16;
            const int64_t per_tile = (int64_t)kBlock * p.unroll;
            const RowSplit rs = row_split(numbered, per_tile, p.push_per_rank);
            const int64_t busy = full - rs.spill;  // whole slots the row tiles fold
            const bool fills = busy * 8 >= rs.tiles * per_tile * 7 || rs.tiles >= 8;
            if (full > 0 && (fills || (flags & PTORED_ROW_TILES) != 0))
                p.rows_mode = kWalkRowTiles;
        }
    } else {
        p.slots = (p.total_elems + vec - 1) / vec;
    }
    // Count launches (the same runs and bands run() walks).
    int64_t launches = 0;
    const int64_t es = p.esize, win = p.max_launch_bytes;
    const int64_t row_end = p.lead + valid_cols * es;
    if (!p.rows_mode) {  // windows meeting [lead, lead + span)
        launches = (p.lead + p.total_elems * es + win - 1) / win - p.lead / win;
    } else if (row_end <= win) {
        const int64_t ldb = ld * es;
        const int64_t rpl = (win - row_end) / ldb + 1;
        launches = (valid_rows + rpl - 1) / rpl;
    } else {
        launches = valid_rows * ((row_end + win - 1) / win - p.lead / win);
    }
    p.launches = launches;
    return PTORED_OK;
}

// Granlund-Montgomery multiplier for division by d >= 1 (32-bit dividends).
FastDiv fast_div_for(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    FastDiv f;
    f.mul = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    f.sh1 = l < 1 ? l : 1;
    f.sh2 = l > 1 ? l - 1 : 0;
    return f;
}

int launch_one(const Plan& p, const KArgs& a, int cu, hipStream_t s) {
    switch (p.dtype) {
    case PTORED_F32: return launch_f32(p, a, cu, s);
    case PTORED_BF16: return launch_bf16(p, a, cu, s);
    case PTORED_F16: return launch_f16(p, a, cu, s);
    default: return launch_i32(p, a, cu, s);
    }
}

void finish_tiles(const Plan& p, KArgs& a) {
    const uint64_t per_main = (uint64_t)kBlock * p.unroll;
    const uint64_t per_tail = (uint64_t)kBlock * (p.family == kFamElem ? kElemUnroll : 1);
    a.main_tiles = (uint32_t)((a.nslots + per_main - 1) / per_main);
    a.total_tiles = a.main_tiles + (uint32_t)(((uint64_t)a.ntail + a.nhead + a.nspill +
                                               per_tail - 1) / per_tail);
}

// One launch over bytes [lo, hi) of every buffer, counted from byte `base`
// of each (its launch base).  Vector path: the base is aligned to the slot
// origin and lo < 1024; slots are numbered from the base, those before lo
// skipped; bytes [lo, next 16-byte boundary) form a head when lo is inside
// a slot, then full 16-byte slots, then the remainder after the last full
// slot.  Element-wise path: lo == 0, every element is a tail item.
int launch_span(const Plan& p, KArgs a, const char* const* ordered, char* dst, int64_t base,
                int64_t lo, int64_t hi, int cu, hipStream_t s) {
    for (int r = 0; r < p.nranks; ++r) a.src[r] = ordered[r] + base;
    a.dst = dst + base;
    a.extent = (uint32_t)hi;
    a.ld_bytes = 0;
    a.div_slots = fast_div_for(1);
    a.div_tail = fast_div_for(1);
    a.tiles_per_row = 1;
    a.div_tiles = fast_div_for(1);
    a.nhead = 0;
    a.head_off = 0;
    a.head_lo = 0;
    a.slot_skip = 0;
    a.nspill = 0;
    a.spill_per_row = 0;
    a.spill_v0 = 0;
    a.div_spill = fast_div_for(1);
    if (p.family == kFamElem) {
        const int64_t elems = (hi - lo) / p.esize;
        a.nslots = 0;
        a.ntail = (uint32_t)elems;
        a.tail_per_row = (uint32_t)elems;
        a.tail_bytes = 0;
        a.tail_col_bytes = (uint32_t)lo;
    } else {
        const int64_t first = (lo + 15) / 16 * 16, last = hi / 16 * 16;
        a.slot_skip = (uint32_t)(first / 16);
        a.nslots = (uint32_t)(last / 16);
        a.nhead = lo % 16 != 0 ? 1u : 0u;
        a.head_off = (uint32_t)(lo / 16 * 16);
        a.head_lo = (uint32_t)(lo % 16);
        a.ntail = hi > last ? 1u : 0u;
        a.tail_per_row = 0;
        a.tail_bytes = (uint32_t)(hi - last);
        a.tail_col_bytes = (uint32_t)last;
    }
    a.slots_per_row = a.nslots;
    finish_tiles(p, a);
    Plan q = p;
    q.rows_mode = kWalkContig;
    return launch_one(q, a, cu, s);
}

// Launches over one run of bytes [lo, hi) counted from launch bases on the
// slot origin (lo < 1024), cut into windows of at most max_launch_bytes
// whose starts stay on the 16-byte grid.
int launch_run(const Plan& p, const KArgs& a, const char* const* ordered, char* dst,
               int64_t base, int64_t lo, int64_t hi, int cu, hipStream_t s) {
    int rc = 0;
    for (int64_t w0 = lo / p.max_launch_bytes * p.max_launch_bytes; w0 < hi && rc == 0;
         w0 += p.max_launch_bytes) {
        const int64_t l = std::max(lo, w0) - w0;
        const int64_t h = std::min(hi, w0 + p.max_launch_bytes) - w0;
        rc = launch_span(p, a, ordered, dst, base + w0, l, h, cu, s);
    }
    return rc;
}

// One launch over `nrows` rows of the valid rectangle starting at row `row0`.
// Vector path: each row's valid bytes are [lead, lead + valid_cols * esize)
// from its start on the slot origin -- skipped slots, a head when lead is
// inside a slot, full slots, a remainder.
int launch_rows(const Plan& p, KArgs a, const char* const* ordered, char* dst, int64_t row0,
                int64_t nrows, int cu, hipStream_t s) {
    const int64_t byte_off = row0 * p.ld * p.esize;
    for (int r = 0; r < p.nranks; ++r) a.src[r] = ordered[r] + byte_off;
    a.dst = dst + byte_off;
    a.extent = (uint32_t)((nrows - 1) * p.ld * p.esize + p.lead + p.valid_cols * p.esize);
    a.ld_bytes = nrows > 1 ? (uint32_t)(p.ld * p.esize) : 0u;
    a.tiles_per_row = 1;
    a.div_tiles = fast_div_for(1);
    a.nhead = 0;
    a.head_off = 0;
    a.head_lo = 0;
    a.slot_skip = 0;
    a.nspill = 0;
    a.spill_per_row = 0;
    a.spill_v0 = 0;
    a.div_spill = fast_div_for(1);
    if (p.family == kFamElem) {
        a.nslots = 0;
        a.slots_per_row = 0;
        a.div_slots = fast_div_for(1);
        a.ntail = (uint32_t)(nrows * p.valid_cols);
        a.tail_per_row = (uint32_t)p.valid_cols;
        a.div_tail = fast_div_for((uint32_t)p.valid_cols);
        a.tail_bytes = 0;
        a.tail_col_bytes = 0;
    } else {
        const int64_t end = p.lead + p.valid_cols * p.esize;  // row bytes from its start
        const int64_t first = (p.lead + 15) / 16 * 16, last = end / 16 * 16;
        const int64_t numbered = last / 16;  // slots numbered per row, skipped ones included
        a.slot_skip = (uint32_t)(first / 16);
        a.slots_per_row = (uint32_t)numbered;
        a.nslots = (uint32_t)(numbered * nrows);
        a.div_slots = fast_div_for(numbered > 0 ? (uint32_t)numbered : 1u);
        a.nhead = p.lead % 16 != 0 ? (uint32_t)nrows : 0u;
        a.head_off = (uint32_t)(p.lead / 16 * 16);
        a.head_lo = (uint32_t)(p.lead % 16);
        a.ntail = end > last ? (uint32_t)nrows : 0u;
        a.tail_per_row = 0;
        a.div_tail = fast_div_for(1);
        a.tail_bytes = (uint32_t)(end - last);
        a.tail_col_bytes = (uint32_t)last;
    }
    if (p.rows_mode == kWalkRowTiles) {
        const RowSplit rs = row_split(a.slots_per_row, (int64_t)kBlock * p.unroll,
                                      p.push_per_rank);
        a.tiles_per_row = (uint32_t)rs.tiles;
        a.div_tiles = fast_div_for(a.tiles_per_row);
        if (rs.spill > 0) {
            a.spill_per_row = (uint32_t)rs.spill;
            a.spill_v0 = a.slots_per_row - (uint32_t)rs.spill;
            a.nspill = (uint32_t)(rs.spill * nrows);
            a.div_spill = fast_div_for(a.spill_per_row);
        }
    }
    finish_tiles(p, a);
    if (p.rows_mode == kWalkRowTiles) {
        const uint32_t tail_tiles = a.total_tiles - a.main_tiles;
        a.main_tiles = (uint32_t)nrows * a.tiles_per_row;
        a.total_tiles = a.main_tiles + tail_tiles;
    }
    return launch_one(p, a, cu, s);
}

// Per-device facts the launches need, read once per device.
struct DeviceFacts {
    int cu;            // compute units
    int lds_per_cu;    // LDS bytes per CU
    int lds_per_block; // LDS bytes one workgroup may hold
};
std::atomic<int> g_dev_cu[256], g_dev_lds_cu[256], g_dev_lds_block[256];

int facts_of_current_device(DeviceFacts& f) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PTORED_ERR_HIP;
    const bool cacheable = dev >= 0 && dev < 256;
    if (cacheable && g_dev_cu[dev].load(std::memory_order_acquire) > 0) {
        f.lds_per_cu = g_dev_lds_cu[dev].load(std::memory_order_relaxed);
        f.lds_per_block = g_dev_lds_block[dev].load(std::memory_order_relaxed);
        f.cu = g_dev_cu[dev].load(std::memory_order_relaxed);
        return PTORED_OK;
    }
    int cu = 0, lds_cu = 0, lds_block = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu < 1)
        return PTORED_ERR_HIP;
    if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess) {
        lds_cu = 0;  // no occupancy limit without these
        lds_block = 0;
    }
    if (cacheable) {
        g_dev_lds_cu[dev].store(lds_cu, std::memory_order_relaxed);
        g_dev_lds_block[dev].store(lds_block, std::memory_order_relaxed);
        g_dev_cu[dev].store(cu, std::memory_order_release);
    }
    f.cu = cu;
    f.lds_per_cu = lds_cu;
    f.lds_per_block = lds_block;
    return PTORED_OK;
}

// The LDS reservation that lets exactly `wgs` workgroups share one CU:
// more than lds_per_cu / (wgs + 1), at most lds_per_cu / wgs, in whole
// allocation units, and within one workgroup's limit; 0 when no such size
// exists (no whole number of units fits exactly `wgs`, as for 13 or 15).
uint32_t cap_lds_bytes(const DeviceFacts& f, int wgs) {
    if (wgs < 1 || f.lds_per_cu <= 0) return 0;
    const int64_t grain = (int64_t)f.lds_per_cu / kLdsUnitsPerCu;
    if (grain <= 0) return 0;
    const int64_t lds = (int64_t)f.lds_per_cu / wgs / grain * grain;
    if (lds * (wgs + 1) <= (int64_t)f.lds_per_cu || lds > (int64_t)f.lds_per_block) return 0;
    return (uint32_t)lds;
}

// The plan with the occupancy limit resolved for this device.
Plan with_device(const Plan& p, const DeviceFacts& f) {
    Plan q = p;
    q.cap_lds = cap_lds_bytes(f, p.wgs_per_cu);
    q.cap_min_tiles = (uint64_t)kCapMinRounds * (uint64_t)f.cu * (uint64_t)(p.wgs_per_cu > 0 ? p.wgs_per_cu : 0);
    return q;
}

// Fold order of [TREDUCE] §4.3: the root's buffer first, then every other
// rank in ascending order.
void root_first_order(const void* const* srcs, int nranks, int root, const char** ordered) {
    ordered[0] = static_cast<const char*>(srcs[root]);
    int k = 1;
    for (int r = 0; r < nranks; ++r)
        if (r != root) ordered[k++] = static_cast<const char*>(srcs[r]);
}

// Launch the plan over buffers given in fold order (the kernels fold
// ordered[0], ordered[1], ... in index order).
int run(const Plan& plan, const char* const* ordered, void* dst, hipStream_t stream) {
    if (plan.family == kFamNone) return PTORED_OK;
    DeviceFacts f;
    int st = facts_of_current_device(f);
    if (st != PTORED_OK) return st;
    const Plan p = with_device(plan, f);
    const int cu = f.cu;

    KArgs a{};
    a.nranks = (uint32_t)p.nranks;
    a.xcd_remap = p.xcd_remap ? 1u : 0u;
    // Vector path: address every buffer from its slot origin, `lead` bytes
    // before the data (a 1 KiB, 128-byte or 16-byte boundary of every buffer,
    // or of dst alone when the buffers share no offset; for a pitch off the
    // 16-byte grid, lead is 0 and each row's slots start at the row).
    const char* base[PTORED_MAX_RANKS];
    for (int r = 0; r < p.nranks; ++r) base[r] = ordered[r] - p.lead;
    char* d = static_cast<char*>(dst) - p.lead;
    const int64_t es = p.esize;
    const int64_t row_end = p.lead + p.valid_cols * es;  // a valid row's bytes from its base
    int rc = 0;
    if (!p.rows_mode) {
        // One contiguous span, cut into launches of at most max_launch_bytes.
        rc = launch_run(p, a, base, d, 0, p.lead, p.lead + p.total_elems * es, cu, stream);
    } else if (row_end <= p.max_launch_bytes) {
        // Row bands whose byte extent fits in 32-bit offsets.
        const int64_t ldb = p.ld * es;
        const int64_t rpl = (p.max_launch_bytes - row_end) / ldb + 1;
        for (int64_t r0 = 0; r0 < p.valid_rows && rc == 0; r0 += rpl)
            rc = launch_rows(p, a, base, d, r0, std::min(rpl, p.valid_rows - r0), cu, stream);
    } else {
        // Rows longer than one launch: every row is a run of its own.
        for (int64_t r = 0; r < p.valid_rows && rc == 0; ++r)
            rc = launch_run(p, a, base, d, r * p.ld * es, p.lead, row_end, cu, stream);
    }
    if (rc == kLaunchNoKernel) return PTORED_ERR_UNSUPPORTED;
    return rc == kLaunchOk ? PTORED_OK : PTORED_ERR_HIP;
}

// TREDUCE arguments: validate, then plan.  ptrs = sources then dst.
int plan_treduce(const void* const* srcs, int nranks, int root, const void* dst, int64_t rows,
                 int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols, int dtype,
                 int op, const ptored_tuning* tuning, Plan& p) {
    if (nranks < 1 || nranks > PTORED_MAX_RANKS) return PTORED_ERR_INVALID_ARG;
    if (root < 0 || root >= nranks) return PTORED_ERR_INVALID_ARG;
    if (srcs == nullptr || dst == nullptr) return PTORED_ERR_INVALID_ARG;
    const void* ptrs[PTORED_MAX_RANKS + 1];
    for (int r = 0; r < nranks; ++r) ptrs[r] = srcs[r];
    ptrs[nranks] = dst;
    int st = validate_common(ptrs, nranks + 1, nranks, rows, cols, ld, valid_rows, valid_cols,
                             dtype, op);
    if (st != PTORED_OK) return st;
    // dst may be exactly a source (in place: each element is read by the one
    // thread that later writes it); any other overlap is a race.
    const int64_t span = valid_span_bytes(valid_rows, valid_cols, ld, esize_of(dtype));
    st = check_pairs(&ptrs[nranks], 1, ptrs, nranks, span, true);
    if (st != PTORED_OK) return st;
    return make_plan(ptrs, nranks + 1, nranks, valid_rows, valid_cols, ld, dtype, op, tuning,
                     kModeReduce, p);
}

// Segment boundaries of the ring schedule ([N6] pld.tensor.allreduce, ring
// mode): balanced floor(i * count / N); for 2-byte elements each interior
// boundary rounded up to 16 elements (32 bytes) and capped at count.
void ring_bounds(int64_t count, int nranks, int dtype, int64_t* bounds) {
    bounds[0] = 0;
    for (int i = 1; i < nranks; ++i) {
        // the product is formed in 128 bits; the quotient is at most count
        int64_t b = (int64_t)(((unsigned __int128)i * (uint64_t)count) / (uint64_t)nranks);
        if (esize_of(dtype) == 2) b = std::min<int64_t>(count, (b + 15) / 16 * 16);
        bounds[i] = b;
    }
    bounds[nranks] = count;
}

int launch_ring(const Plan& p, const RingArgs& a, int cu, hipStream_t s) {
    switch (p.dtype) {
    case PTORED_F32: return launch_ring_f32(p, a, cu, s);
    case PTORED_BF16: return launch_ring_bf16(p, a, cu, s);
    case PTORED_F16: return launch_ring_f16(p, a, cu, s);
    default: return launch_ring_i32(p, a, cu, s);
    }
}

// The ring reduce-scatter in one launch per window of max_launch_bytes (one
// launch in all for streams up to 2 GiB).  Windows are counted from `lead`
// bytes before every stream's start in multiples of 16, so whole slots stay
// whole (aligned when the streams share their offset within a 16-byte block,
// else on the last dst's alignment, the others accessed unaligned).
// `bounds` are the segment boundaries in elements.
int run_ring(const Plan& plan, const void* const* srcs, void* const* dsts, const int64_t* bounds,
             int64_t count, hipStream_t stream) {
    DeviceFacts f;
    int st = facts_of_current_device(f);
    if (st != PTORED_OK) return st;
    const Plan p = with_device(plan, f);
    const int cu = f.cu;
    const int n = p.nranks;
    // Every stream is addressed from `lead` bytes before its start (a 16-byte
    // boundary of every stream, or of the last dst); segment bounds move by
    // the same bytes.
    const int64_t es = p.esize, lead = p.lead, total = lead + count * es;
    RingArgs a{};
    a.nranks = (uint32_t)n;
    a.xcd_remap = p.xcd_remap ? 1u : 0u;
    int rc = 0;
    for (int64_t w0 = 0; w0 < total && rc == 0; w0 += p.max_launch_bytes) {
        const int64_t w1 = std::min(total, w0 + p.max_launch_bytes);
        int s0 = -1, s1 = -1;  // segments that meet [w0, w1)
        for (int s = 0; s < n; ++s)
            if (lead + bounds[s] * es < w1 && lead + bounds[s + 1] * es > w0) {
                if (s0 < 0) s0 = s;
                s1 = s;
            }
        if (s0 < 0) continue;
        for (int s = 0; s <= n; ++s)
            a.bounds[s] = (uint32_t)std::clamp<int64_t>(lead + bounds[s] * es - w0, 0, w1 - w0);
        uint32_t main_max = 0, edge = 0;
        for (int s = s0; s <= s1; ++s) {
            const uint32_t lo = a.bounds[s], hi = a.bounds[s + 1];
            const uint32_t first = (lo + 15u) & ~15u, end = hi & ~15u;
            const uint32_t from = first & ~1023u;  // slots numbered from a 1 KiB boundary
            const uint32_t nslots = first < end ? (end - from) / 16u : 0u;
            main_max = std::max(main_max, (nslots + (uint32_t)kBlock - 1) / (uint32_t)kBlock);
            const uint32_t head_end = std::min(hi, first);
            const uint32_t tail_lo = first <= end ? end : hi;
            if (head_end > lo || hi > tail_lo) edge = 1;
        }
        if (main_max + edge == 0) continue;
        for (int r = 0; r < n; ++r) {
            a.src[r] = a.src[r + n] = static_cast<const char*>(srcs[r]) - lead + w0;
            a.dst[r] = static_cast<char*>(dsts[r]) - lead + w0;
        }
        a.extent = (uint32_t)(w1 - w0);
        a.seg0 = (uint32_t)s0;
        a.nseg = (uint32_t)(s1 - s0 + 1);
        a.edge = edge;
        a.tiles_per_seg = main_max + edge;
        a.div_seg = fast_div_for(a.tiles_per_seg);
        rc = launch_ring(p, a, cu, stream);
    }
    if (rc == kLaunchNoKernel) return PTORED_ERR_UNSUPPORTED;
    return rc == kLaunchOk ? PTORED_OK : PTORED_ERR_HIP;
}

}  // namespace
}  // namespace ptored

using namespace ptored;

extern "C" int ptored_treduce_ex(const void* const* srcs, int nranks, int root, void* dst,
                                 int64_t rows, int64_t cols, int64_t ld, int64_t valid_rows,
                                 int64_t valid_cols, int dtype, int op,
                                 const ptored_tuning* tuning, hipStream_t stream) {
    Plan p;
    const int st = plan_treduce(srcs, nranks, root, dst, rows, cols, ld, valid_rows, valid_cols,
                                dtype, op, tuning, p);
    if (st != PTORED_OK) return st;
    const char* ordered[PTORED_MAX_RANKS];
    root_first_order(srcs, nranks, root, ordered);
    return run(p, ordered, dst, stream);
}

extern "C" int ptored_treduce(const void* const* srcs, int nranks, int root, void* dst,
                              int64_t rows, int64_t cols, int64_t ld, int64_t valid_rows,
                              int64_t valid_cols, int dtype, int op, hipStream_t stream) {
    return ptored_treduce_ex(srcs, nranks, root, dst, rows, cols, ld, valid_rows, valid_cols,
                             dtype, op, nullptr, stream);
}

extern "C" int ptored_treduce_plan(const void* const* srcs, int nranks, int root,
                                   const void* dst, int64_t rows, int64_t cols, int64_t ld,
                                   int64_t valid_rows, int64_t valid_cols, int dtype, int op,
                                   const ptored_tuning* tuning, ptored_plan_info* info) {
    Plan p;
    const int st = plan_treduce(srcs, nranks, root, dst, rows, cols, ld, valid_rows, valid_cols,
                                dtype, op, tuning, p);
    if (st != PTORED_OK) return st;
    if (info) {
        info->path = p.family;
        info->rows_mode = p.rows_mode;
        info->vec_elems = p.vec_elems;
        info->slots_per_thread = p.unroll;
        info->slots = p.slots;
        info->launches = p.launches;
        info->wgs_per_cu = p.wgs_per_cu;
        info->lead = p.lead;
    }
    return PTORED_OK;
}

extern "C" int ptored_allreduce(void* const* bufs, int nranks, int root, int64_t rows,
                                int64_t cols, int64_t ld, int64_t valid_rows, int64_t valid_cols,
                                int dtype, int op, const ptored_tuning* tuning,
                                hipStream_t stream) {
    if (nranks < 1 || nranks > PTORED_MAX_RANKS) return PTORED_ERR_INVALID_ARG;
    if (root < 0 || root >= nranks) return PTORED_ERR_INVALID_ARG;
    if (bufs == nullptr) return PTORED_ERR_INVALID_ARG;
    const void* const* ptrs = bufs;
    int st = validate_common(ptrs, nranks, nranks, rows, cols, ld, valid_rows, valid_cols, dtype,
                             op);
    if (st != PTORED_OK) return st;
    const int64_t span = valid_span_bytes(valid_rows, valid_cols, ld, esize_of(dtype));
    for (int i = 0; i < nranks; ++i) {  // pairwise: the same buffer or disjoint
        st = check_pairs(&ptrs[i], 1, &ptrs[i + 1], nranks - 1 - i, span, true);
        if (st != PTORED_OK) return st;
    }
    if (nranks == 1) return PTORED_OK;  // the fold of one buffer is itself
    Plan p;
    st = make_plan(ptrs, nranks, nranks, valid_rows, valid_cols, ld, dtype, op, tuning,
                   kModeAllreduce, p);
    if (st != PTORED_OK) return st;
    const char* ordered[PTORED_MAX_RANKS];
    root_first_order(ptrs, nranks, root, ordered);
    return run(p, ordered, bufs[0], stream);
}

extern "C" int ptored_ring_bounds(int64_t count, int nranks, int dtype, int64_t* bounds) {
    if (nranks < 1 || nranks > PTORED_MAX_RANKS || count < 0 || count > kMaxElems ||
        bounds == nullptr)
        return PTORED_ERR_INVALID_ARG;
    if (dtype < PTORED_F32 || dtype > PTORED_I32) return PTORED_ERR_UNSUPPORTED;
    ring_bounds(count, nranks, dtype, bounds);
    return PTORED_OK;
}

extern "C" int ptored_reduce_scatter_ring(const void* const* srcs, int nranks, void* const* dsts,
                                          int64_t count, int dtype, int op,
                                          const ptored_tuning* tuning, hipStream_t stream) {
    if (nranks < 1 || nranks > PTORED_MAX_RANKS) return PTORED_ERR_INVALID_ARG;
    if (srcs == nullptr || dsts == nullptr) return PTORED_ERR_INVALID_ARG;
    if (count < 0 || count > kMaxElems) return PTORED_ERR_INVALID_ARG;
    const void* ptrs[2 * PTORED_MAX_RANKS];
    for (int r = 0; r < nranks; ++r) {
        ptrs[r] = srcs[r];
        ptrs[nranks + r] = dsts[r];
    }
    int st = validate_common(ptrs, 2 * nranks, nranks, 1, count, count, 1, count, dtype, op);
    if (st != PTORED_OK) return st;
    // Each dst is the same buffer as a source or as another dst, or disjoint
    // from all of them: segments are disjoint, and each element is read and
    // written by one thread of one launch.
    const int64_t span = count * esize_of(dtype);
    st = check_pairs(&ptrs[nranks], nranks, ptrs, nranks, span, true);
    if (st != PTORED_OK) return st;
    for (int i = 0; i < nranks; ++i) {
        st = check_pairs(&ptrs[nranks + i], 1, &ptrs[nranks + i + 1], nranks - 1 - i, span, true);
        if (st != PTORED_OK) return st;
    }
    int64_t bounds[PTORED_MAX_RANKS + 1];
    ring_bounds(count, nranks, dtype, bounds);
    const uint32_t flags = tuning ? tuning->flags : 0u;
    if (nranks >= 2 && count > 0 && (flags & PTORED_SEGMENT_LAUNCHES) == 0) {
        // One launch over every segment when the 2N streams take 16-byte slots
        // (at any alignment; not through the LDS variant or element-wise).
        Plan p;
        st = make_plan(ptrs, 2 * nranks, nranks, 1, count, count, dtype, op, tuning, kModeReduce,
                       p);
        if (st != PTORED_OK) return st;
        if ((p.family == kFamVecFixed || p.family == kFamVecRuntime) && !p.lds_stages)
            return run_ring(p, srcs, dsts, bounds, count, stream);  // the reduction's residency
    }
    const int es = esize_of(dtype);
    for (int s = 0; s < nranks; ++s) {
        const int64_t lo = bounds[s], len = bounds[s + 1] - bounds[s];
        if (len == 0) continue;
        // Ring fold order of segment s: ranks s+1, s+2, ..., s (mod N).
        const char* ordered[PTORED_MAX_RANKS];
        const void* seg[PTORED_MAX_RANKS + 1];
        for (int k = 0; k < nranks; ++k) {
            ordered[k] = static_cast<const char*>(srcs[(s + 1 + k) % nranks]) + lo * es;
            seg[k] = ordered[k];
        }
        char* d = static_cast<char*>(dsts[s]) + lo * es;
        seg[nranks] = d;
        Plan p;
        st = make_plan(seg, nranks + 1, nranks, 1, len, len, dtype, op, tuning, kModeReduce, p);
        if (st != PTORED_OK) return st;
        st = run(p, ordered, d, stream);
        if (st != PTORED_OK) return st;
    }
    return PTORED_OK;
}

extern "C" int ptored_accumulate_add(const void* const* srcs, int nranks, void* dst,
                                     int64_t rows, int64_t cols, int64_t ld, int64_t valid_rows,
                                     int64_t valid_cols, int dtype, const ptored_tuning* tuning,
                                     hipStream_t stream) {
    if (nranks < 1 || nranks > PTORED_MAX_RANKS) return PTORED_ERR_INVALID_ARG;
    if (srcs == nullptr || dst == nullptr) return PTORED_ERR_INVALID_ARG;
    const void* ptrs[PTORED_MAX_RANKS + 1];
    for (int r = 0; r < nranks; ++r) ptrs[r] = srcs[r];
    ptrs[nranks] = dst;
    int st = validate_common(ptrs, nranks + 1, nranks, rows, cols, ld, valid_rows, valid_cols,
                             dtype, PTORED_SUM);
    if (st != PTORED_OK) return st;
    // dst may not be any source, not even exactly: a source read while other
    // ranks' additions land in it would race.
    const int64_t span = valid_span_bytes(valid_rows, valid_cols, ld, esize_of(dtype));
    st = check_pairs(&ptrs[nranks], 1, ptrs, nranks, span, false);
    if (st != PTORED_OK) return st;
    Plan p;
    st = make_plan(ptrs, nranks + 1, nranks, valid_rows, valid_cols, ld, dtype, PTORED_SUM,
                   tuning, kModeAccumulate, p);
    if (st != PTORED_OK) return st;
    const char* ordered[PTORED_MAX_RANKS];
    for (int r = 0; r < nranks; ++r) ordered[r] = static_cast<const char*>(srcs[r]);
    return run(p, ordered, dst, stream);
}

extern "C" const char* ptored_status_string(int status) {
    switch (status) {
    case PTORED_OK: return "PTORED_OK";
    case PTORED_ERR_INVALID_ARG: return "PTORED_ERR_INVALID_ARG: bad rank count, root, pointer or shape";
    case PTORED_ERR_UNSUPPORTED: return "PTORED_ERR_UNSUPPORTED: unknown dtype or op";
    case PTORED_ERR_OVERLAP: return "PTORED_ERR_OVERLAP: buffers overlap in a way the call cannot allow";
    case PTORED_ERR_HIP: return "PTORED_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown ptored status";
    }
}

extern "C" int ptored_abi_version(void) { return PTORED_ABI_VERSION; }

extern "C" int ptored_max_ranks(void) { return PTORED_MAX_RANKS; }
