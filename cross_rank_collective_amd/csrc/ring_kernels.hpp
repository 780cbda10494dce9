// ring_kernels.hpp -- the ring reduce-scatter in one launch.
//
// Source: "Distributed Operators (N6)", PyPTO docs, pld.tensor.allreduce in
// ring mode: the stream is cut into one segment per rank, and segment s
// reaches its owner after passing through ranks s+1, s+2, ..., s (mod N),
// each adding its own share.  On one device the N streams are N buffers, so
// segment s is the fold of src[s+1], src[s+2], ..., src[s] in that order.
//
// One launch covers every segment of a window: tile t belongs to segment
// seg0 + t / tiles_per_seg (a per-workgroup scalar), and the source table
// is doubled, so the rotated order is a run of consecutive table entries.  A segment's whole 16-byte
// slots are folded exactly like the reduction's main tiles; its elements
// before the first and after the last whole slot (segment bounds need not
// be 16-byte aligned) are folded one per lane in the segment's last tile.
#pragma once

#include "treduce_kernels.hpp"

namespace ptored {

template <int DT, int OP, int ES, int NR>
__global__ __launch_bounds__(kBlock) void ring_kernel(const RingArgs a) {
    const uint32_t grid = gridDim.x;
    const uint32_t total = a.nseg * a.tiles_per_seg;
    const uint32_t n = NR > 0 ? (uint32_t)NR : a.nranks;
    // Every launched block's first tile exists (at most one block per tile,
    // no launch without tiles), so it is taken without a check, as in
    // treduce_kernel; `continue` below moves on to the next tile.
    uint32_t t = logical_block(blockIdx.x, grid, a.xcd_remap != 0u);
    do {
        const uint32_t q = fast_div(t, a.div_seg);
        const uint32_t local = t - q * a.tiles_per_seg;
        const uint32_t s = a.seg0 + q;
        const uint32_t lo = a.bounds[s], hi = a.bounds[s + 1];
        const uint32_t first = (lo + 15u) & ~15u;  // start of the whole slots
        const uint32_t end = hi & ~15u;            // end of the whole slots (if first <= end)
        // k-th source of the segment's fold: rank (s + 1 + k) mod N
        const void* const* ring = a.src + (s + 1u);
        const auto src = [&](uint32_t k) { return make_rsrc(ring[k], a.extent); };
        const rsrc_t rd = make_rsrc(a.dst[s], a.extent);
        if (a.edge != 0u && local + 1u == a.tiles_per_seg) {
            // Ragged ends: [lo, min(hi, first)) and [end, hi) when the
            // segment has whole slots, else all of [lo, hi) as its head.
            const uint32_t head_end = hi < first ? hi : first;
            const uint32_t head_n = (head_end - lo) / (uint32_t)ES;
            const uint32_t tail_lo = first <= end ? end : hi;
            const uint32_t items = head_n + (hi - tail_lo) / (uint32_t)ES;
            if (threadIdx.x < items) {
                const uint32_t off = threadIdx.x < head_n
                                         ? lo + threadIdx.x * (uint32_t)ES
                                         : tail_lo + (threadIdx.x - head_n) * (uint32_t)ES;
                Acc<DT, OP> acc;
                acc.init(load_elem<ES>(src(0u), off));
                for (uint32_t k = 1; k < n; ++k) acc.add(load_elem<ES>(src(k), off));
                store_elem<ES, store_policy_for(NR)>(rd, off, acc.get());
            }
        } else {
            // slots numbered from the 1 KiB boundary at or below the first
            // one, so that every wave's 1 KiB run is one aligned KiB
            const uint32_t from = first & ~1023u;
            const uint32_t nslots = first < end ? (end - from) >> 4 : 0u;
            const uint32_t base = local * (uint32_t)kBlock;
            if (base >= nslots) continue;  // a shorter segment's spare tile
            const uint32_t j = base + threadIdx.x, o = from + j * 16u;
            const uint32_t off[1] = {j < nslots && o >= first ? o : kOutOfRange};
            u32x4 out[1];
            fold_slots<DT, OP, NR, 1>(src, n, off, out);
            store16<store_policy_for(NR)>(rd, off[0], out[0]);
        }
    } while ((t += grid) < total);
}

}  // namespace ptored
