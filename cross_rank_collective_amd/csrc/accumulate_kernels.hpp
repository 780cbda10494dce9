// accumulate_kernels.hpp -- push-with-add, one atomic per source element.
//
// Source: "Distributed Operators (N6)", PyPTO docs, pld.tile.remote_store /
// pld.tensor.put with atomic = AtomicType.kAdd: a push that adds into the
// peer's slice instead of overwriting it (the combine an all-to-all needs),
// for fp32 / bf16 / fp16 / int32 among others.  With N ranks pushing into one
// slice the contributions land in an unspecified order; on one GPU the N
// pushes are the N source buffers and the slice is dst.
//
// This is the per-rank form (PTORED_ACC_PER_RANK): every source's words are
// added into dst on their own, as N ranks' remote stores would land, so dst
// takes N atomics per word.  The default push-with-add folds the call's N
// sources first and adds the fold with one atomic per word (treduce_kernel
// with StoreMode kStoreAdd).
//
// Each workgroup pushes one rank's tile of 64 16-byte slots (blockIdx.y =
// rank): the tile's 32-bit words are loaded from that rank's buffer and added
// into dst with one device-scope atomic per word, consecutive lanes on
// consecutive words (atomic_add_word, atomic_add_elem and push_elements in
// treduce_kernels.hpp).  The order in which ranks' additions land differs
// from run to run, so float results agree with any fixed order only to
// within the rounding of N additions; i32 additions wrap and are exact.
#pragma once

#include "treduce_kernels.hpp"

namespace ptored {

// Tiles as in treduce_kernel (U = 1): row remainders and heads, then main
// tiles of 16-byte slots; without VEC, element tiles only.  gridDim.y = N.
template <int DT, int ES, int WALK, bool VEC>
__global__ __launch_bounds__(kBlock) void accumulate_kernel(const KArgs a) {
    const rsrc_t rs = make_rsrc(a.src[blockIdx.y], a.extent);
    char* const d = static_cast<char*>(a.dst);
    for (uint32_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        if constexpr (VEC) {
            const uint32_t tails = a.total_tiles - a.main_tiles;  // issued first, as in treduce_kernel
            if (t >= tails) {
                // The tile's 64 slots as 256 32-bit words, word j of the tile
                // taken by lane j % 64 in step j / 64: every load and atomic
                // instruction of the wave covers 256 contiguous bytes (16
                // slots), two cache lines, where 16 bytes per lane would
                // spread each instruction's atomics over eight lines -- on
                // MI355X four times slower at the memory side, where the
                // atomics are done.
                // Row tiles: tile = column chunk c of row r, its slots
                // numbered from the row's slot origin, so every run stays
                // inside one row and on the line grid.
                const uint32_t tile = t - tails;
                uint32_t slot0 = tile * (uint32_t)kBlock, row_off = 0;
                if constexpr (WALK == kWalkRowTiles) {
                    const uint32_t row = fast_div(tile, a.div_tiles);
                    slot0 = (tile - row * a.tiles_per_row) * (uint32_t)kBlock;
                    row_off = row * a.ld_bytes;
                }
                const uint32_t lane = threadIdx.x, byte_in_slot = 4u * (lane & 3u);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t v = slot0 + (uint32_t)(w * 16) + (lane >> 2);
                    uint32_t off;
                    if constexpr (WALK == kWalkRowTiles) {
                        off = v < a.slots_per_row && v >= a.slot_skip ? row_off + v * 16u
                                                                      : kOutOfRange;
                    } else {
                        off = slot_offset<WALK>(a, v);
                    }
                    if (off != kOutOfRange)
                        atomic_add_word<DT>(d + off + byte_in_slot,
                                            load_elem<4>(rs, off + byte_in_slot));
                }
            } else {
                const uint32_t q = t * (uint32_t)kBlock + threadIdx.x;
                // Remainders and heads lie in one 16-byte block of dst that
                // starts on a 16-byte boundary: whole 32-bit words take one
                // atomic each, only a lone 16-bit element the half-word one.
                if (q < a.ntail) {  // row remainder: bytes [0, tail_bytes) of its block
                    const uint32_t off = q * a.ld_bytes + a.tail_col_bytes;
                    uint32_t e = 0;
                    for (; e + 4u <= a.tail_bytes; e += 4u)
                        atomic_add_word<DT>(d + off + e, load_elem<4>(rs, off + e));
                    if (e < a.tail_bytes)
                        atomic_add_elem<DT, ES>(d + off + e, load_elem<ES>(rs, off + e));
                } else if (q - a.ntail < a.nhead) {  // row head: bytes [head_lo, 16)
                    const uint32_t off = (q - a.ntail) * a.ld_bytes + a.head_off;
                    uint32_t e = a.head_lo;
                    if (e & 2u) {
                        atomic_add_elem<DT, ES>(d + off + e, load_elem<ES>(rs, off + e));
                        e += 2u;
                    }
                    for (; e < 16u; e += 4u)
                        atomic_add_word<DT>(d + off + e, load_elem<4>(rs, off + e));
                }
            }
        } else {
            uint32_t off[kElemUnroll];
#pragma unroll
            for (int u = 0; u < kElemUnroll; ++u)
                off[u] = tail_offset<WALK, ES>(
                    a, t * (uint32_t)(kBlock * kElemUnroll) + (uint32_t)(u * kBlock) + threadIdx.x);
            uint32_t v[kElemUnroll];
#pragma unroll
            for (int u = 0; u < kElemUnroll; ++u)
                v[u] = off[u] != kOutOfRange ? load_elem<ES>(rs, off[u]) : 0u;
            push_elements<DT, ES, kElemUnroll>(d, off, v);
        }
    }
}

}  // namespace ptored
