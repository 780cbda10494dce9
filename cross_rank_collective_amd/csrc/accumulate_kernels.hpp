// accumulate_kernels.hpp -- push-with-add: dst += src_r for every rank r.
//
// Source: "Distributed Operators (N6)", PyPTO docs, pld.tile.remote_store /
// pld.tensor.put with atomic = AtomicType.kAdd: a push that adds into the
// peer's slice instead of overwriting it (the combine an all-to-all needs),
// for fp32 / bf16 / fp16 / int32 among others.  With N ranks pushing into one
// slice the contributions land in an unspecified order; on one GPU the N
// pushes are the N source buffers and the slice is dst.
//
// Each workgroup pushes one rank's tile of 64 16-byte slots (blockIdx.y =
// rank): the tile's 32-bit words are loaded from that rank's buffer and added
// into dst with one device-scope atomic per word (global_atomic_add_f32,
// global_atomic_pk_add_f16, global_atomic_pk_add_bf16, global_atomic_add_u32),
// consecutive lanes on consecutive words.  A 16-bit element that
// does not fill its 32-bit word (row remainders, the element-wise path) is
// added with a compare-and-swap loop on the containing word that rewrites
// only its own half, so the neighbouring half keeps its bits exactly; on the
// element-wise path two neighbouring elements that fill one word are added
// together with one packed atomic.  The
// order in which ranks' additions land differs from run to run, so float
// results agree with any fixed order only to within the rounding of N
// additions; i32 additions wrap and are exact.
#pragma once

#include "treduce_kernels.hpp"

namespace ptored {

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

// Add one element at p (ES bytes) atomically.
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
                // MI355X four times slower at the L2's atomic units.
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
            if constexpr (ES == 4) {
#pragma unroll
                for (int u = 0; u < kElemUnroll; ++u)
                    if (off[u] != kOutOfRange)
                        atomic_add_word<DT>(d + off[u], load_elem<4>(rs, off[u]));
            } else {
                // 16-bit elements: a lane whose element opens a 32-bit word
                // and whose right neighbour -- the next lane, or lane 0 of
                // the next slice of the tile for lane 63 -- holds the word's
                // other half adds both with one packed atomic; every other
                // element takes the half-word compare-and-swap.  The
                // shuffles run on every lane, before any branch.
                uint32_t v[kElemUnroll];
#pragma unroll
                for (int u = 0; u < kElemUnroll; ++u)
                    v[u] = off[u] != kOutOfRange ? load_elem<2>(rs, off[u]) : 0u;
                const uint32_t lane = threadIdx.x;
#pragma unroll
                for (int u = 0; u < kElemUnroll; ++u) {
                    const bool valid = off[u] != kOutOfRange;
                    uint32_t next_off = (uint32_t)__shfl_down((int)off[u], 1, kBlock);
                    uint32_t next_v = (uint32_t)__shfl_down((int)v[u], 1, kBlock);
                    uint32_t prev_off = (uint32_t)__shfl_up((int)off[u], 1, kBlock);
                    if (u + 1 < kElemUnroll) {
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
    }
}

}  // namespace ptored
