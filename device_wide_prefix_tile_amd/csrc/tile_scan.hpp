// tile_scan.hpp -- single-pass tile scan and fused stream compaction (gfx950).
//
// Pages cited:
//   [L7]    "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
//           (UIUC ECE408 course notes, runguoli.com)
//   [PMPP9] "第9章并行模式：前缀和 - Scan算法" (PMPP chapter 9 notes, bittern.cn)
//
// One workgroup scans one tile of TILE = BLOCK * ITEMS elements:
//   1. take the next tile number from a counter (start order, not hardware
//      order);
//   2. load the tile with 16-byte loads: wavefront w owns 64 * ITEMS
//      consecutive elements, in R = ITEMS / VEC rounds of 64 * VEC elements,
//      lane l holding VEC consecutive elements of each round, so every load
//      instruction of a wavefront reads 1 KiB of contiguous memory;
//   3. scan each lane's VEC elements serially in registers (thread
//      coarsening, [L7 concept 6 and its kernel-2 register array]);
//   4. scan the lane totals across the wavefront with DPP (wave_ops.hpp);
//   5. combine the wavefront totals through LDS with one barrier;
//   6. wavefront 0 publishes the tile total, looks back for the prefix of all
//      earlier tiles and publishes the tile's inclusive prefix
//      (lookback.hpp) -- this replaces the hierarchical scan's second and
//      third kernels [L7 concept 6], so the data cross HBM once each way;
//   7. apply the prefix and store with 16-byte stores.
// Exclusive scans put the identity at y[0] and use the value before each
// element [L7 concept 1; PMPP9 §9.1].  The tail tile pads with the identity
// in registers and never stores the padding.  In SINGLE mode one workgroup
// walks all tiles in order and carries the prefix in registers instead of
// using the status array (the small-n path: no workspace, no atomics).
//
// Compaction [L7 concept 2 "扫描的典型应用"; PMPP9 §9.6]: the predicate
// x > 0 is evaluated in registers, the 0/1 flags are scanned the same way
// (uint32 count), kept elements are packed in LDS at their rank inside the
// tile and written out as one contiguous run at the tile's prefix count, so
// flags and positions never touch HBM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lookback.hpp"
#include "scan_ops.hpp"
#include "wave_ops.hpp"

namespace dwpt {

struct ScanParams {
    const void* in;
    void* out;
    const uint8_t* heads;  // segmented scans only
    uint32_t* count;       // compaction only: number of kept elements
    uint64_t n;
    uint32_t num_tiles;
    uint32_t ctr_base;     // counter value when this launch started
    uint32_t* tile_ctr;
    Lookback lb;
    int vec_ok;            // 16-byte aligned pointers: vector loads/stores
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class Op> struct IsSeg { static constexpr bool value = false; };
template <class B> struct IsSeg<OpSeg<B>> { static constexpr bool value = true; };

template <class Op>
__device__ __forceinline__ typename Op::value_t make_value(typename Op::elem_t e, uint32_t head)
{
    if constexpr (IsSeg<Op>::value) return {head, e};
    else return e;
}
template <class Op>
__device__ __forceinline__ typename Op::elem_t elem_of(typename Op::value_t v)
{
    if constexpr (IsSeg<Op>::value) return v.v;
    else return v;
}
template <class Op>
__device__ __forceinline__ bool resets(typename Op::value_t v)
{
    if constexpr (IsSeg<Op>::value) return v.f != 0u;
    else return false;
}

template <typename E, int VEC>
__device__ __forceinline__ void load_vec(const E* p, E (&e)[VEC])
{
    static_assert(sizeof(E) * VEC == 16, "16-byte vector");
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    __builtin_memcpy(e, &v, 16);
}
template <typename E, int VEC>
__device__ __forceinline__ void store_vec(E* p, const E (&e)[VEC])
{
    u32x4 v;
    __builtin_memcpy(&v, e, 16);
    *reinterpret_cast<u32x4*>(p) = v;
}

// ------------------------------------------------------------------ scan
template <class Op, bool EXCL, int BLOCK, int ITEMS, bool SINGLE>
__global__ __launch_bounds__(BLOCK) void tile_scan_kernel(ScanParams p)
{
    using E = typename Op::elem_t;
    using V = typename Op::value_t;
    using C = typename Op::carry_t;
    constexpr bool SEG = IsSeg<Op>::value;
    constexpr int VEC = 16 / (int)sizeof(E);
    constexpr int R = ITEMS / VEC;
    constexpr int NW = BLOCK / 64;
    constexpr int WAVE_ELEMS = 64 * ITEMS;
    constexpr int TILE = BLOCK * ITEMS;
    static_assert(ITEMS % VEC == 0 && BLOCK % 64 == 0, "tile shape");
    static_assert(!SEG || VEC == 4, "segmented scans use 4-byte elements");

    __shared__ V s_wave[NW];
    __shared__ C s_prefix;
    __shared__ uint32_t s_tile;

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const E* __restrict__ in = static_cast<const E*>(p.in);
    E* __restrict__ out = static_cast<E*>(p.out);
    const V ident = Op::identity();
    const auto comb = [](V a, V b) { return Op::combine(a, b); };

    C running = Op::carry_identity();  // SINGLE mode carry
    const uint32_t tiles_here = SINGLE ? p.num_tiles : 1u;

    for (uint32_t it = 0; it < tiles_here; ++it) {
        uint32_t tile;
        if constexpr (SINGLE) {
            tile = it;
        } else {
            if (threadIdx.x == 0)
                s_tile = __hip_atomic_fetch_add(p.tile_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                         p.ctr_base;
            __syncthreads();
            tile = s_tile;
            if (tile >= p.num_tiles) {  // counter out of step with this launch: never index past the grid
                if (threadIdx.x == 0)
                    __hip_atomic_fetch_or(p.lb.err, (uint32_t)kErrCounter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
        }

        const uint64_t tile_base = (uint64_t)tile * TILE;
        const uint64_t wave_base = tile_base + (uint64_t)w * WAVE_ELEMS;
        const bool full = tile_base + TILE <= p.n;

        // ---- load (2)
        V x[R][VEC];
        uint32_t raw_head[R];  // bit j: element j of round r is a segment head
        if (full && p.vec_ok) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint64_t i0 = wave_base + (uint64_t)(r * 64 + lane) * VEC;
                E e[VEC];
                load_vec<E, VEC>(in + i0, e);
                uint32_t hb = 0;
                if constexpr (SEG) {
                    const uint32_t h4 = *reinterpret_cast<const uint32_t*>(p.heads + i0);
#pragma unroll
                    for (int j = 0; j < VEC; ++j) hb |= ((h4 >> (8 * j)) & 0xFFu) ? (1u << j) : 0u;
                    if (i0 == 0) hb |= 1u;
                }
                raw_head[r] = hb;
#pragma unroll
                for (int j = 0; j < VEC; ++j) x[r][j] = make_value<Op>(e[j], (hb >> j) & 1u);
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint64_t i0 = wave_base + (uint64_t)(r * 64 + lane) * VEC;
                uint32_t hb = 0;
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const uint64_t i = i0 + j;
                    if (i < p.n) {
                        uint32_t h = 0;
                        if constexpr (SEG) h = (i == 0 || p.heads[i]) ? 1u : 0u;
                        hb |= h << j;
                        x[r][j] = make_value<Op>(in[i], h);
                    } else {
                        x[r][j] = ident;
                    }
                }
                raw_head[r] = hb;
            }
        }

        // ---- serial scan in registers (3)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 1; j < VEC; ++j) x[r][j] = Op::combine(x[r][j - 1], x[r][j]);

        // ---- wavefront scans of the lane totals (4)
        V lane_excl[R];
        V round_carry[R + 1];
        round_carry[0] = ident;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const V incl = wave_inclusive_scan(x[r][VEC - 1], ident, comb);
            lane_excl[r] = wave_shift_up(incl, ident);
            round_carry[r + 1] = Op::combine(round_carry[r], read_lane(incl, 63));
        }

        // ---- cross-wavefront combine (5)
        if (lane == 0) s_wave[w] = round_carry[R];
        __syncthreads();
        V wave_prefix = ident, tile_total = ident;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const V a = s_wave[k];
            if (k < w) wave_prefix = Op::combine(wave_prefix, a);
            tile_total = Op::combine(tile_total, a);
        }

        // ---- inter-tile prefix (6)
        C P;
        if constexpr (SINGLE) {
            P = running;
            running = Op::combine_carry(running, Op::to_carry(tile_total));
        } else {
            if (w == 0) {
                const C agg = Op::to_carry(tile_total);
                // A tile with no predecessor, or whose total restarts the
                // fold (a segment head inside it), already knows its inclusive
                // prefix: publish it as PREFIX straight away.
                const bool known = (tile == 0) || resets<Op>(tile_total);
                if (lane == 0) publish<Op>(p.lb, tile, agg, known ? kStatePrefix : kStateAggregate);
                C excl = Op::carry_identity();
                // Elements before the tile's first head still need the prefix.
                bool need = tile != 0;
                if constexpr (SEG) need = need && !(__builtin_amdgcn_readfirstlane(raw_head[0]) & 1u);
                if (need) excl = lookback<Op>(p.lb, tile);
                if (!known && lane == 0) publish<Op>(p.lb, tile, Op::combine_carry(excl, agg), kStatePrefix);
                if (lane == 0) s_prefix = excl;
            }
            __syncthreads();
            P = s_prefix;
        }

        // ---- apply and store (7)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const V in_tile = Op::combine(Op::combine(wave_prefix, round_carry[r]), lane_excl[r]);
            const typename Op::prep_t pc = Op::prepare(Op::combine_carry(P, Op::to_carry(in_tile)));
            E e[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                V y;
                if constexpr (EXCL) {
                    y = Op::apply(pc, j == 0 ? ident : x[r][j - 1]);
                    if constexpr (SEG)
                        if ((raw_head[r] >> j) & 1u) y = ident;
                } else {
                    y = Op::apply(pc, x[r][j]);
                }
                e[j] = elem_of<Op>(y);
            }
            const uint64_t i0 = wave_base + (uint64_t)(r * 64 + lane) * VEC;
            if (full && p.vec_ok) {
                store_vec<E, VEC>(out + i0, e);
            } else {
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    if (i0 + j < p.n) out[i0 + j] = e[j];
            }
        }
        if constexpr (SINGLE) __syncthreads();  // s_wave is rewritten by the next tile
    }
}

// ------------------------------------------------------------ compaction
template <typename T>
__device__ __forceinline__ bool keep(T x) { return x > T(0); }

template <typename T, int BLOCK, int ITEMS, bool SINGLE>
__global__ __launch_bounds__(BLOCK) void compact_kernel(ScanParams p)
{
    using Cnt = OpAdd<uint32_t>;
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int R = ITEMS / VEC;
    constexpr int NW = BLOCK / 64;
    constexpr int WAVE_ELEMS = 64 * ITEMS;
    constexpr int TILE = BLOCK * ITEMS;
    static_assert(ITEMS % VEC == 0 && BLOCK % 64 == 0, "tile shape");

    __shared__ T s_keep[TILE];
    __shared__ uint32_t s_wave[NW];
    __shared__ uint32_t s_prefix;
    __shared__ uint32_t s_tile;

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const T* __restrict__ in = static_cast<const T*>(p.in);
    T* __restrict__ out = static_cast<T*>(p.out);
    const auto add = [](uint32_t a, uint32_t b) { return a + b; };

    uint32_t running = 0;
    const uint32_t tiles_here = SINGLE ? p.num_tiles : 1u;
    for (uint32_t it = 0; it < tiles_here; ++it) {
        uint32_t tile;
        if constexpr (SINGLE) {
            tile = it;
        } else {
            if (threadIdx.x == 0)
                s_tile = __hip_atomic_fetch_add(p.tile_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                         p.ctr_base;
            __syncthreads();
            tile = s_tile;
            if (tile >= p.num_tiles) {
                if (threadIdx.x == 0)
                    __hip_atomic_fetch_or(p.lb.err, (uint32_t)kErrCounter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
        }
        const uint64_t tile_base = (uint64_t)tile * TILE;
        const uint64_t wave_base = tile_base + (uint64_t)w * WAVE_ELEMS;
        const bool full = tile_base + TILE <= p.n;

        T x[R][VEC];
        uint32_t kept[R];  // bit j: element j of round r passes the predicate
        if (full && p.vec_ok) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                load_vec<T, VEC>(in + wave_base + (uint64_t)(r * 64 + lane) * VEC, x[r]);
                uint32_t b = 0;
#pragma unroll
                for (int j = 0; j < VEC; ++j) b |= keep(x[r][j]) ? (1u << j) : 0u;
                kept[r] = b;
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint64_t i0 = wave_base + (uint64_t)(r * 64 + lane) * VEC;
                uint32_t b = 0;
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    x[r][j] = (i0 + j < p.n) ? in[i0 + j] : T(0);
                    b |= (i0 + j < p.n && keep(x[r][j])) ? (1u << j) : 0u;
                }
                kept[r] = b;
            }
        }

        // flag counts: per lane, then across the wavefront, then across wavefronts
        uint32_t lane_excl[R];
        uint32_t round_base[R + 1];
        round_base[0] = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t incl = wave_inclusive_scan((uint32_t)__builtin_popcount(kept[r]), 0u, add);
            lane_excl[r] = wave_shift_up(incl, 0u);
            round_base[r + 1] = round_base[r] + read_lane(incl, 63);
        }
        if (lane == 0) s_wave[w] = round_base[R];
        __syncthreads();
        uint32_t wave_prefix = 0, tile_total = 0;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const uint32_t a = s_wave[k];
            if (k < w) wave_prefix += a;
            tile_total += a;
        }

        // pack kept elements at their rank inside the tile
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t rank = wave_prefix + round_base[r] + lane_excl[r];
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                if ((kept[r] >> j) & 1u) s_keep[rank++] = x[r][j];
        }

        uint32_t P;
        if constexpr (SINGLE) {
            P = running;
            running += tile_total;
            __syncthreads();
        } else {
            if (w == 0) {
                if (lane == 0) publish<Cnt>(p.lb, tile, tile_total, tile == 0 ? kStatePrefix : kStateAggregate);
                uint32_t excl = 0;
                if (tile != 0) {
                    excl = lookback<Cnt>(p.lb, tile);
                    if (lane == 0) publish<Cnt>(p.lb, tile, excl + tile_total, kStatePrefix);
                }
                if (lane == 0) s_prefix = excl;
            }
            __syncthreads();
            P = s_prefix;
        }

        // one contiguous run out[P .. P + tile_total)
        for (uint32_t i = threadIdx.x; i < tile_total; i += BLOCK) out[(uint64_t)P + i] = s_keep[i];
        if (!SINGLE && tile == p.num_tiles - 1 && threadIdx.x == 0) *p.count = P + tile_total;
        if constexpr (SINGLE) __syncthreads();
    }
    if (SINGLE && threadIdx.x == 0) *p.count = running;
}

}  // namespace dwpt
