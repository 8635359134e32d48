// Reduce-then-scan: the hierarchical alternative to the single-pass look-back
// scan, in three launches on the caller's stream.
//
//   1. every workgroup reduces one tile and stores the tile's total;
//   2. one workgroup scans the tile totals in tile order (exclusive), and
//      keeps the grand total;
//   3. every workgroup scans its tile again, seeded with the fold of all
//      tiles before it, and stores the result.
//
// This is the three-step hierarchical scan of "Lecture 7: 并行模式五 —— 前缀和 /
// 扫描" (concept 6: scan the blocks, scan the block sums, add them back), with
// the add-back fused into a rescan so that the intermediate per-element scan
// never goes to memory: the input is read twice and the output written once
// (12 bytes per element for 4-byte scans, against 8 for the single pass), but
// no tile ever waits for another, and the association of a float sum depends
// only on n, not on timing.  It runs behind the same entry points as the
// single pass (scan_set_multi_tile_mode(3)), as a measured alternative.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_scan.hpp"

namespace dwpt {

// Pass 1: tile `blockIdx.x` -> totals[tile].
template <class Op, int BLOCK, int ITEMS>
__global__ __launch_bounds__(BLOCK) void tile_reduce_kernel(ScanParams p, typename Op::carry_t* totals)
{
    using G = Geometry<Op, BLOCK, ITEMS>;
    using V = typename Op::value_t;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    __shared__ V s_wave[ND];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const uint32_t tile = blockIdx.x;
    const uint64_t tile_base = (uint64_t)tile * G::TILE;
    const uint64_t wave_base = tile_base + (uint64_t)w * G::WAVE_ELEMS;
    const bool vec = p.vec_ok && tile_base + G::TILE <= p.n;
    if (w < ND) {
        V x[R][VEC], lane_excl[R], round_carry[R + 1];
        uint32_t raw_head[R];
        load_wave<Op, R, VEC>(p, wave_base, vec, lane, x, raw_head);
        scan_wave<Op, R, VEC>(x, lane_excl, round_carry);
        if (lane == 0) s_wave[w] = round_carry[R];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        V total = Op::identity();
#pragma unroll
        for (int k = 0; k < ND; ++k) total = Op::combine(total, s_wave[k]);
        totals[tile] = Op::to_carry(total);
    }
}

// Pass 2: excl[t] = totals[0] + ... + totals[t-1] (tile order, the earlier
// total on the left) for t < T, and *grand = the fold of all T, by one
// workgroup: each thread folds a run of consecutive totals, the workgroup
// scans the runs' folds in order, and each thread writes its run's prefixes.
template <class Op, int BLOCK>
__global__ __launch_bounds__(BLOCK) void carry_scan_kernel(const typename Op::carry_t* totals,
                                                           typename Op::carry_t* excl, uint32_t T,
                                                           typename Op::carry_t* grand)
{
    using C = typename Op::carry_t;
    constexpr int NW = BLOCK / 64;
    __shared__ C s_wave[NW];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const C ident = Op::carry_identity();
    const auto comb = [](C a, C b) { return Op::combine_carry(a, b); };
    const uint32_t per = (T + BLOCK - 1) / BLOCK;
    const uint64_t lo = (uint64_t)threadIdx.x * per;
    const uint64_t hi = lo + per < T ? lo + per : T;
    C run = ident;
    for (uint64_t j = lo; j < hi; ++j) run = comb(run, totals[j]);
    const C incl = wave_inclusive_scan(run, ident, comb);
    if (lane == 63) s_wave[w] = incl;
    __syncthreads();
    C before = ident;  // fold of the runs of earlier wavefronts
    for (int k = 0; k < NW; ++k)
        if (k < w) before = comb(before, s_wave[k]);
    C acc = comb(before, wave_shift_up(incl, ident));
    for (uint64_t j = lo; j < hi; ++j) {
        const C t = totals[j];
        excl[j] = acc;
        acc = comb(acc, t);
    }
    if (threadIdx.x == BLOCK - 1) *grand = acc;
}

// Pass 3: tile `blockIdx.x` scanned again and seeded with excl[tile].
template <class Op, bool EXCL, int BLOCK, int ITEMS>
__global__ __launch_bounds__(BLOCK) void tile_scan_seeded_kernel(ScanParams p, const typename Op::carry_t* excl)
{
    using G = Geometry<Op, BLOCK, ITEMS>;
    using V = typename Op::value_t;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    __shared__ V s_wave[ND];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const uint32_t tile = blockIdx.x;
    const uint64_t tile_base = (uint64_t)tile * G::TILE;
    const uint64_t wave_base = tile_base + (uint64_t)w * G::WAVE_ELEMS;
    const bool vec = p.vec_ok && tile_base + G::TILE <= p.n;
    V x[R][VEC], lane_excl[R], round_carry[R + 1];
    uint32_t raw_head[R];
    if (w < ND) {
        load_wave<Op, R, VEC>(p, wave_base, vec, lane, x, raw_head);
        scan_wave<Op, R, VEC>(x, lane_excl, round_carry);
        if (lane == 0) s_wave[w] = round_carry[R];
    }
    __syncthreads();
    if (w < ND) {
        V wave_prefix = Op::identity();
#pragma unroll
        for (int k = 0; k < ND; ++k)
            if (k < w) wave_prefix = Op::combine(wave_prefix, s_wave[k]);
        apply_store<Op, EXCL, R, VEC>(p, wave_base, vec, lane, excl[tile], wave_prefix, x, lane_excl, round_carry,
                                      raw_head);
    }
}

// Compaction, pass 1: the number of kept elements of tile `blockIdx.x`.
template <typename T, int BLOCK, int ITEMS>
__global__ __launch_bounds__(BLOCK) void tile_count_kernel(ScanParams p, uint32_t* totals)
{
    using G = Geometry<OpAdd<uint32_t>, BLOCK, ITEMS>;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    __shared__ uint32_t s_wave[ND];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const uint32_t tile = blockIdx.x;
    const uint64_t tile_base = (uint64_t)tile * G::TILE;
    const bool vec = p.vec_ok && tile_base + G::TILE <= p.n;
    if (w < ND) {
        T x[R][VEC];
        uint32_t kept[R];
        load_flags<T, R, VEC>(p, tile_base + (uint64_t)w * G::WAVE_ELEMS, vec, lane, x, kept);
        uint32_t c = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) c += (uint32_t)__builtin_popcount(kept[r]);
        const auto add = [](uint32_t a, uint32_t b) { return a + b; };
        c = read_lane(wave_inclusive_scan(c, 0u, add), 63);
        if (lane == 0) s_wave[w] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t total = 0;
#pragma unroll
        for (int k = 0; k < ND; ++k) total += s_wave[k];
        totals[tile] = total;
    }
}

// Compaction, pass 3: tile `blockIdx.x` packed again and written from
// position excl[tile] on.
template <typename T, int BLOCK, int ITEMS>
__global__ __launch_bounds__(BLOCK) void compact_seeded_kernel(ScanParams p, const uint32_t* excl)
{
    using G = Geometry<OpAdd<uint32_t>, BLOCK, ITEMS>;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    __shared__ T s_keep[G::TILE];  // wavefront w packs into [w * WAVE_ELEMS, ...)
    __shared__ uint32_t s_wave[ND];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const uint32_t tile = blockIdx.x;
    const uint64_t tile_base = (uint64_t)tile * G::TILE;
    const bool vec = p.vec_ok && tile_base + G::TILE <= p.n;
    T* region = s_keep + (w < ND ? w : 0) * G::WAVE_ELEMS;
    uint32_t cnt = 0;
    if (w < ND) {
        T x[R][VEC];
        uint32_t kept[R];
        load_flags<T, R, VEC>(p, tile_base + (uint64_t)w * G::WAVE_ELEMS, vec, lane, x, kept);
        cnt = pack_wave<T, R, VEC>(x, kept, region);
        if (lane == 0) s_wave[w] = cnt;
    }
    __syncthreads();
    if (w < ND) {
        uint32_t wave_prefix = 0;
#pragma unroll
        for (int k = 0; k < ND; ++k)
            if (k < w) wave_prefix += s_wave[k];
        T* __restrict__ out = static_cast<T*>(p.out);
        const uint64_t dst = (uint64_t)excl[tile] + wave_prefix;
        for (uint32_t i = lane; i < cnt; i += 64) out[dst + i] = region[i];
    }
}

}  // namespace dwpt
