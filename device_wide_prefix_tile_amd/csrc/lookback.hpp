// lookback.hpp -- inter-tile prefix by decoupled look-back over a status array.
//
// Pages cited:
//   [L7] "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
//        (UIUC ECE408 course notes, runguoli.com)
//
// The lecture's hierarchical scan [L7 concept 6 "层次化扫描（Hierarchical
// Scan）"] writes each block's total to a global array and scans it in a
// second kernel, because blocks can only see each other's global writes
// across a kernel boundary.  It names the single-kernel alternative: block
// totals plus global flags, with careful memory ordering and spinning
// ("decoupled look-back").  This file is that mechanism, in the form
// published by Merrill and Garland (2016), written for CDNA:
//
//  * Each tile owns kWords 64-bit status words.  A word holds one 32-bit
//    payload word and a 32-bit tag = epoch << 3 | flag << 2 | state, with
//    state EMPTY (0), AGGREGATE (1: the tile's own total) or PREFIX (2: the
//    fold of every element up to the end of the tile).  Each word is written
//    and read as one 64-bit agent-scope atomic, so a tag always describes
//    the payload beside it; a payload of two words is accepted only when both
//    tags agree.  No cache flush or fence is needed: the payload travels in
//    the word itself.
//  * The epoch is the call's sequence number.  Words left by earlier calls
//    carry another epoch and read as EMPTY, so the array is never cleared
//    between calls.
//  * The flag bit carries the segmented scan's "contains a head" bit; a tile
//    whose total has it set ends every later tile's look-back, like a PREFIX.
//  * A waiting wavefront polls 64 predecessors at once, one per lane, folds
//    the window right to left (earlier values on the left) and stops at the
//    nearest PREFIX.  Tiles only wait on lower tile numbers, and tile numbers
//    are handed out in the order workgroups start, so every awaited tile has
//    already started.  The wait is bounded: past `spin_limit` polls the tile
//    records an error code and carries on with what it has, so every wave
//    always exits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_ops.hpp"
#include "wave_ops.hpp"

namespace dwpt {

enum : uint32_t { kStateEmpty = 0u, kStateAggregate = 1u, kStatePrefix = 2u };
enum : uint32_t { kEpochBits = 29u };
enum : uint32_t { kErrTimeout = 1u, kErrCounter = 2u };

struct Lookback {
    uint64_t* status;    // kWords words per tile
    uint32_t* err;       // device error word (bit flags)
    uint32_t epoch;      // 1 .. 2^29 - 1
    uint32_t spin_limit; // polls before giving up
};

__device__ __forceinline__ uint32_t make_tag(uint32_t epoch, uint32_t flag, uint32_t state)
{
    return (epoch << 3) | (flag << 2) | state;
}

// Called by a single lane.
template <class Op>
__device__ __forceinline__ void publish(const Lookback& lb, uint64_t tile, typename Op::carry_t c,
                                        uint32_t state)
{
    uint32_t w[Op::kWords];
    uint32_t flag;
    Op::pack(c, w, flag);
    const uint64_t tag = (uint64_t)make_tag(lb.epoch, flag, state) << 32;
    uint64_t* dst = lb.status + tile * Op::kWords;
#pragma unroll
    for (int k = 0; k < Op::kWords; ++k)
        __hip_atomic_store(dst + k, tag | (uint64_t)w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of `tile` (fold of all earlier tiles), computed by one
// full wavefront; the result is the same in every lane.  Requires tile > 0.
template <class Op>
__device__ typename Op::carry_t lookback(const Lookback& lb, uint64_t tile)
{
    using C = typename Op::carry_t;
    const int lane = lane_id();
    const C ident = Op::carry_identity();
    C acc = ident;
    int64_t base = (int64_t)tile;  // window covers tiles [base - 64, base)
    uint32_t polls = 0;
    while (true) {
        const int64_t j = base - 64 + lane;
        bool valid = true, terminal = true;
        C val = ident;
        if (j >= 0) {
            uint32_t w[Op::kWords];
            uint32_t tag0 = 0;
            bool same = true;
            const uint64_t* src = lb.status + (uint64_t)j * Op::kWords;
#pragma unroll
            for (int k = 0; k < Op::kWords; ++k) {
                const uint64_t s = __hip_atomic_load(src + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                w[k] = (uint32_t)s;
                const uint32_t tag = (uint32_t)(s >> 32);
                if (k == 0) tag0 = tag;
                else same = same && (tag == tag0);
            }
            const uint32_t state = tag0 & 3u;
            const uint32_t flag = (tag0 >> 2) & 1u;
            valid = same && (tag0 >> 3) == lb.epoch && state != kStateEmpty;
            terminal = valid && (state == kStatePrefix || flag != 0u);
            val = Op::unpack(w, flag);
        }
        const uint64_t invalid = wave_ballot(!valid);
        const uint64_t term = wave_ballot(terminal);
        const int p = term ? 63 - __builtin_clzll(term) : -1;  // nearest terminal lane
        const uint64_t must = (p < 0) ? ~0ull : (p == 63 ? 0ull : (~0ull << (p + 1)));
        if (invalid & must) {
            if (++polls > lb.spin_limit) {
                if (lane == 0) __hip_atomic_fetch_or(lb.err, (uint32_t)kErrTimeout, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                return acc;
            }
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        C v = (lane >= p) ? val : ident;
        v = wave_inclusive_scan(v, ident, [](C a, C b) { return Op::combine_carry(a, b); });
        acc = Op::combine_carry(read_lane(v, 63), acc);
        if (p >= 0) return acc;
        base -= 64;
    }
}

}  // namespace dwpt
