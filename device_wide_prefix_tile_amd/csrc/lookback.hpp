// lookback.hpp -- inter-tile prefix by two-level decoupled look-back.
//
// Pages cited:
//   [L7] "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
//        (UIUC ECE408 course notes, runguoli.com)
//
// The lecture's hierarchical scan [L7 concept 6 "层次化扫描（Hierarchical
// Scan）"] writes each block's total to a global array and scans it in a
// second kernel, because blocks only see each other's global writes across a
// kernel boundary.  It mentions a single-kernel alternative in which blocks
// publish their totals and flags in global memory and wait on each other,
// which works only with deliberate ordering of the memory operations and
// spin-waiting (the method published by Merrill and Garland in 2016 as
// decoupled look-back).  This file is that mechanism, reorganised for a GPU
// that keeps ~2000 tiles in flight:
//
//  * Status words.  Every tile, and every group of 64 consecutive tiles, owns
//    kWords 64-bit words.  A word holds a 49-bit payload under a 15-bit tag =
//    epoch << 3 | flag << 2 | state, with state EMPTY (0), AGGREGATE (1: the
//    fold of the tile's -- or the group's -- own elements) or PREFIX (2: the
//    fold of every element up to its end).  Words are written and read as
//    single 64-bit agent-scope atomics, so a tag always describes the payload
//    beside it; a payload of several words is accepted only when all tags
//    agree.  No cache flush or fence is needed: the payload travels in the
//    word itself.  Most carries put 32 bits in each word; the float32 sum's
//    double carry fits one word (scan_ops.hpp, OpAdd<float>::pack), which
//    halves the status traffic of that scan (float32 add 2^28: 336.7 ->
//    334.7 us measured with a one-word carry).
//  * Epochs.  The tag carries the call's sequence number modulo 2^12 (0 is
//    never used); words left by earlier calls read as EMPTY, so the arrays
//    are cleared only when the number wraps, every 4095 calls.
//  * Segment heads.  The flag bit carries the segmented scan's "contains a
//    head" bit; a word with it set ends a look-back like a PREFIX does.
//  * Two levels.  Tile t of group g first folds the tiles of its own group
//    before it (one 64-lane window), then the groups before g, 64 groups
//    (4096 tiles) per window, until it meets a PREFIX or the start (the
//    second group's tiles fold the first group's 64 tile words instead).  The
//    last tile of a group publishes the group's AGGREGATE as soon as its
//    in-group fold is done and the group's PREFIX with its own.  A flat look-back would
//    make every tile walk back through all unresolved tiles in flight, 64 per
//    status round trip, and the polling traffic then competes with the data;
//    two levels bound the walk to about two windows.
//  * A wavefront of its own.  The look-back is done by a wavefront that
//    loads no data, so it walks the predecessors while the tile's own loads
//    are in flight; the data wavefronts publish the tile's AGGREGATE the
//    moment their totals are combined (the last one to arrive does it), and
//    the look-back wavefront publishes the PREFIX after that publication has
//    been performed.
//  * Progress.  Tiles wait only on lower tile numbers and groups made of
//    them; tile numbers are handed out in the order workgroups start, so
//    every awaited tile has started, and an AGGREGATE never waits for
//    anything but loads and lower tiles.  Waits are bounded: past
//    `spin_limit` polls a tile records an error and carries on with what it
//    has, so every wave always exits.  A wait that gives up also marks the
//    launch as aborted (the abort word takes the launch's epoch); every other
//    wait of the launch, on status words or on LDS, looks at that word now
//    and then and gives up at once when it is set, so one lost total ends the
//    launch in microseconds per remaining wait, not a full budget each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_ops.hpp"
#include "wave_ops.hpp"

namespace dwpt {

enum : uint32_t { kStateEmpty = 0u, kStateAggregate = 1u, kStatePrefix = 2u };
enum : uint32_t { kEpochBits = 12u };
constexpr int kPayloadBits = 49;  // status word: tag << kPayloadBits | payload
constexpr uint64_t kPayloadMask = (1ull << kPayloadBits) - 1;
enum : uint32_t { kErrTimeout = 1u, kErrCounter = 2u };
enum : int { kGroupShift = 6 };  // 64 tiles per group

#ifndef DWPT_LB_SLEEP
#define DWPT_LB_SLEEP 1  // s_sleep units (64 clocks) between polls
#endif
// Persistent kernel: s_sleep between polls of a published prefix, and the
// spacing of published prefixes and of tile totals, in entries.  With one
// prefix per 128-byte line the resolver's stores and the workgroups' polls
// no longer meet on shared lines (measured: 403 -> 374 us for the float32
// add at 2^28); spacing the totals gave nothing, and fewer, slower polls
// are a little better than fast ones (a second poll kept in flight was
// measured 5% slower).
#ifndef DWPT_FETCH_SLEEP
#define DWPT_FETCH_SLEEP 8
#endif
#ifndef DWPT_PREFIX_PAD
#define DWPT_PREFIX_PAD 16
#endif
#ifndef DWPT_AGG_PAD
#define DWPT_AGG_PAD 1
#endif


struct Lookback {
    uint64_t* status;    // kWords words per tile
    uint64_t* groups;    // kWords words per group of 64 tiles
    uint32_t* err;       // device error word (bit flags)
    uint32_t* abort;     // epoch of the last launch that gave up a wait
    uint32_t epoch;      // 1 .. 2^12 - 1
    uint32_t spin_limit; // polls before giving up
};

// Bounded waits.  Every failed poll counts; past the budget the wait gives
// up, records the timeout in the error word and marks the launch aborted.
// Every kAbortCheck polls a wait also reads the abort word and gives up at
// once if another wait of this launch already did (waits that succeed
// normally take far fewer polls than that, so the check costs nothing then).
// LDS waits poll about 16 times as often as status-word waits (no memory
// round trip, a shorter sleep), so their budget is 16 times larger: about
// the same wall time.
#ifndef DWPT_ABORT_CHECK
#define DWPT_ABORT_CHECK 64
#endif
enum : uint32_t { kAbortCheck = DWPT_ABORT_CHECK, kLdsPollScale = 16u };

// Called by the whole wavefront (the result is uniform).
__device__ __forceinline__ bool launch_aborted(const Lookback& lb)
{
    const uint32_t a = __hip_atomic_load(lb.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)a) == lb.epoch;
}

// One failed poll of a wavefront's bounded wait (wave-uniform `polls`):
// true once the wait must give up.
__device__ __forceinline__ bool give_up(const Lookback& lb, uint64_t& polls, uint64_t limit)
{
    ++polls;
    if (polls > limit) {
        if (lane_id() == 0) {
            __hip_atomic_fetch_or(lb.err, (uint32_t)kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(lb.abort, lb.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return true;
    }
    if (polls % kAbortCheck == 0 && launch_aborted(lb)) {
        polls = limit + 1;  // sticky: later waits sharing this counter give up at once
        return true;
    }
    return false;
}

__device__ __forceinline__ uint64_t lds_poll_limit(const Lookback& lb)
{
    return (uint64_t)lb.spin_limit * kLdsPollScale;
}

__device__ __forceinline__ uint32_t make_tag(uint32_t epoch, uint32_t flag, uint32_t state)
{
    return (epoch << 3) | (flag << 2) | state;
}

__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> kPayloadBits); }

// Called by a single lane.
template <class Op>
__device__ __forceinline__ void publish(const Lookback& lb, uint64_t* arr, uint64_t idx, typename Op::carry_t c,
                                        uint32_t state)
{
    uint64_t w[Op::kWords];
    uint32_t flag;
    Op::pack(c, w, flag);
    const uint64_t tag = (uint64_t)make_tag(lb.epoch, flag, state) << kPayloadBits;
    uint64_t* dst = arr + idx * Op::kWords;
#pragma unroll
    for (int k = 0; k < Op::kWords; ++k)
        __hip_atomic_store(dst + k, tag | w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

enum : int { kWinFound = 0, kWinBoundary = 1, kWinNone = 2, kWinTimeout = 3 };

// Folds the 64 entries top-63 .. top of `arr` (lane l <-> entry top-63+l),
// earlier entries on the left, starting at the highest terminal entry: a
// PREFIX, a flagged AGGREGATE, or an entry below `lo` (a boundary that
// contributes the identity).  Waits until every entry above that point is
// valid; an entry already seen valid is not read again.  Returns how the
// fold ended; `out` is the same in every lane.
template <class Op>
__device__ int fold_window(const Lookback& lb, const uint64_t* arr, int64_t top, int64_t lo,
                           typename Op::carry_t& out, uint64_t& polls)
{
    using C = typename Op::carry_t;
    const int lane = lane_id();
    const C ident = Op::carry_identity();
    const int64_t j = top - 63 + lane;
    const bool boundary = j < lo;
    bool have = boundary, term = boundary;
    C val = ident;
    while (true) {
        if (!have) {
            uint64_t w[Op::kWords];
            uint32_t tag0 = 0;
            bool same = true;
            const uint64_t* src = arr + (uint64_t)j * Op::kWords;
#pragma unroll
            for (int q = 0; q < Op::kWords; ++q) {
                const uint64_t s = __hip_atomic_load(src + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                w[q] = s & kPayloadMask;
                const uint32_t tag = word_tag(s);
                if (q == 0) tag0 = tag;
                else same = same && (tag == tag0);
            }
            const uint32_t state = tag0 & 3u;
            const uint32_t flag = (tag0 >> 2) & 1u;
            if (same && (tag0 >> 3) == lb.epoch && state != kStateEmpty) {
                have = true;
                term = (state == kStatePrefix) || flag != 0u;
                val = Op::unpack(w, flag);
            }
        }
        const uint64_t tmask = wave_ballot(term);
        const int p = tmask ? 63 - __builtin_clzll(tmask) : -1;  // highest terminal lane
        const uint64_t from_p = (p < 0) ? ~0ull : (~0ull << p);
        if (wave_ballot(!have) & from_p) {
            if (give_up(lb, polls, lb.spin_limit)) {
                out = ident;
                return kWinTimeout;
            }
            __builtin_amdgcn_s_sleep(DWPT_LB_SLEEP);
            continue;
        }
        C v = (lane >= p) ? val : ident;
        v = wave_inclusive_scan(v, ident, [](C a, C b) { return Op::combine_carry(a, b); });
        out = read_lane(v, 63);
        if (p < 0) return kWinNone;
        return ((wave_ballot(boundary) >> p) & 1ull) ? kWinBoundary : kWinFound;
    }
}

// Wide variant of fold_window: SPAN consecutive entries per lane, lanes in
// entry order, so one poll covers the 64 * SPAN entries top-64*SPAN+1 .. top.
// All loads of a poll are issued together, so the window costs one memory
// round trip however wide it is.  Same results as fold_window.
template <class Op, int SPAN>
__device__ int fold_window_wide(const Lookback& lb, const uint64_t* arr, int64_t top, int64_t lo,
                                typename Op::carry_t& out, uint64_t& polls)
{
    using C = typename Op::carry_t;
    const int lane = lane_id();
    const C ident = Op::carry_identity();
    const int64_t j0 = top - 64 * SPAN + 1 + (int64_t)lane * SPAN;
    bool have[SPAN], term[SPAN];
    C val[SPAN];
#pragma unroll
    for (int k = 0; k < SPAN; ++k) {
        have[k] = term[k] = (j0 + k < lo);  // below lo: boundary, the identity
        val[k] = ident;
    }
    while (true) {
        uint64_t raw[SPAN][Op::kWords];
#pragma unroll
        for (int k = 0; k < SPAN; ++k)
            if (!have[k]) {
                const uint64_t* src = arr + (uint64_t)(j0 + k) * Op::kWords;
#pragma unroll
                for (int q = 0; q < Op::kWords; ++q)
                    raw[k][q] = __hip_atomic_load(src + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
        for (int k = 0; k < SPAN; ++k)
            if (!have[k]) {
                uint64_t w[Op::kWords];
                const uint32_t tag0 = word_tag(raw[k][0]);
                bool same = true;
#pragma unroll
                for (int q = 0; q < Op::kWords; ++q) {
                    w[q] = raw[k][q] & kPayloadMask;
                    same = same && word_tag(raw[k][q]) == tag0;
                }
                const uint32_t state = tag0 & 3u;
                const uint32_t flag = (tag0 >> 2) & 1u;
                if (same && (tag0 >> 3) == lb.epoch && state != kStateEmpty) {
                    have[k] = true;
                    term[k] = (state == kStatePrefix) || flag != 0u;
                    val[k] = Op::unpack(w, flag);
                }
            }
        // per lane: the last terminal entry, and whether everything after it
        // (everything, without one) is valid
        int last_term = -1;
        bool ok = true;
#pragma unroll
        for (int k = 0; k < SPAN; ++k)
            if (term[k]) last_term = k;
#pragma unroll
        for (int k = 0; k < SPAN; ++k)
            if (k > last_term && !have[k]) ok = false;
        const uint64_t tmask = wave_ballot(last_term >= 0);
        const int p = tmask ? 63 - __builtin_clzll(tmask) : -1;  // lane with the nearest terminal entry
        const uint64_t from_p = (p < 0) ? ~0ull : (~0ull << p);
        if (wave_ballot(!ok) & from_p) {
            if (give_up(lb, polls, lb.spin_limit)) {
                out = ident;
                return kWinTimeout;
            }
            __builtin_amdgcn_s_sleep(DWPT_LB_SLEEP);
            continue;
        }
        C v = ident;
#pragma unroll
        for (int k = 0; k < SPAN; ++k)
            if (lane > p || (lane == p && k >= last_term)) v = Op::combine_carry(v, val[k]);
        v = wave_inclusive_scan(v, ident, [](C a, C b) { return Op::combine_carry(a, b); });
        out = read_lane(v, 63);
        if (p < 0) return kWinNone;
        // boundary entries are below lo; in lane p, entry last_term
        const bool boundary = j0 + last_term < lo;
        return ((wave_ballot(boundary) >> p) & 1ull) ? kWinBoundary : kWinFound;
    }
}

// Exclusive prefix of `tile` from tile statuses alone: fold windows of
// 64 * SPAN predecessors back to the nearest PREFIX (or the start).
template <class Op, int SPAN>
__device__ typename Op::carry_t walk_tiles(const Lookback& lb, int64_t tile, uint64_t& polls)
{
    using C = typename Op::carry_t;
    C acc = Op::carry_identity();
    for (int64_t top = tile - 1; top >= 0; top -= 64 * SPAN) {
        C w;
        const int r = fold_window_wide<Op, SPAN>(lb, lb.status, top, 0, w, polls);
        acc = Op::combine_carry(w, acc);
        if (r != kWinNone) break;
    }
    return acc;
}

// ------------------------------------------------------------------ resolver
// Streaming resolver of the persistent kernel: one wavefront that scans the
// published tile totals in tile order, 64 * SPAN at a time, and publishes
// every tile's exclusive prefix (state PREFIX in `excl`) as soon as all
// totals before it are in.  Entries past `num_tiles` count as the identity.
// Only totals not yet seen are read again.  (Keeping a second poll in flight
// was measured slower: the extra status reads cost more than the earlier
// sighting gains.)  Returns the fold of every tile total.
template <class Op, int SPAN>
__device__ typename Op::carry_t resolve_stream(const Lookback& lb, const uint64_t* agg, uint64_t* excl,
                                               uint32_t num_tiles)
{
    using C = typename Op::carry_t;
    constexpr int W = 64 * SPAN;
    const int lane = lane_id();
    const C ident = Op::carry_identity();
    C carry = ident;
    uint64_t polls = 0;  // not reset per window: once the resolver gave up, it gives up at once
    for (uint64_t B = 0; B < num_tiles; B += W) {
        const uint64_t j0 = B + (uint64_t)lane * SPAN;
        bool have[SPAN];
        C val[SPAN];
#pragma unroll
        for (int k = 0; k < SPAN; ++k) {
            have[k] = j0 + k >= num_tiles;
            val[k] = ident;
        }
        const uint32_t want = (uint32_t)((num_tiles - B) < (uint64_t)W ? (num_tiles - B) : (uint64_t)W);
        uint32_t done = 0;  // entries [B, B + done) already published
        while (true) {
            uint64_t raw[SPAN][Op::kWords];
#pragma unroll
            for (int k = 0; k < SPAN; ++k)
                if (!have[k])
#pragma unroll
                    for (int q = 0; q < Op::kWords; ++q)
                        raw[k][q] = __hip_atomic_load(agg + (j0 + k) * (Op::kWords * DWPT_AGG_PAD) + q, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int k = 0; k < SPAN; ++k)
                if (!have[k]) {
                    uint64_t w[Op::kWords];
                    const uint32_t tag0 = word_tag(raw[k][0]);
                    bool same = true;
#pragma unroll
                    for (int q = 0; q < Op::kWords; ++q) {
                        w[q] = raw[k][q] & kPayloadMask;
                        same = same && word_tag(raw[k][q]) == tag0;
                    }
                    if (same && (tag0 >> 3) == lb.epoch && (tag0 & 3u) != kStateEmpty) {
                        have[k] = true;
                        val[k] = Op::unpack(w, (tag0 >> 2) & 1u);
                    }
                }
            // leading run of available totals, in tile order
            int first_missing = SPAN;
#pragma unroll
            for (int k = SPAN - 1; k >= 0; --k)
                if (!have[k]) first_missing = k;
            const uint64_t gaps = wave_ballot(first_missing < SPAN);
            const int gl = gaps ? __builtin_ctzll(gaps) : 64;
            const uint32_t ready = gaps ? (uint32_t)(gl * SPAN) + (uint32_t)__builtin_amdgcn_readlane(first_missing, gl)
                                        : (uint32_t)W;
            const uint32_t upto = ready < want ? ready : want;
            if (upto > done) {
                // exclusive prefixes of the available run: lane folds, a
                // wavefront scan, then each lane's own entries
                C lane_total = ident;
#pragma unroll
                for (int k = 0; k < SPAN; ++k)
                    if ((uint32_t)(lane * SPAN + k) < upto) lane_total = Op::combine_carry(lane_total, val[k]);
                const C incl = wave_inclusive_scan(lane_total, ident, [](C a, C b) { return Op::combine_carry(a, b); });
                C run = Op::combine_carry(carry, wave_shift_up(incl, ident));
#pragma unroll
                for (int k = 0; k < SPAN; ++k) {
                    const uint32_t idx = (uint32_t)(lane * SPAN + k);
                    if (idx >= done && idx < upto) publish<Op>(lb, excl, (j0 + k) * DWPT_PREFIX_PAD, run, kStatePrefix);
                    run = Op::combine_carry(run, val[k]);
                }
                done = upto;
                if (done == want) {
                    carry = Op::combine_carry(carry, read_lane(incl, 63));
                    break;
                }
            }
            if (give_up(lb, polls, lb.spin_limit)) {
                // count the missing totals as the identity, so that every
                // waiting tile still gets a (wrong) prefix and exits
#pragma unroll
                for (int k = 0; k < SPAN; ++k) have[k] = true;
                continue;
            }
            __builtin_amdgcn_s_sleep(DWPT_LB_SLEEP);
        }
    }
    return carry;
}


template <class Op>
__device__ __forceinline__ void read_words(const uint64_t* src, uint64_t (&raw)[Op::kWords])
{
#pragma unroll
    for (int q = 0; q < Op::kWords; ++q) raw[q] = __hip_atomic_load(src + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True (and the carry in `out`) when the words hold this call's PREFIX entry.
template <class Op>
__device__ __forceinline__ bool prefix_ready(const Lookback& lb, const uint64_t (&raw)[Op::kWords],
                                             typename Op::carry_t& out)
{
    uint64_t w[Op::kWords];
    const uint32_t tag0 = word_tag(raw[0]);
    bool same = true;
#pragma unroll
    for (int q = 0; q < Op::kWords; ++q) {
        w[q] = raw[q] & kPayloadMask;
        same = same && word_tag(raw[q]) == tag0;
    }
    if (!(same && (tag0 >> 3) == lb.epoch && (tag0 & 3u) == kStatePrefix)) return false;
    out = Op::unpack(w, (tag0 >> 2) & 1u);
    return true;
}

// The exclusive prefix of `tile` published by the resolver (every lane
// reads the same words; the result is uniform).  `polls` is the caller's
// counter: reset per tile while within budget, so each tile has the whole
// budget, but once a wait gave up every later one gives up after one read.
template <class Op>
__device__ typename Op::carry_t wait_excl(const Lookback& lb, const uint64_t* excl, uint64_t tile, uint64_t& polls)
{
    const uint64_t* src = excl + tile * (Op::kWords * DWPT_PREFIX_PAD);
    typename Op::carry_t out;
    if (polls <= lb.spin_limit) polls = 0;
    while (true) {
        uint64_t raw[Op::kWords];
        read_words<Op>(src, raw);
        if (prefix_ready<Op>(lb, raw, out)) return out;
        if (give_up(lb, polls, lb.spin_limit)) return Op::carry_identity();
        __builtin_amdgcn_s_sleep(DWPT_FETCH_SLEEP);
    }
}

// Fold of the groups g-1, g-2, ... back to the nearest PREFIX (or the start).
template <class Op>
__device__ typename Op::carry_t walk_groups(const Lookback& lb, int64_t g, uint64_t& polls)
{
    using C = typename Op::carry_t;
    C acc = Op::carry_identity();
    for (int64_t top = g - 1; top >= 0; top -= 64) {
        C w;
        const int r = fold_window<Op>(lb, lb.groups, top, 0, w, polls);
        acc = Op::combine_carry(w, acc);
        if (r != kWinNone) break;
    }
    return acc;
}

// Publication whose completion is awaited: an exchange returns only once it
// has been performed at the device coherence point, so a later store to the
// same word by another wavefront cannot overtake it.
template <class Op>
__device__ __forceinline__ void publish_acked(const Lookback& lb, uint64_t* arr, uint64_t idx,
                                              typename Op::carry_t c, uint32_t state)
{
    uint64_t w[Op::kWords];
    uint32_t flag;
    Op::pack(c, w, flag);
    const uint64_t tag = (uint64_t)make_tag(lb.epoch, flag, state) << kPayloadBits;
    uint64_t* dst = arr + idx * Op::kWords;
    uint64_t sink = 0;
#pragma unroll
    for (int k = 0; k < Op::kWords; ++k)
        sink ^= __hip_atomic_exchange(dst + k, tag | w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"((uint32_t)sink), "v"((uint32_t)(sink >> 32)));
}

// Workgroup-local hand-over of the tile total from the data wavefronts to
// the look-back wavefront (LDS, workgroup scope).
struct TileHandover {
    uint32_t arrived;      // data wavefronts that have stored their total
    uint32_t total_ready;  // set once the tile total is stored and published
};

// Bounded like every other wait; on giving up the caller goes on with
// whatever the LDS holds (the launch's results are then wrong and flagged).
__device__ __forceinline__ void wait_total(const Lookback& lb, TileHandover* h)
{
    uint64_t polls = 0;
    const uint64_t limit = lds_poll_limit(lb);
    while (__hip_atomic_load(&h->total_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u) {
        if (give_up(lb, polls, limit)) return;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Look-back wavefront of tile `tile` (a full wavefront; result uniform).
// Runs while the data wavefronts are still loading: it folds the earlier
// tiles of the group, publishes the group's AGGREGATE if the tile closes a
// group, walks the earlier groups, then -- once the tile total `*total` is
// handed over -- publishes the tile's (and group's) PREFIX.  Returns the
// exclusive prefix of the tile.  `known`: the data wavefronts already
// published the tile's PREFIX (first tile, or a tile holding a segment head).
template <class Op>
__device__ typename Op::carry_t lookback_wave(const Lookback& lb, uint32_t tile, TileHandover* h,
                                              const typename Op::carry_t* total, const bool* known)
{
    using C = typename Op::carry_t;
    const int lane = lane_id();
    const int64_t g = (int64_t)(tile >> kGroupShift);
    const bool last_in_group = (tile & 63u) == 63u;
    uint64_t polls = 0;

    C acc;
    const int r = fold_window<Op>(lb, lb.status, (int64_t)tile - 1, g << kGroupShift, acc, polls);
    if (r == kWinBoundary && g > 0) {
        if (last_in_group) {
            wait_total(lb, h);
            if (lane == 0) publish<Op>(lb, lb.groups, (uint64_t)g, Op::combine_carry(acc, *total), kStateAggregate);
        }
        if (g == 1) {
            // the first group has no AGGREGATE of its own (its PREFIX comes from
            // its last tile's look-back, one round trip after that tile's
            // total): the tiles of the second group fold its 64 tile words
            // instead (int32 add at 65-128 tiles: the step of ~1 us at 64 -> 65
            // tiles, 2^20 elements 7.6 -> 6.7 us)
            C w0;
            (void)fold_window<Op>(lb, lb.status, (int64_t)(1 << kGroupShift) - 1, 0, w0, polls);
            acc = Op::combine_carry(w0, acc);
        } else {
            acc = Op::combine_carry(walk_groups<Op>(lb, g, polls), acc);
        }
    }
    wait_total(lb, h);
    if (lane == 0) {
        const C incl = Op::combine_carry(acc, *total);
        if (!*known) publish<Op>(lb, lb.status, tile, incl, kStatePrefix);
        if (last_in_group) publish<Op>(lb, lb.groups, (uint64_t)g, incl, kStatePrefix);
    }
    return acc;
}

}  // namespace dwpt
