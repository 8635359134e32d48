// tile_scan.hpp -- single-pass tile scan and fused stream compaction (gfx950).
//
// Pages cited:
//   [L7]    "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
//           (UIUC ECE408 course notes, runguoli.com)
//   [PMPP9] "第9章并行模式：前缀和 - Scan算法" (PMPP chapter 9 notes, bittern.cn)
//
// One workgroup scans one tile of TILE = ND * 64 * ITEMS elements, with ND =
// BLOCK/64 - 1 data wavefronts and one look-back wavefront:
//   1. take the next tile number from a counter (start order, not hardware
//      order);
//   2. load the tile with 16-byte loads: data wavefront w owns 64 * ITEMS
//      consecutive elements, in R = ITEMS / VEC rounds of 64 * VEC elements,
//      lane l holding VEC consecutive elements of each round, so every load
//      instruction of a wavefront reads 1 KiB of contiguous memory
//      (elements wider than 16 bytes: K 16-byte loads per lane and round,
//      which the persistent kernel issues chunk by chunk instead);
//   3. scan each lane's VEC elements serially in registers (thread
//      coarsening, [L7 concept 6 and its kernel-2 register array]);
//   4. scan the lane totals across the wavefront with DPP (wave_ops.hpp);
//   5. combine the wavefront totals through LDS: the last data wavefront to
//      arrive forms the tile total and publishes it;
//   6. meanwhile the look-back wavefront has been folding the earlier tiles'
//      published totals (two-level decoupled look-back, lookback.hpp); it
//      publishes the tile's inclusive prefix -- this replaces the
//      hierarchical scan's second and third kernels [L7 concept 6], so the
//      data cross HBM once each way;
//   7. after one barrier, apply the prefix and store with 16-byte stores.
// Exclusive scans put the identity at y[0] and use the value before each
// element [L7 concept 1; PMPP9 §9.1].  The tail tile pads with the identity
// in registers and never stores the padding.  In SINGLE mode one workgroup
// walks all tiles in order and carries the prefix in registers instead of
// using the status array (the small-n path: no workspace, no atomics).
//
// Large inputs run the persistent kernel (tile_scan_persistent): as many
// workgroups as fit stay resident and pipeline several tiles each, a
// resolver workgroup turns the published tile totals into prefixes in tile
// order, and the same steps 2-7 run per tile.  There, operators with
// expensive combines keep each lane's elements in element order ("blocked
// lane layout", exchanged through LDS after the loads and before the
// stores), so that a tile needs one wavefront scan instead of R.
//
// Compaction [L7 concept 2 "扫描的典型应用"; PMPP9 §9.6]: the predicate
// x > 0 is evaluated in registers, the 0/1 flags are scanned the same way
// (uint32 count), each wavefront packs its kept elements in LDS in order and
// writes them out as one contiguous run at the tile's prefix count plus the
// counts of the earlier wavefronts, so flags and positions never touch HBM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
    uint32_t* pipe_ctr;    // persistent kernel: next tile, roles taken, workgroups retired (kCtrStride apart)
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

// Build-time tuning switches (chosen by measurement; see the defaults).
#ifndef DWPT_NT_LOADS
#define DWPT_NT_LOADS 1   // streaming (non-temporal) hint on tile loads
#endif
#ifndef DWPT_NT_STORES
#define DWPT_NT_STORES 1  // streaming (non-temporal) hint on tile stores
#endif
#ifndef DWPT_STATIC_TILES
#define DWPT_STATIC_TILES 0  // 1: tile number = workgroup index instead of a counter
#endif

// One lane's VEC consecutive elements: one 16-byte access, or K of them for
// elements that do not divide 16 bytes (3x3 matrices: 4 x 36 bytes = K = 9).
template <typename E, int VEC>
__device__ __forceinline__ void load_vec(const E* p, E (&e)[VEC])
{
    constexpr int K = (int)sizeof(E) * VEC / 16;
    static_assert(sizeof(E) * VEC % 16 == 0, "whole 16-byte chunks");
    u32x4 v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
#if DWPT_NT_LOADS
        v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + k);
#else
        v[k] = reinterpret_cast<const u32x4*>(p)[k];
#endif
    }
    __builtin_memcpy(e, v, 16 * K);
}
template <typename E, int VEC>
__device__ __forceinline__ void store_vec(E* p, const E (&e)[VEC])
{
    constexpr int K = (int)sizeof(E) * VEC / 16;
    static_assert(sizeof(E) * VEC % 16 == 0, "whole 16-byte chunks");
    u32x4 v[K];
    __builtin_memcpy(v, e, 16 * K);
#pragma unroll
    for (int k = 0; k < K; ++k) {
#if DWPT_NT_STORES
        __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(p) + k);
#else
        reinterpret_cast<u32x4*>(p)[k] = v[k];
#endif
    }
}

// Whole-tile stores of the round-order path (apply_store) go through a buffer
// descriptor of the wavefront's output share, so that their cache policy can
// be set: streaming (nt) plus sc1, measured 1.6% faster than the streaming
// hint alone (float32 add at 2^28: 340.0 against 345.6 us; int32 add 335.9
// against 340.4), with identical results; nt alone through the same path
// gained nothing.  The descriptor's base is made wavefront-uniform, so it
// lives in scalar registers.  Compaction's packed stores and most
// blocked-layout stores keep the plain streaming hint (see BlockedStorePolicy).
#ifndef DWPT_STORE_POLICY
#define DWPT_STORE_POLICY (DWPT_NT_STORES ? 18 : 0)  // cache-policy bits: 2 nt, 16 sc1 (1 sc0)
#endif
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* base)
{
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    // raw buffer, no stride, no range limit below 4 GiB of offset; the gfx9 format word
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, -1, 0x00020000);
}
// One lane's VEC elements (K 16-byte chunks) at byte_off from the descriptor's base.
template <typename E, int VEC>
__device__ __forceinline__ void store_vec_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_off, const E (&e)[VEC])
{
    constexpr int K = (int)sizeof(E) * VEC / 16;
    static_assert(sizeof(E) * VEC % 16 == 0, "whole 16-byte chunks");
    u32x4 v[K];
    __builtin_memcpy(v, e, 16 * K);
#pragma unroll
    for (int k = 0; k < K; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(v[k], rsrc, byte_off + 16u * k, 0, DWPT_STORE_POLICY);
}

// Tile number of this workgroup: taken from a counter in the order
// workgroups start, so a tile only ever waits on tiles that have started.
// Returns num_tiles (and records an error) if the counter is out of step.
__device__ __forceinline__ uint32_t take_tile(const ScanParams& p, uint32_t* s_tile)
{
#if DWPT_STATIC_TILES
    (void)s_tile;
    __syncthreads();
    return blockIdx.x;
#else
    if (threadIdx.x == 0)
        *s_tile = __hip_atomic_fetch_add(p.tile_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - p.ctr_base;
    __syncthreads();
    const uint32_t tile = *s_tile;
    if (tile >= p.num_tiles && threadIdx.x == 0)
        __hip_atomic_fetch_or(p.lb.err, (uint32_t)kErrCounter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return tile;
#endif
}

// ------------------------------------------------------------------ pieces
// Elements per lane and round: one 16-byte chunk's worth, or for elements
// larger than 16 bytes the fewest that fill whole chunks (K of them).
template <typename E>
struct VecShape {
    static constexpr int VEC = sizeof(E) <= 16 ? 16 / (int)sizeof(E) : sizeof(E) % 16 == 0 ? 1
                               : sizeof(E) % 8 == 0                  ? 2
                                                                     : 4;
    static constexpr int K = (int)sizeof(E) * VEC / 16;
    static_assert(sizeof(E) % 4 == 0 && sizeof(E) * VEC % 16 == 0, "whole 16-byte chunks");
};

// Tile geometry: ND data wavefronts of 64 lanes, each lane holding R rounds
// of VEC consecutive elements (ITEMS = R * VEC per lane); the last wavefront
// of the workgroup does the look-back.
template <class Op, int BLOCK, int ITEMS>
struct Geometry {
    using E = typename Op::elem_t;
    static constexpr int VEC = VecShape<E>::VEC;
    static constexpr int K = VecShape<E>::K;  // 16-byte chunks per round and lane
    static constexpr int R = ITEMS / VEC;
    static constexpr int NW = BLOCK / 64;
    static constexpr int ND = NW - 1;
    static constexpr int WAVE_ELEMS = 64 * ITEMS;
    static constexpr int TILE = ND * WAVE_ELEMS;
    static_assert(ITEMS % VEC == 0 && BLOCK % 64 == 0 && NW >= 2, "tile shape");
};

// Loads one wavefront's share of a tile (2): 16-byte loads when the whole
// tile is in range and the pointers are aligned, else element loads with the
// identity past n.  raw_head[r] bit j: element j of round r is a segment head.
template <class Op, int R, int VEC>
__device__ __forceinline__ void load_wave(const ScanParams& p, uint64_t wave_base, bool vec, int lane,
                                          typename Op::value_t (&x)[R][VEC], uint32_t (&raw_head)[R])
{
    using E = typename Op::elem_t;
    constexpr bool SEG = IsSeg<Op>::value;
    const E* __restrict__ in = static_cast<const E*>(p.in);
    if (vec) {
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
        // a tile that reaches past n: lanes whose VEC elements are all below n
        // still take one 16-byte access, the rest go element by element
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint64_t i0 = wave_base + (uint64_t)(r * 64 + lane) * VEC;
            uint32_t hb = 0;
            if (p.vec_ok && i0 + VEC <= p.n) {
                E e[VEC];
                load_vec<E, VEC>(in + i0, e);
                if constexpr (SEG) {
                    const uint32_t h4 = *reinterpret_cast<const uint32_t*>(p.heads + i0);
#pragma unroll
                    for (int j = 0; j < VEC; ++j) hb |= ((h4 >> (8 * j)) & 0xFFu) ? (1u << j) : 0u;
                    if (i0 == 0) hb |= 1u;
                }
#pragma unroll
                for (int j = 0; j < VEC; ++j) x[r][j] = make_value<Op>(e[j], (hb >> j) & 1u);
            } else {
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const uint64_t i = i0 + j;
                    if (i < p.n) {
                        uint32_t h = 0;
                        if constexpr (SEG) h = (i == 0 || p.heads[i]) ? 1u : 0u;
                        hb |= h << j;
                        x[r][j] = make_value<Op>(in[i], h);
                    } else {
                        x[r][j] = Op::identity();
                    }
                }
            }
            raw_head[r] = hb;
        }
    }
}

// Inclusive wavefront scan under the operator (float32 add takes the variant
// with fused DPP broadcasts, wave_ops.hpp).
template <class Op>
__device__ __forceinline__ typename Op::value_t op_wave_scan(typename Op::value_t v)
{
    using V = typename Op::value_t;
    if constexpr (std::is_same<Op, OpAdd<float>>::value) return wave_inclusive_scan_fadd(v);
    else return wave_inclusive_scan(v, Op::identity(), [](V a, V b) { return Op::combine(a, b); });
}

// Serial scan of each lane's elements (3) and wavefront scans of the lane
// totals (4): afterwards x holds in-lane inclusive prefixes, lane_excl[r]
// the fold of the lower lanes' round-r totals and round_carry[r] the fold of
// the wavefront's rounds before r (round_carry[R]: the wavefront total).
template <class Op, int R, int VEC>
__device__ __forceinline__ void scan_wave(typename Op::value_t (&x)[R][VEC], typename Op::value_t (&lane_excl)[R],
                                          typename Op::value_t (&round_carry)[R + 1])
{
    using V = typename Op::value_t;
    const V ident = Op::identity();
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 1; j < VEC; ++j) x[r][j] = Op::combine(x[r][j - 1], x[r][j]);
    round_carry[0] = ident;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const V incl = op_wave_scan<Op>(x[r][VEC - 1]);
        lane_excl[r] = wave_shift_up(incl, ident);
        round_carry[r + 1] = Op::combine(round_carry[r], read_lane(incl, 63));
    }
}

// Applies the prefix of everything before the lane's elements and stores (7).
template <class Op, bool EXCL, int R, int VEC>
__device__ __forceinline__ void apply_store(const ScanParams& p, uint64_t wave_base, bool vec, int lane,
                                            typename Op::carry_t P, typename Op::value_t wave_prefix,
                                            const typename Op::value_t (&x)[R][VEC],
                                            const typename Op::value_t (&lane_excl)[R],
                                            const typename Op::value_t (&round_carry)[R + 1],
                                            const uint32_t (&raw_head)[R])
{
    using E = typename Op::elem_t;
    using V = typename Op::value_t;
    constexpr bool SEG = IsSeg<Op>::value;
    const V ident = Op::identity();
    E* __restrict__ out = static_cast<E*>(p.out);
    const __amdgpu_buffer_rsrc_t rsrc = wave_rsrc(out + wave_base);
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
        if (vec) {
            store_vec_buf<E, VEC>(rsrc, (uint32_t)((r * 64 + lane) * VEC * sizeof(E)), e);
        } else if (p.vec_ok && i0 + VEC <= p.n) {  // partial tile, this lane's elements all below n
            store_vec<E, VEC>(out + i0, e);
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                if (i0 + j < p.n) out[i0 + j] = e[j];
        }
    }
}

// Data wavefront w hands its total over; the last one to arrive combines all
// totals, publishes the tile's AGGREGATE (or PREFIX, when it is already
// known) and releases the look-back wavefront.
template <class Op, int ND>
__device__ __forceinline__ void hand_over(const ScanParams& p, uint32_t tile, int w, int lane,
                                          typename Op::value_t wave_total, typename Op::value_t* s_wave,
                                          TileHandover* h, typename Op::carry_t* s_total, bool* s_known)
{
    using V = typename Op::value_t;
    if (lane == 0) s_wave[w] = wave_total;
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(&h->arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)(ND - 1)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // every lane sees the other totals
    V total = Op::identity();
#pragma unroll
    for (int k = 0; k < ND; ++k) total = Op::combine(total, s_wave[k]);
    if (lane == 0) {
        const bool known = (tile == 0) || resets<Op>(total);
        const typename Op::carry_t agg = Op::to_carry(total);
        publish_acked<Op>(p.lb, p.lb.status, tile, agg, known ? kStatePrefix : kStateAggregate);
        *s_total = agg;
        *s_known = known;
        __hip_atomic_store(&h->total_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// ------------------------------------------------------------------ scan
template <class Op, bool EXCL, int BLOCK, int ITEMS, bool SINGLE>
__global__ __launch_bounds__(BLOCK) void tile_scan_kernel(ScanParams p)
{
    using G = Geometry<Op, BLOCK, ITEMS>;
    using V = typename Op::value_t;
    using C = typename Op::carry_t;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    static_assert(!IsSeg<Op>::value || VEC == 4, "segmented scans use 4-byte elements");

    __shared__ V s_wave[ND];
    __shared__ C s_excl;
    __shared__ C s_total;
    __shared__ bool s_known;
    __shared__ TileHandover s_h;
    __shared__ uint32_t s_tile;

    const int lane = lane_id();
    // one tile per workgroup: the wavefront index through readfirstlane (the
    // compiler then keeps what derives from it in scalar registers; back to
    // back at 2^20, A/B on one machine: segmented add 8.6 -> 8.3 us, affine 10.3
    // -> 9.9, int32 add within 0.2 either way; compaction's one-tile kernel
    // gained nothing); the single workgroup keeps the plain index
    const int w = SINGLE ? (int)(threadIdx.x >> 6) : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const V ident = Op::identity();

    if constexpr (SINGLE) {
        // Small-n path: one workgroup walks the tiles in order and carries the
        // prefix in registers; the last wavefront idles.
        C running = Op::carry_identity();
        for (uint32_t tile = 0; tile < p.num_tiles; ++tile) {
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
            V wave_prefix = ident, tile_total = ident;
#pragma unroll
            for (int k = 0; k < ND; ++k) {
                const V a = s_wave[k];
                if (k < w) wave_prefix = Op::combine(wave_prefix, a);
                tile_total = Op::combine(tile_total, a);
            }
            if (w < ND)
                apply_store<Op, EXCL, R, VEC>(p, wave_base, vec, lane, running, wave_prefix, x, lane_excl,
                                              round_carry, raw_head);
            running = Op::combine_carry(running, Op::to_carry(tile_total));
            __syncthreads();  // s_wave is rewritten by the next tile
        }
        return;
    }

    // ---- (1) tile number; reset the hand-over state
    if (threadIdx.x == 0) {
        s_h.arrived = 0u;
        s_h.total_ready = 0u;
    }
    const uint32_t tile = take_tile(p, &s_tile);
    if (tile >= p.num_tiles) return;  // never index past the grid
    const uint64_t tile_base = (uint64_t)tile * G::TILE;
    const uint64_t wave_base = tile_base + (uint64_t)w * G::WAVE_ELEMS;
    const bool vec = p.vec_ok && tile_base + G::TILE <= p.n;

    V x[R][VEC], lane_excl[R], round_carry[R + 1];
    uint32_t raw_head[R];
    if (w < ND) {
        // ---- (2)-(5) data wavefronts: load, scan, hand the total over
        load_wave<Op, R, VEC>(p, wave_base, vec, lane, x, raw_head);
        scan_wave<Op, R, VEC>(x, lane_excl, round_carry);
        hand_over<Op, ND>(p, tile, w, lane, round_carry[R], s_wave, &s_h, &s_total, &s_known);
    } else {
        // ---- (6) look-back wavefront, concurrent with the loads
        const C excl = lookback_wave<Op>(p.lb, tile, &s_h, &s_total, &s_known);
        if (lane == 0) s_excl = excl;
    }
    __syncthreads();
    if (w < ND) {
        V wave_prefix = ident;
#pragma unroll
        for (int k = 0; k < ND; ++k)
            if (k < w) wave_prefix = Op::combine(wave_prefix, s_wave[k]);
        apply_store<Op, EXCL, R, VEC>(p, wave_base, vec, lane, s_excl, wave_prefix, x, lane_excl, round_carry,
                                      raw_head);
    }
}

// ------------------------------------------------------------ compaction
template <typename T>
__device__ __forceinline__ bool keep(T x) { return x > T(0); }

// Predicate flags of one wavefront's elements: loads (as load_wave) and
// returns in kept[r] bit j whether element j of round r is kept.
template <typename T, int R, int VEC>
__device__ __forceinline__ void load_flags(const ScanParams& p, uint64_t wave_base, bool vec, int lane,
                                           T (&x)[R][VEC], uint32_t (&kept)[R])
{
    const T* __restrict__ in = static_cast<const T*>(p.in);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint64_t i0 = wave_base + (uint64_t)(r * 64 + lane) * VEC;
        uint32_t b = 0;
        if (vec) {
            load_vec<T, VEC>(in + i0, x[r]);
#pragma unroll
            for (int j = 0; j < VEC; ++j) b |= keep(x[r][j]) ? (1u << j) : 0u;
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                x[r][j] = (i0 + j < p.n) ? in[i0 + j] : T(0);
                b |= (i0 + j < p.n && keep(x[r][j])) ? (1u << j) : 0u;
            }
        }
        kept[r] = b;
    }
}

// Packs a wavefront's kept elements, in order, at the start of its own LDS
// region; returns the wavefront's count.
template <typename T, int R, int VEC>
__device__ __forceinline__ uint32_t pack_wave(const T (&x)[R][VEC], const uint32_t (&kept)[R], T* region)
{
    const auto add = [](uint32_t a, uint32_t b) { return a + b; };
    uint32_t base = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t incl = wave_inclusive_scan((uint32_t)__builtin_popcount(kept[r]), 0u, add);
        uint32_t rank = base + wave_shift_up(incl, 0u);
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            if ((kept[r] >> j) & 1u) region[rank++] = x[r][j];
        base += read_lane(incl, 63);
    }
    return base;
}

template <typename T, int BLOCK, int ITEMS, bool SINGLE>
__global__ __launch_bounds__(BLOCK) void compact_kernel(ScanParams p)
{
    using Cnt = OpAdd<uint32_t>;
    using G = Geometry<Cnt, BLOCK, ITEMS>;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    static_assert(sizeof(T) == 4, "4-byte elements");

    __shared__ T s_keep[G::TILE];  // wavefront w packs into [w * WAVE_ELEMS, ...)
    __shared__ uint32_t s_wave[ND];
    __shared__ uint32_t s_excl;
    __shared__ uint32_t s_total;
    __shared__ bool s_known;
    __shared__ TileHandover s_h;
    __shared__ uint32_t s_tile;

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    T* __restrict__ out = static_cast<T*>(p.out);
    T* region = s_keep + w * G::WAVE_ELEMS;

    if constexpr (SINGLE) {
        uint32_t running = 0;
        for (uint32_t tile = 0; tile < p.num_tiles; ++tile) {
            const uint64_t tile_base = (uint64_t)tile * G::TILE;
            const uint64_t wave_base = tile_base + (uint64_t)w * G::WAVE_ELEMS;
            const bool vec = p.vec_ok && tile_base + G::TILE <= p.n;
            uint32_t cnt = 0;
            if (w < ND) {
                T x[R][VEC];
                uint32_t kept[R];
                load_flags<T, R, VEC>(p, wave_base, vec, lane, x, kept);
                cnt = pack_wave<T, R, VEC>(x, kept, region);
                if (lane == 0) s_wave[w] = cnt;
            }
            __syncthreads();
            uint32_t wave_prefix = 0, total = 0;
#pragma unroll
            for (int k = 0; k < ND; ++k) {
                if (k < w) wave_prefix += s_wave[k];
                total += s_wave[k];
            }
            if (w < ND)
                for (uint32_t i = lane; i < cnt; i += 64) out[(uint64_t)running + wave_prefix + i] = region[i];
            running += total;
            __syncthreads();
        }
        if (threadIdx.x == 0) *p.count = running;
        return;
    }

    if (threadIdx.x == 0) {
        s_h.arrived = 0u;
        s_h.total_ready = 0u;
    }
    const uint32_t tile = take_tile(p, &s_tile);
    if (tile >= p.num_tiles) return;
    const uint64_t tile_base = (uint64_t)tile * G::TILE;
    const uint64_t wave_base = tile_base + (uint64_t)w * G::WAVE_ELEMS;
    const bool vec = p.vec_ok && tile_base + G::TILE <= p.n;

    uint32_t cnt = 0;
    if (w < ND) {
        T x[R][VEC];
        uint32_t kept[R];
        load_flags<T, R, VEC>(p, wave_base, vec, lane, x, kept);
        cnt = pack_wave<T, R, VEC>(x, kept, region);
        hand_over<Cnt, ND>(p, tile, w, lane, cnt, s_wave, &s_h, &s_total, &s_known);
    } else {
        const uint32_t excl = lookback_wave<Cnt>(p.lb, tile, &s_h, &s_total, &s_known);
        if (lane == 0) s_excl = excl;
    }
    __syncthreads();
    if (w < ND) {
        uint32_t wave_prefix = 0;
#pragma unroll
        for (int k = 0; k < ND; ++k)
            if (k < w) wave_prefix += s_wave[k];
        // one contiguous run per wavefront at out[prefix of the tile + earlier wavefronts]
        const uint64_t dst = (uint64_t)s_excl + wave_prefix;
        for (uint32_t i = lane; i < cnt; i += 64) out[dst + i] = region[i];
    }
    if (tile == p.num_tiles - 1 && threadIdx.x == 0) *p.count = s_excl + s_total;
}

// ============================================================ persistent
// Persistent, software-pipelined variant of the multi-tile path: a normal
// launch of as many workgroups as fit on the GPU, each looping over tiles.
//
//  * Roles.  The first workgroup to start becomes the resolver: one
//    wavefront that streams through the tile totals in tile order, scans
//    them 64 * RSPAN at a time and publishes each tile's exclusive prefix
//    (lookback.hpp, resolve_stream).  It loads no data, so its status reads
//    do not queue behind tile loads, and each total is read about once.  (A
//    look-back by every tile would have hundreds of tiles in flight reading
//    the same status words; measured, those reads queued behind the tile
//    data on every CU.)
//  * Tiles.  The other workgroups take tile numbers from a counter, in the
//    order they ask (the scans first take a batch; see take_first_batch).
//    A tile therefore only ever waits on tiles already taken by running
//    workgroups, and the resolver has started before any tile is taken, so
//    no co-residency guarantee is needed (a cooperative launch was measured
//    to cost ~17 us per call).  The last workgroup to retire resets the
//    counters for the next launch on the stream.
//  * Pipeline.  Every data wavefront keeps WAIT + 1 of its tiles in flight
//    as raw elements in registers: while it waits for the prefix of its
//    oldest tile, the totals of the next WAIT - 1 are already published and
//    the loads of the newest are on their way.  WAIT is set per class of
//    scan with the tile shape (scan_api.hip): 3 for the plain 4-byte scans
//    (measured: 430 us against 466 us at WAIT = 2 for the float32 add at
//    2^28), 4 for compaction, 2 for segmented scans, 1 for 3x3 matrices --
//    the deepest pipeline the registers hold, then the fastest measured
//    (3x3 matrices hold their waiting tile in LDS instead; see
//    persistent_reload_loop).  The in-register scan is cheap, so a tile is
//    reduced once for its total and scanned again when its prefix arrives.
//    The last wavefront of a data workgroup only fetches the prefixes the
//    resolver publishes, one word per tile.  Wavefront 0 asks for the next
//    tile number one iteration before it is needed.
//  * Rings.  Data and prefix wavefronts meet through rings of LDS slots (the
//    k-th tile of the workgroup uses slot k mod 16) with sequence numbers
//    instead of barriers.  In the loop the total of the k-th tile is handed
//    over WAIT - 1 iterations before its prefix is awaited, but the first
//    batch hands over the totals of tiles 0 .. WAIT before iteration 0.  A
//    wavefront that hands over tile k + S has passed the prefix wait of tile
//    k + S - WAIT, which needed every wavefront's hand-over of that tile: for
//    a tile of the first batch that says nothing about where a slow
//    wavefront is, and k + S - WAIT > WAIT holds for every k only when
//    S >= 2 * WAIT + 1; then every wavefront has finished tile k.  So slots
//    are never rewritten early; the tile-number ring (S >= WAIT + 1) is safe
//    by the same argument.  A host model of the protocol (CPU tests) finds
//    stale wave totals and lost tile totals with S = 2 * WAIT (e.g. WAIT 8
//    with these 16 slots) and none from S = 2 * WAIT + 1.
//  * Progress.  Every wait is on lower tiles or on the resolver, which only
//    waits for totals; a total is published before its workgroup waits for
//    any later prefix; every wait, on status words and on the LDS rings, is
//    bounded by the spin limit, and a wait that gives up makes the others of
//    the launch give up too (lookback.hpp, give_up).
constexpr int kPipeSlots = 16;  // >= 2 * WAIT + 1 (see the ring note above)
// Tiles per lane of the resolver's window (64 * span tiles per poll round),
// as measured at full size: windows of 64 tiles against 128 and 256 —
// float32 add 349.5 / 352 / 354.5 us, int32 exclusive add 346.8 / 349.5 /
// 349, affine 190.2 / 191.6 / 197, compaction 332.5 / 334 / 334; segmented
// scans 246.7 / 227.3 / 227; (maximum, count) 423 (64 and 128) / 421 (256)
// and 2x2 matrices 254 (128) / 252 (256).  Re-measured with the one-pass
// scans after the wait (A/B of library builds on one machine, us; 64 / 128 / 256 /
// 512 tiles): (maximum, count) 2^27 355.8 / 348.4 / 354.0 / -, 2x2 matrices
// 2^25 208.7 / 211.4 / 208.7 / 226.2; affine 2^26 177.2 / 180.0 / 191.4;
// segmented add 2^27 241.2 / 202.3 / 210.5; 3x3 matrices 2^24 464.3 / 448.2
// / 498.4.
template <class Op> struct ResolveSpan { static constexpr int value = 1; };
template <class B> struct ResolveSpan<OpSeg<B>> { static constexpr int value = 2; };
template <> struct ResolveSpan<OpMaxCount> { static constexpr int value = 2; };
template <> struct ResolveSpan<OpMat2> { static constexpr int value = 4; };
#ifndef DWPT_RELOAD36
#define DWPT_RELOAD36 1
#endif
#ifndef DWPT_RESOLVE_SPAN36
#define DWPT_RESOLVE_SPAN36 2
#endif
template <> struct ResolveSpan<OpMat3> { static constexpr int value = DWPT_RESOLVE_SPAN36; };


template <class V, class C, int ND>
struct PipeSlot {
    uint32_t arrived;     // data-wavefront arrivals, counted over all uses of the slot
    uint32_t prefix_seq;  // k + 1 once the exclusive prefix of iteration k is here
    C prefix;
    V wave_total[ND];
};

template <class Op>
__device__ __forceinline__ typename Op::elem_t elem_identity()
{
    if constexpr (IsSeg<Op>::value) return Op::identity().v;
    else return Op::identity();
}

// Issues one wavefront's loads of a tile into raw registers (the data is not
// used here, so nothing waits for it).  Out-of-range elements read as the
// identity; h4[r] holds the head-flag bytes of round r.
// Elements wider than 16 bytes (K > 1 chunks per round) are only scanned in
// the blocked layout, and load their chunks round by round instead: chunk c
// of the lane is chunk c * 64 + lane of the wavefront's share (one 16-byte
// access per lane and round, like every other type), and the share's tail
// past n reads as identity words.
template <class Op, int R, int VEC, bool LANE_VEC = true>
__device__ __forceinline__ void issue_loads(const ScanParams& p, uint64_t wave_base, bool vec, int lane,
                                            typename Op::elem_t (&e)[R][VEC], uint32_t (&h4)[R])
{
    using E = typename Op::elem_t;
    constexpr bool SEG = IsSeg<Op>::value;
    const E* __restrict__ in = static_cast<const E*>(p.in);
    constexpr int K = VecShape<E>::K;
    if constexpr (K > 1) {
        static_assert(!SEG, "wide elements are not segmented");
        constexpr int C = R * K, W = (int)sizeof(E) / 4;
        u32x4 v[C];
        const uint32_t* __restrict__ src = static_cast<const uint32_t*>(p.in) + wave_base * W;
        if (vec) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
#if DWPT_NT_LOADS
                v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + c * 64 + lane);
#else
                v[c] = reinterpret_cast<const u32x4*>(src)[c * 64 + lane];
#endif
            }
        } else {
            uint32_t id[W];
            to_words(elem_identity<Op>(), id);
            const uint64_t words_in = wave_base < p.n ? (p.n - wave_base) * W : 0;  // words of the share below n
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t wq = (uint32_t)((c * 64 + lane) * 4 + q);
                    uint32_t x = id[0];
#pragma unroll
                    for (int t = 1; t < W; ++t)
                        if (wq % W == (uint32_t)t) x = id[t];
                    v[c][q] = wq < words_in ? src[wq] : x;
                }
        }
        __builtin_memcpy(e, v, 16 * C);
#pragma unroll
        for (int r = 0; r < R; ++r) h4[r] = 0;
        return;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint64_t i0 = wave_base + (uint64_t)(r * 64 + lane) * VEC;
        h4[r] = 0;
        if (vec) {
            load_vec<E, VEC>(in + i0, e[r]);
            if constexpr (SEG) h4[r] = *reinterpret_cast<const uint32_t*>(p.heads + i0);
        } else if (LANE_VEC && p.vec_ok && i0 + VEC <= p.n) {  // partial tile, this lane's elements all below n
            load_vec<E, VEC>(in + i0, e[r]);
            if constexpr (SEG) h4[r] = *reinterpret_cast<const uint32_t*>(p.heads + i0);
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const uint64_t i = i0 + j;
                e[r][j] = (i < p.n) ? in[i] : elem_identity<Op>();
                if constexpr (SEG)
                    if (i < p.n && p.heads[i]) h4[r] |= 0xFFu << (8 * j);
            }
        }
    }
}

// Raw elements -> scan values and head bits (element 0 of the input is a head).
template <class Op, int R, int VEC>
__device__ __forceinline__ void to_values(uint64_t wave_base, int lane, const typename Op::elem_t (&e)[R][VEC],
                                          const uint32_t (&h4)[R], typename Op::value_t (&x)[R][VEC],
                                          uint32_t (&raw_head)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        uint32_t hb = 0;
        if constexpr (IsSeg<Op>::value) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) hb |= ((h4[r] >> (8 * j)) & 0xFFu) ? (1u << j) : 0u;
            if (wave_base + (uint64_t)(r * 64 + lane) * VEC == 0) hb |= 1u;
        }
        raw_head[r] = hb;
#pragma unroll
        for (int j = 0; j < VEC; ++j) x[r][j] = make_value<Op>(e[r][j], (hb >> j) & 1u);
    }
}

// Fold of one wavefront's share of a tile, in element order.
template <class Op, int R, int VEC>
__device__ __forceinline__ typename Op::value_t reduce_wave(uint64_t wave_base, int lane,
                                                            const typename Op::elem_t (&e)[R][VEC],
                                                            const uint32_t (&h4)[R])
{
    using V = typename Op::value_t;
    const V ident = Op::identity();
    V x[R][VEC];
    uint32_t raw_head[R];
    to_values<Op, R, VEC>(wave_base, lane, e, h4, x, raw_head);
#ifndef DWPT_COMMUTATIVE_REDUCE
#define DWPT_COMMUTATIVE_REDUCE 1
#endif
    if constexpr (DWPT_COMMUTATIVE_REDUCE && IsCommutative<Op>::value) {
        // order-free: each lane folds all its elements, then one wavefront pass
        V t = x[0][0];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = (r == 0 ? 1 : 0); j < VEC; ++j) t = Op::combine(t, x[r][j]);
        return read_lane(op_wave_scan<Op>(t), 63);
    }
    V total = ident;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        V t = x[r][0];
#pragma unroll
        for (int j = 1; j < VEC; ++j) t = Op::combine(t, x[r][j]);
        total = Op::combine(total, read_lane(op_wave_scan<Op>(t), 63));
    }
    return total;
}

// Data wavefront w hands its total over; the last one of the workgroup to
// arrive for this tile publishes the tile total.
template <class Op, class Slot, int ND>
__device__ __forceinline__ void hand_over_slot(const ScanParams& p, uint32_t tile, uint32_t k, int w, int lane,
                                               typename Op::value_t wave_total, Slot* slot)
{
    using V = typename Op::value_t;
    if (lane == 0) slot->wave_total[w] = wave_total;
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(&slot->arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (k / kPipeSlots) * ND + (ND - 1)) return;  // not the last data wavefront of this use
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    V total = Op::identity();
    // (Folding the exclusive wavefront prefixes here, once, into the slot for the
    // data wavefronts to read made the float32 add at 2^28 11 us slower and the
    // 3x3 matrices 1-2% faster: not kept.)
#pragma unroll
    for (int q = 0; q < ND; ++q) total = Op::combine(total, slot->wave_total[q]);
    if (lane == 0) publish<Op>(p.lb, p.lb.status, (uint64_t)tile * DWPT_AGG_PAD, Op::to_carry(total), kStateAggregate);
}

// LDS waits of the persistent kernels.  Every one of them ends:
//  * the prefix wavefront's waits (for a tile number) count their polls
//    against the spin limit scaled to LDS polling (lookback.hpp,
//    lds_poll_limit), and its status-word waits are bounded; if it gives up
//    a wait for a tile number it releases every slot of the prefix ring
//    (release_slots) before it stops, so no data wavefront waits on it again;
//  * a data wavefront waits only for prefixes (posted by the prefix
//    wavefront, or released) and for tile numbers (posted by wavefront 0,
//    which itself only waits for prefixes).
// So the data wavefronts' waits end without a count of their own.  They may
// still count (COUNTED) and give up past the limit; whether that is faster
// was measured per kernel class (counted_lds_waits): the 4-byte scans gain
// 1-2 us at 2^28 with the counted loop and 2x2 matrices ~3 us at 2^26, while
// (maximum, count) at 2^27 loses 130 us (567 against 437), segmented add 5,
// compaction at 2^28 50 (381 against 322 us), so those are not counted.
// Counted or not, a loop touches nothing but LDS: a data wavefront's global
// load would complete only after its own tile loads in flight (one counter
// covers a wavefront's loads).  A wave that gave up goes on with what the
// slot holds, so every wave exits, and records the timeout in the error word
// and the abort word once its loop is over (record_lds_timeout).
struct LdsWait {
    uint32_t limit;     // polls before giving up
    uint32_t* abort;    // the workgroup's flag: some wait of the workgroup gave up
    bool gave_up;       // this wavefront gave up a wait (uniform)
    __device__ __forceinline__ LdsWait(const Lookback& lb, uint32_t* flag)
        : limit(lds_poll_limit(lb) > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)lds_poll_limit(lb)), abort(flag),
          gave_up(false)
    {
    }
    // after kAbortCheck more failed polls: true once the wait must give up
    __device__ __forceinline__ bool fail_batch(uint32_t& polls)
    {
        polls += kAbortCheck;
        if (polls > limit || __hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u) {
            if (lane_id() == 0) __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            gave_up = true;
            return true;
        }
        return false;
    }
};

// After a wavefront's loop: a wait that gave up is recorded for the host and
// the rest of the launch.
__device__ __forceinline__ void record_lds_timeout(const Lookback& lb, const LdsWait& lw)
{
    if (lw.gave_up && lane_id() == 0) {
        __hip_atomic_fetch_or(lb.err, (uint32_t)kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(lb.abort, lb.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Waits until *seq >= want.  Counted: polls in batches of kAbortCheck with
// nothing but the poll in the inner loop, the budget and the flag checked
// between batches.
template <bool COUNTED>
__device__ __forceinline__ void wait_seq(LdsWait& lw, uint32_t* seq, uint32_t want)
{
    if constexpr (!COUNTED) {
        (void)lw;
        while (__hip_atomic_load(seq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < want) __builtin_amdgcn_s_sleep(1);
    } else {
        uint32_t polls = 0;
        while (true) {
            for (uint32_t i = 0; i < kAbortCheck; ++i) {
                if (__hip_atomic_load(seq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= want) return;
                __builtin_amdgcn_s_sleep(1);
            }
            if (lw.fail_batch(polls)) return;
        }
    }
}



// The persistent kernel's counters, each on its own 128-byte line so that
// their atomics do not queue behind one another.
enum : int { kCtrTiles = 0, kCtrRoles = 1, kCtrRetired = 2, kCtrCount = 3 };
constexpr int kCtrStride = 32;  // words
__device__ __forceinline__ uint32_t* pipe_counter(const ScanParams& p, int q) { return p.pipe_ctr + q * kCtrStride; }

// Tile numbers of a data workgroup, in the order it processes them.
struct TileIdRing {
    uint32_t id[kPipeSlots];
    uint32_t seq[kPipeSlots];  // k + 1 once id[k mod kPipeSlots] holds the k-th tile number
    uint32_t abort;            // set once a wait of this workgroup gave up
};

__device__ __forceinline__ void put_id(TileIdRing* r, uint32_t k, uint32_t id)
{
    r->id[k % kPipeSlots] = id;
    __hip_atomic_store(&r->seq[k % kPipeSlots], k + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The k-th tile number of the workgroup (counted: UINT32_MAX, past every
// tile, so that the caller's loop ends, if the wait gives up).
template <bool COUNTED>
__device__ __forceinline__ uint32_t get_id(LdsWait& lw, TileIdRing* r, uint32_t k)
{
    uint32_t* seq = &r->seq[k % kPipeSlots];
    if constexpr (!COUNTED) {
        (void)lw;
        while (__hip_atomic_load(seq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < k + 1) __builtin_amdgcn_s_sleep(1);
    } else {
        uint32_t polls = 0;
        while (true) {
            bool here = false;
            for (uint32_t i = 0; i < kAbortCheck; ++i) {
                if (__hip_atomic_load(seq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= k + 1) {
                    here = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (here) break;
            if (lw.fail_batch(polls)) return UINT32_MAX;
        }
    }
    return r->id[k % kPipeSlots];
}

// Workgroup start: take a role (0 = resolver) and clear the LDS rings.
template <class Slot>
__device__ __forceinline__ uint32_t start_workgroup(const ScanParams& p, Slot* slots, TileIdRing* ids,
                                                    uint32_t* s_role)
{
    if (threadIdx.x == 0)
        *s_role = __hip_atomic_fetch_add(pipe_counter(p, kCtrRoles), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < kPipeSlots) {
        slots[threadIdx.x].arrived = 0u;
        slots[threadIdx.x].prefix_seq = 0u;
        ids->seq[threadIdx.x] = 0u;
    }
    if (threadIdx.x == 0) ids->abort = 0u;
    __syncthreads();
    return *s_role;
}

// Called by one lane once its workgroup is done with the counters; the last
// workgroup of the launch resets them for the next one.
__device__ __forceinline__ void retire_workgroup(const ScanParams& p)
{
    const uint32_t d = __hip_atomic_fetch_add(pipe_counter(p, kCtrRetired), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == gridDim.x - 1) {
#pragma unroll
        for (int q = 0; q < kCtrCount; ++q) __hip_atomic_store(pipe_counter(p, q), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}


// The scan kernels' start: the first NT numbers as one consecutive batch,
// with a single atomic (every lower number is then held by a running
// workgroup, as with single numbers).  The workgroup publishes the totals of
// the whole batch before it waits for any prefix, so the batch does not chain
// the workgroups one after another.  Taken one round trip apart instead, the
// 255 workgroups' first numbers queue on the counter and the first loads go
// out ~22 us after the launch (measured; the scans gain ~3%, compaction, which
// keeps single numbers, does not).  Returns true once a number past the last
// tile came back.
template <int NT>
__device__ __forceinline__ bool take_first_batch(const ScanParams& p, TileIdRing* ids)
{
    uint32_t b = p.num_tiles;
    if (lane_id() == 0)
        b = __hip_atomic_fetch_add(pipe_counter(p, kCtrTiles), (uint32_t)NT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    b = (uint32_t)__builtin_amdgcn_readfirstlane((int)b);
    if (lane_id() == 0)
#pragma unroll
        for (int q = 0; q < NT; ++q) put_id(ids, (uint32_t)q, (uint64_t)b + q < p.num_tiles ? b + q : p.num_tiles);
    return (uint64_t)b + NT >= p.num_tiles;
}

// The first NT numbers in consecutive pieces: NA numbers, then pieces of NB,
// each taken once the one before has come back (by then the other
// workgroups' pieces of the same rank are mostly out), every tile's loads
// going out as soon as its number is known.  With one batch, the prefix chain
// cannot pass a workgroup before all NT of its tiles are in, i.e. before
// nearly the whole first batch of the chip (61 MB for the plain scans) is
// read, and no tile is stored meanwhile; with a first piece of one tile it
// passes every workgroup's first tile once those are in.  Every lower number
// is still held by a running workgroup.  Measured (timing harness, µs):
// float32 / int32 add at 2^28, pieces (1, 3) 332.1 / 331.5 against one batch
// 335.5 / 334.5, (2, 2) 332.8 / 332.4, (1, 2, 1) 334.0 / 333.2, (2, 1, 1)
// 334.8 / 334.4, (1, 1, 1, 1) 336.0 / 335.2.  In the library, on one machine:
// float32 add 2^28 335.3 -> 331.5, affine 2^26 184.1 -> 178.5, 2x2 matrices
// 2^25 219.7 -> 216.9 (which operators take pieces: FirstPieces).
template <int NT, int NA, int NB>
__device__ __forceinline__ bool take_first_pieces(const ScanParams& p, TileIdRing* ids)
{
    static_assert(NA >= 1 && NB >= 1, "pieces of at least one number");
    bool ex = false;
#pragma unroll
    for (int q = 0; q < NT;) {
        const int m = (q == 0 ? NA : NB) < NT - q ? (q == 0 ? NA : NB) : NT - q;
        uint32_t b = p.num_tiles;
        if (!ex) {
            if (lane_id() == 0)
                b = __hip_atomic_fetch_add(pipe_counter(p, kCtrTiles), (uint32_t)m, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            b = (uint32_t)__builtin_amdgcn_readfirstlane((int)b);
        }
        if (lane_id() == 0)
#pragma unroll
            for (int j = 0; j < m; ++j)
                put_id(ids, (uint32_t)(q + j), !ex && (uint64_t)b + j < p.num_tiles ? b + j : p.num_tiles);
        ex = ex || (uint64_t)b + m >= p.num_tiles;
        q += m;
    }
    return ex;
}

// Wavefront 0 asks for a tile number one iteration before it is needed: the
// request goes out at the top of the iteration (lane 0) and its result is
// used only at the end, so the counter's round trip overlaps the iteration.
__device__ __forceinline__ uint32_t ask_id(const ScanParams& p, bool exhausted)
{
    uint32_t id = p.num_tiles;
    if (!exhausted && lane_id() == 0)
        id = __hip_atomic_fetch_add(pipe_counter(p, kCtrTiles), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return id;  // valid in lane 0
}

__device__ __forceinline__ void post_id(const ScanParams& p, TileIdRing* ids, uint32_t k, uint32_t id, bool& exhausted)
{
    if (lane_id() == 0) put_id(ids, k, id);
    exhausted = exhausted || (uint32_t)__builtin_amdgcn_readfirstlane((int)id) >= p.num_tiles;
}

// Prefix wavefront of a data workgroup: fetches the prefix of each of the
// workgroup's tiles, in order, into the slot ring.  If it gives up waiting
// for a tile number it releases every slot (sequence number UINT32_MAX), so
// that no data wavefront waits for a prefix that will not come.
template <class Op, class Slot>
__device__ __forceinline__ void fetch_prefixes(const ScanParams& p, TileIdRing* ids, Slot* slots)
{
    uint64_t polls = 0;
    LdsWait lw(p.lb, &ids->abort);
    for (uint32_t k = 0;; ++k) {
        const uint32_t tile = get_id<true>(lw, ids, k);
        if (tile >= p.num_tiles) break;
        const typename Op::carry_t excl = wait_excl<Op>(p.lb, p.lb.groups, tile, polls);
        if (polls > p.lb.spin_limit && lane_id() == 0)  // gave up: let the data wavefronts know
            __hip_atomic_store(&ids->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        Slot* slot = &slots[k % kPipeSlots];
        if (lane_id() == 0) {
            slot->prefix = excl;
            __hip_atomic_store(&slot->prefix_seq, k + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    if (lw.gave_up && lane_id() < kPipeSlots)
        __hip_atomic_store(&slots[lane_id()].prefix_seq, UINT32_MAX, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    record_lds_timeout(p.lb, lw);
}

// Position of a data wavefront's share of a tile.
template <class G>
struct WaveTile {
    uint32_t tile;
    uint64_t base;  // first element of the wavefront's share
    bool vec;       // whole tile in range and aligned: 16-byte accesses
    __device__ __forceinline__ void set(const ScanParams& p, uint32_t t, int w)
    {
        tile = t;
        base = (uint64_t)t * G::TILE + (uint64_t)w * G::WAVE_ELEMS;
        vec = p.vec_ok && (uint64_t)t * G::TILE + G::TILE <= p.n;
    }
};

// ------------------------------------------------------------ blocked layout
// Operators with expensive combines (32-bit multiplies, compare-and-select
// pairs) are scanned in a blocked layout: each lane holds R consecutive
// 16-byte chunks of the wavefront's share instead of one chunk per round, so
// a tile takes one wavefront scan for its total and one for the exclusive
// lane prefixes instead of R each, and the serial in-lane scan covers all
// ITEMS elements.  Loads and stores stay one chunk per lane and round (lanes
// reading R consecutive chunks each were measured at 0.7-3.9 TB/s against
// 6.1-6.5 for this order); the chunks change places through LDS, within the
// wavefront (its LDS operations take effect in order, so no barrier).
#ifndef DWPT_BLOCKED
#define DWPT_BLOCKED 1
#endif
template <class Op> struct UseBlocked { static constexpr bool value = false; };
#if DWPT_BLOCKED
template <> struct UseBlocked<OpAffine> { static constexpr bool value = true; };
template <> struct UseBlocked<OpMaxCount> { static constexpr bool value = true; };
template <> struct UseBlocked<OpMat2> { static constexpr bool value = true; };
#ifndef DWPT_BLOCKED_SEG
#define DWPT_BLOCKED_SEG 1
#endif
#if DWPT_BLOCKED_SEG
template <class B> struct UseBlocked<OpSeg<B>> { static constexpr bool value = true; };
#endif
#endif
template <> struct UseBlocked<OpMat3> { static constexpr bool value = true; };  // always (wide elements)

// How the persistent kernel takes its first tile numbers: in pieces of
// `first`, then `next` (take_first_pieces), or, with first == 0, as one
// batch.  Segmented scans keep one batch (pieces of 1 then 2, or 2 then 1:
// 216 against 214 us at 2^27); (maximum, count) at 2^27 with pieces of 1
// then 3 / 1 then 4 / 2 then 3: 362.9 / 363.3 / 363.6 against 364.5-365.3.
template <class Op> struct FirstPieces { static constexpr int first = 1, next = 3; };
template <class B> struct FirstPieces<OpSeg<B>> { static constexpr int first = 0, next = 0; };

// Whether the persistent kernel tells the compiler that the wavefront index
// is the same in every lane (readfirstlane): the tile bookkeeping derived
// from it then lives in scalar registers.  Per operator, because the
// changed schedule helps some and costs others (timing harness, µs, without
// / with): segmented add 2^27 214.0 / 204.4 (spilled bytes per lane 48 / 8),
// 2x2 matrices 2^26 411.2 / 408.6; float32 add 2^28 331.2 / 350.0, int32 add
// 330.6 / 345.4, 3x3 matrices 2^25 966 / 1030, compaction 256.2 / 259.2;
// affine and (maximum, count) equal by themselves (128 -> 119 and 246 -> 229
// VGPRs), and the registers freed hold their kept lane prefixes
// (KeepLanePrefix).
template <class Op> struct UniformWaveIndex { static constexpr bool value = false; };
template <class B> struct UniformWaveIndex<OpSeg<B>> { static constexpr bool value = true; };
template <> struct UniformWaveIndex<OpMat2> { static constexpr bool value = true; };
template <> struct UniformWaveIndex<OpAffine> { static constexpr bool value = true; };
template <> struct UniformWaveIndex<OpMaxCount> { static constexpr bool value = true; };

// LDS chunk slot of chunk c: one chunk of padding after every R, which keeps
// both orders of access free of bank conflicts.
template <int R>
__device__ __forceinline__ int tr_slot(int c)
{
    return c + c / R;
}
template <int R>
constexpr int tr_slots()
{
    return 64 * R + 64;
}

// In place: round-ordered chunks (chunk c of this lane is chunk c * 64 + lane
// of the wavefront) to lane-ordered ones (chunk c is lane * C + c), or back;
// C = R chunks, or R * K for elements wider than 16 bytes.
template <int R, int VEC, typename E>
__device__ __forceinline__ void transpose_chunks(u32x4* tr, int lane, E (&e)[R][VEC], bool to_blocked)
{
    static_assert(sizeof(E) * VEC % 16 == 0, "16-byte chunks");
    constexpr int C = R * (int)(sizeof(E) * VEC / 16);
    u32x4 v[C];
    __builtin_memcpy(v, e, 16 * C);
#pragma unroll
    for (int c = 0; c < C; ++c) tr[tr_slot<C>(to_blocked ? c * 64 + lane : lane * C + c)] = v[c];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = tr[tr_slot<C>(to_blocked ? lane * C + c : c * 64 + lane)];
    __builtin_memcpy(e, v, 16 * C);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
}

// The same for the head-flag bytes of segmented scans (one 32-bit word per
// chunk), in place.
template <int R>
__device__ __forceinline__ void transpose_words(uint32_t* trh, int lane, uint32_t (&h)[R], bool to_blocked)
{
#pragma unroll
    for (int r = 0; r < R; ++r) trh[tr_slot<R>(to_blocked ? r * 64 + lane : lane * R + r)] = h[r];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < R; ++r) h[r] = trh[tr_slot<R>(to_blocked ? lane * R + r : r * 64 + lane)];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
}

// A tile's chunks in blocked order again, from the LDS area that its
// transposition (transpose_chunks, to_blocked) filled; the wavefront's LDS
// operations take effect in order, so no barrier.
template <int R, int VEC, typename E>
__device__ __forceinline__ void reload_blocked(const u32x4* tr, int lane, E (&e)[R][VEC])
{
    constexpr int C = R * (int)(sizeof(E) * VEC / 16);
    u32x4 v[C];
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = tr[tr_slot<C>(lane * C + c)];
    __builtin_memcpy(e, v, 16 * C);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
}

// The opposite: a tile held in blocked order written back to the LDS area in
// the same layout, so that reload_blocked finds it there.
template <int R, int VEC, typename E>
__device__ __forceinline__ void park_blocked(u32x4* tr, int lane, const E (&e)[R][VEC])
{
    constexpr int C = R * (int)(sizeof(E) * VEC / 16);
    u32x4 v[C];
    __builtin_memcpy(v, e, 16 * C);
#pragma unroll
    for (int c = 0; c < C; ++c) tr[tr_slot<C>(lane * C + c)] = v[c];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
}

// Head bits of the lane's chunks in blocked order (bit j of hb[r]: element j
// of chunk lane * R + r starts a segment; element 0 of the input always does).
// (Packing a waiting tile's flag words into one word when the tile arrives
// halved the segmented kernel's spills, 48 -> 24 bytes, but made it slower:
// 214.5 -> 256 us at 2^27.)
template <class Op, int R, int VEC>
__device__ __forceinline__ void heads_blocked(uint64_t wave_base, int lane, const uint32_t (&h4)[R],
                                              uint32_t (&hb)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        uint32_t b = 0;
        if constexpr (IsSeg<Op>::value) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) b |= ((h4[r] >> (8 * j)) & 0xFFu) ? (1u << j) : 0u;
            if (wave_base + (uint64_t)(lane * R + r) * VEC == 0) b |= 1u;
        }
        hb[r] = b;
    }
}

// Wavefront total of a tile held in blocked order (lane-major: the lane's
// elements are consecutive).
template <class Op, int R, int VEC>
__device__ __forceinline__ typename Op::value_t reduce_blocked(uint64_t wave_base, int lane,
                                                               const typename Op::elem_t (&e)[R][VEC],
                                                               const uint32_t (&h4)[R],
                                                               typename Op::value_t& lane_excl)
{
    using V = typename Op::value_t;
    const V ident = Op::identity();
    const auto comb = [](V a, V b) { return Op::combine(a, b); };
    uint32_t hb[R];
    heads_blocked<Op, R, VEC>(wave_base, lane, h4, hb);
    V t = make_value<Op>(e[0][0], hb[0] & 1u);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = (r == 0 ? 1 : 0); j < VEC; ++j) t = Op::combine(t, make_value<Op>(e[r][j], (hb[r] >> j) & 1u));
    const V incl = wave_inclusive_scan(t, ident, comb);
    lane_excl = wave_shift_up(incl, ident);
    return read_lane(incl, 63);
}

// Blocked-layout operators whose tile stores take the buffer-descriptor path
// with the streaming + sc1 policy (as apply_store).  Measured per operator,
// identical outputs: affine 2^26 187.5 -> 183.8 us, 3x3 matrices 2^24
// 528.6 -> 505.1 us; once the tile bookkeeping of the 512-thread kernels sat
// in scalar registers (2x2: UniformWaveIndex), (maximum, count) 2^27
// 362.5 -> 355.4 and 2x2 matrices 2^26 409.0 -> 400.0 (timing harness).
// Segmented scans keep the plain streaming hint: 204.4 -> 212.0 us at 2^27
// with the descriptor (earlier, when the kernels still spilled at the
// 128-VGPR limit, all three were 9-19% slower with it).
template <class Op> struct BlockedStorePolicy { static constexpr bool value = false; };
template <> struct BlockedStorePolicy<OpAffine> { static constexpr bool value = true; };
template <> struct BlockedStorePolicy<OpMat3> { static constexpr bool value = true; };
template <> struct BlockedStorePolicy<OpMaxCount> { static constexpr bool value = true; };
template <> struct BlockedStorePolicy<OpMat2> { static constexpr bool value = true; };

// Elements wider than 16 bytes: a wavefront's share in round order, chunk c
// of this lane being chunk c * 64 + lane of the share (see issue_loads),
// stored like apply_store.
template <class Op, int R, int VEC>
__device__ __forceinline__ void store_round_chunks(const ScanParams& p, uint64_t wave_base, bool vec, int lane,
                                                   const u32x4 (&v)[R * VecShape<typename Op::elem_t>::K])
{
    using E = typename Op::elem_t;
    constexpr int K = VecShape<E>::K;
    constexpr int C = R * K, W = (int)sizeof(E) / 4;
    uint32_t* __restrict__ dst = static_cast<uint32_t*>(p.out) + wave_base * W;
    if (vec && BlockedStorePolicy<Op>::value) {
        const __amdgpu_buffer_rsrc_t rsrc = wave_rsrc(dst);
#pragma unroll
        for (int c = 0; c < C; ++c)
            __builtin_amdgcn_raw_buffer_store_b128(v[c], rsrc, (uint32_t)(c * 64 + lane) * 16u, 0, DWPT_STORE_POLICY);
    } else if (vec) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
#if DWPT_NT_STORES
            __builtin_nontemporal_store(v[c], reinterpret_cast<u32x4*>(dst) + c * 64 + lane);
#else
            reinterpret_cast<u32x4*>(dst)[c * 64 + lane] = v[c];
#endif
        }
    } else {
        const uint64_t words_in = wave_base < p.n ? (p.n - wave_base) * W : 0;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t wq = (uint32_t)((c * 64 + lane) * 4 + q);
                if (wq < words_in) dst[wq] = v[c][q];
            }
    }
}

// A scanned tile in blocked order (y, changed in place) back to round order
// through LDS, stored like apply_store.
template <class Op, int R, int VEC>
__device__ __forceinline__ void store_blocked_tile(const ScanParams& p, uint64_t wave_base, bool vec, int lane,
                                                   u32x4* tr, typename Op::elem_t (&y)[R][VEC])
{
    using E = typename Op::elem_t;
    transpose_chunks<R, VEC, E>(tr, lane, y, false);
    constexpr int K = VecShape<E>::K;
    if constexpr (K > 1) {
        constexpr int C = R * K;
        u32x4 v[C];
        __builtin_memcpy(v, y, 16 * C);
        store_round_chunks<Op, R, VEC>(p, wave_base, vec, lane, v);
        return;
    }
    E* __restrict__ out = static_cast<E*>(p.out);
    if constexpr (BlockedStorePolicy<Op>::value) {
        if (vec) {
            const __amdgpu_buffer_rsrc_t rsrc = wave_rsrc(out + wave_base);
#pragma unroll
            for (int r = 0; r < R; ++r)
                store_vec_buf<E, VEC>(rsrc, (uint32_t)((r * 64 + lane) * VEC * sizeof(E)), y[r]);
            return;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint64_t i0 = wave_base + (uint64_t)(r * 64 + lane) * VEC;
        if (vec) {
            store_vec<E, VEC>(out + i0, y[r]);
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                if (i0 + j < p.n) out[i0 + j] = y[r][j];
        }
    }
}

// Operators whose combine is exactly associative and whose carry is a value
// of the same type (integer arithmetic mod 2^32, comparisons): the lane's
// running value can start from the prefix, so each output is one combine
// instead of a combine and an apply -- the same words, as
// carry (+) (x_0 (+) .. (+) x_i) == (..(carry (+) x_0) (+) ..) (+) x_i holds
// exactly for them (not for float add, whose carry is a double).
template <class Op> struct FoldCarry { static constexpr bool value = false; };
template <> struct FoldCarry<OpAffine> { static constexpr bool value = true; };
template <> struct FoldCarry<OpMaxCount> { static constexpr bool value = true; };
template <> struct FoldCarry<OpMat2> { static constexpr bool value = true; };
template <> struct FoldCarry<OpMat3> { static constexpr bool value = true; };
// Segmented pairs over an exact integer operator: the running pair starts as
// (no head, prefix); a head inside the lane then discards the prefix exactly
// as applying it to the lane's fold would (segmented add at 2^27, A/B on one
// machine, identical outputs: 204.1 -> 201.7 us).
template <class B> struct FoldCarry<OpSeg<B>> {
    static constexpr bool value =
        std::is_same<typename B::prep_t, typename B::value_t>::value && std::is_integral<typename B::value_t>::value;
};

// Blocked-layout operators that keep each waiting tile's lane prefix (from
// the wavefront scan of its total) until the tile's prefix is in, so that the
// scan after the wait is one serial pass with no second wavefront scan:
// segmented pairs, and the FoldCarry operators, whose pass then needs one
// combine per element.  Measured with identical outputs (A/B on one machine, us):
// 2x2 matrices 2^25 211.4 -> 209.1; affine maps 2^26 and (maximum, count)
// 2^27 179.0 -> 177.6 and 356.3 -> 354.5 with their tile bookkeeping in
// scalar registers (UniformWaveIndex), which makes room for the kept
// prefixes (without it they spill: 179.9 and 365.5).
template <class Op> struct KeepLanePrefix { static constexpr bool value = IsSeg<Op>::value; };
template <> struct KeepLanePrefix<OpMat2> { static constexpr bool value = FoldCarry<OpMat2>::value; };
template <> struct KeepLanePrefix<OpAffine> { static constexpr bool value = FoldCarry<OpAffine>::value; };
template <> struct KeepLanePrefix<OpMaxCount> { static constexpr bool value = FoldCarry<OpMaxCount>::value; };

// Scan of a tile held in blocked order, prefix applied, back to round order
// through LDS, stored like apply_store.
template <class Op, bool EXCL, int R, int VEC, bool KEPT = false>
__device__ __forceinline__ void scan_store_blocked(const ScanParams& p, uint64_t wave_base, bool vec, int lane,
                                                   u32x4* tr, typename Op::carry_t P,
                                                   typename Op::value_t wave_prefix,
                                                   const typename Op::elem_t (&e)[R][VEC], const uint32_t (&h4)[R],
                                                   typename Op::value_t lane_excl, bool have_lane_excl)
{
    using E = typename Op::elem_t;
    using V = typename Op::value_t;
    const V ident = Op::identity();
    const auto comb = [](V a, V b) { return Op::combine(a, b); };
    uint32_t hb[R];
    heads_blocked<Op, R, VEC>(wave_base, lane, h4, hb);
    if constexpr (KEPT) {
        // the lane prefix was kept from the wavefront scan of the total: one
        // serial pass applies the prefix as it goes, with no array of in-lane
        // prefixes held (segmented add at 2^27: 226.6 -> 215.0 us); for the
        // FoldCarry operators the pass starts from the prefix, one combine
        // per element and no separate application of the prefix.
        (void)have_lane_excl;
        const typename Op::prep_t pc =
            Op::prepare(Op::combine_carry(P, Op::to_carry(Op::combine(wave_prefix, lane_excl))));
        constexpr bool FOLD = FoldCarry<Op>::value;
        V run = ident;
        if constexpr (FOLD) {
            if constexpr (IsSeg<Op>::value)
                run = V{0u, pc};
            else
                run = pc;
        }
        static_assert(VecShape<E>::K == 1, "wide elements take scan_store_parked");
        E y[R][VEC];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const V v = make_value<Op>(e[r][j], (hb[r] >> j) & 1u);
                if constexpr (FOLD) {
                    if constexpr (EXCL) {
                        V o = run;
                        if constexpr (IsSeg<Op>::value)
                            if ((hb[r] >> j) & 1u) o = ident;
                        y[r][j] = elem_of<Op>(o);
                    }
                    run = Op::combine(run, v);
                    if constexpr (!EXCL) y[r][j] = elem_of<Op>(run);
                    continue;
                }
                if constexpr (EXCL) {
                    V o = Op::apply(pc, run);
                    if constexpr (IsSeg<Op>::value)
                        if ((hb[r] >> j) & 1u) o = ident;
                    y[r][j] = elem_of<Op>(o);
                }
                run = (r == 0 && j == 0) ? v : Op::combine(run, v);
                if constexpr (!EXCL) y[r][j] = elem_of<Op>(Op::apply(pc, run));
            }
        store_blocked_tile<Op, R, VEC>(p, wave_base, vec, lane, tr, y);
        return;
    }
    V x[R][VEC];
    V run = make_value<Op>(e[0][0], hb[0] & 1u);
    x[0][0] = run;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = (r == 0 ? 1 : 0); j < VEC; ++j) {
            run = Op::combine(run, make_value<Op>(e[r][j], (hb[r] >> j) & 1u));
            x[r][j] = run;
        }
    if (!have_lane_excl) lane_excl = wave_shift_up(wave_inclusive_scan(run, ident, comb), ident);
    const typename Op::prep_t pc =
        Op::prepare(Op::combine_carry(P, Op::to_carry(Op::combine(wave_prefix, lane_excl))));
    E y[R][VEC];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            if constexpr (EXCL) {
                const V before = (r == 0 && j == 0) ? ident : (j == 0 ? x[r - 1][VEC - 1] : x[r][j - 1]);
                V v = Op::apply(pc, before);
                if constexpr (IsSeg<Op>::value)
                    if ((hb[r] >> j) & 1u) v = ident;
                y[r][j] = elem_of<Op>(v);
            } else {
                y[r][j] = elem_of<Op>(Op::apply(pc, x[r][j]));
            }
        }
    store_blocked_tile<Op, R, VEC>(p, wave_base, vec, lane, tr, y);
}

// A wavefront's total of the tile in e; in the blocked layout, e is first
// rearranged into it (in place) for the scan that follows later.
// (lane_excl: in the blocked layout, the fold of the lower lanes' elements,
// kept for the scan of the tile.)
template <class Op, int R, int VEC, bool BLK>
__device__ __forceinline__ typename Op::value_t tile_wave_total(uint64_t wave_base, int lane, u32x4* tr,
                                                                uint32_t* trh, typename Op::elem_t (&e)[R][VEC],
                                                                uint32_t (&h4)[R], typename Op::value_t& lane_excl)
{
    if constexpr (BLK) {
        transpose_chunks<R, VEC, typename Op::elem_t>(tr, lane, e, true);
        if constexpr (IsSeg<Op>::value) transpose_words<R>(trh, lane, h4, true);
        return reduce_blocked<Op, R, VEC>(wave_base, lane, e, h4, lane_excl);
    } else {
        (void)tr;
        (void)trh;
        (void)lane_excl;
        return reduce_wave<Op, R, VEC>(wave_base, lane, e, h4);
    }
}

// The scan after the wait of persistent_reload_loop, read from the LDS area
// where the tile is parked (blocked order: this lane's chunk c in slot
// lane * C + c) one round of VEC elements at a time: each round's results
// replace its chunks in place, then the area leaves in round order as in the
// kept-prefix form of scan_store_blocked.  Only one round of elements and of
// results is held in registers, not the whole tile.
template <class Op, bool EXCL, int R, int VEC>
__device__ __forceinline__ void scan_store_parked(const ScanParams& p, uint64_t wave_base, bool vec, int lane,
                                                  u32x4* tr, typename Op::carry_t P, typename Op::value_t wave_prefix,
                                                  typename Op::value_t lane_excl)
{
    using E = typename Op::elem_t;
    using V = typename Op::value_t;
    constexpr int K = VecShape<E>::K, C = R * K;
    static_assert(!IsSeg<Op>::value && K > 1, "wide elements without head flags");
    const typename Op::prep_t pc =
        Op::prepare(Op::combine_carry(P, Op::to_carry(Op::combine(wave_prefix, lane_excl))));
    constexpr bool FOLD = FoldCarry<Op>::value;
    V run = Op::identity();
    if constexpr (FOLD) run = pc;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        u32x4 c4[K];
#pragma unroll
        for (int k = 0; k < K; ++k) c4[k] = tr[tr_slot<C>(lane * C + r * K + k)];
        E er[VEC], yr[VEC];
        __builtin_memcpy(er, c4, 16 * K);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const V v = make_value<Op>(er[j], 0u);
            if constexpr (FOLD) {
                if constexpr (EXCL) yr[j] = elem_of<Op>(run);
                run = Op::combine(run, v);
                if constexpr (!EXCL) yr[j] = elem_of<Op>(run);
            } else {
                if constexpr (EXCL) yr[j] = elem_of<Op>(Op::apply(pc, run));
                run = (r == 0 && j == 0) ? v : Op::combine(run, v);
                if constexpr (!EXCL) yr[j] = elem_of<Op>(Op::apply(pc, run));
            }
        }
        __builtin_memcpy(c4, yr, 16 * K);
#pragma unroll
        for (int k = 0; k < K; ++k) tr[tr_slot<C>(lane * C + r * K + k)] = c4[k];
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
    u32x4 v[C];
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = tr[tr_slot<C>(c * 64 + lane)];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
    store_round_chunks<Op, R, VEC>(p, wave_base, vec, lane, v);
}

// Elements wider than 16 bytes with one tile waiting (3x3 matrices): a
// data wavefront holds only its newest tile in registers.  The waiting
// tile's data stay in the wavefront's LDS transposition area from its
// hand-over until its prefix is in, and are read back from there, one round
// at a time, for the scan (scan_store_parked) -- instead of keeping a second
// tile in registers across the wait,
// which at 72 words per tile spilled.  The first two tiles' totals are both
// published before any wait (the second one's first, so that the LDS area
// then holds the first tile); the second tile is written back to the area in
// its turn.
// Counted data-wavefront waits (see LdsWait): for the unsegmented 4-byte
// scans and 2x2 matrices.
template <class Op>
constexpr bool counted_lds_waits()
{
    return !IsSeg<Op>::value && (sizeof(typename Op::value_t) == 4 || sizeof(typename Op::value_t) == 16);
}

#ifndef DWPT_RELOAD_KEEP
#define DWPT_RELOAD_KEEP 1
#endif
template <class Op> struct ReloadAfterWait { static constexpr bool value = false; };
template <> struct ReloadAfterWait<OpMat3> { static constexpr bool value = DWPT_RELOAD36; };

template <class Op, bool EXCL, class G, class Slot>
__device__ __forceinline__ void persistent_reload_loop(const ScanParams& p, Slot* s_slot, TileIdRing* s_ids, u32x4* tr,
                                                       int w, int lane, bool exhausted)
{
    using E = typename Op::elem_t;
    using V = typename Op::value_t;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    E e0[R][VEC], e1[R][VEC];  // the tile to finish (round order, until it is transposed), the next one
    uint32_t h0[R], h1[R];
    V lx, lx1;  // lane prefixes from the wavefront scans of the tiles' totals (tile in e0; the second tile)
    WaveTile<G> t0, t1;
    LdsWait lw(p.lb, &s_ids->abort);
    t0.set(p, get_id<counted_lds_waits<Op>()>(lw, s_ids, 0), w);
    t1.set(p, get_id<counted_lds_waits<Op>()>(lw, s_ids, 1), w);
    if (t0.tile < p.num_tiles) issue_loads<Op, R, VEC, false>(p, t0.base, t0.vec, lane, e0, h0);
    if (t1.tile < p.num_tiles) issue_loads<Op, R, VEC, false>(p, t1.base, t1.vec, lane, e1, h1);
    if (t1.tile < p.num_tiles)
        hand_over_slot<Op, Slot, ND>(p, t1.tile, 1, w, lane,
                                     tile_wave_total<Op, R, VEC, true>(t1.base, lane, tr, nullptr, e1, h1, lx1),
                                     &s_slot[1]);
    if (t0.tile < p.num_tiles)
        hand_over_slot<Op, Slot, ND>(p, t0.tile, 0, w, lane,
                                     tile_wave_total<Op, R, VEC, true>(t0.base, lane, tr, nullptr, e0, h0, lx),
                                     &s_slot[0]);
    for (uint32_t k = 0; t0.tile < p.num_tiles; ++k) {
        uint32_t next_id = p.num_tiles;
        if (w == 0) next_id = ask_id(p, exhausted);
        if (k >= 1) {
            // e0 holds tile k: raw, and its total is published now; or, for
            // the second tile, in blocked order with its total out
            if (k >= 2)
                hand_over_slot<Op, Slot, ND>(p, t0.tile, k, w, lane,
                                             tile_wave_total<Op, R, VEC, true>(t0.base, lane, tr, nullptr, e0, h0, lx),
                                             &s_slot[k % kPipeSlots]);
            else
                park_blocked<R, VEC, E>(tr, lane, e0);
            if (t1.tile < p.num_tiles) issue_loads<Op, R, VEC, false>(p, t1.base, t1.vec, lane, e1, h1);
        }
        Slot* slot = &s_slot[k % kPipeSlots];
        wait_seq<counted_lds_waits<Op>()>(lw, &slot->prefix_seq, k + 1);
        V wave_prefix = Op::identity();
#pragma unroll
        for (int q = 0; q < ND; ++q)
            if (q < w) wave_prefix = Op::combine(wave_prefix, slot->wave_total[q]);
        if constexpr (DWPT_RELOAD_KEEP) {
            scan_store_parked<Op, EXCL, R, VEC>(p, t0.base, t0.vec, lane, tr, slot->prefix, wave_prefix, lx);
        } else {
            reload_blocked<R, VEC, E>(tr, lane, e0);
            scan_store_blocked<Op, EXCL, R, VEC, DWPT_RELOAD_KEEP>(p, t0.base, t0.vec, lane, tr, slot->prefix,
                                                                   wave_prefix, e0, h0, lx, DWPT_RELOAD_KEEP);
        }
        t0 = t1;
        lx = lx1;  // the second tile's; every later tile's comes from its own hand-over
#pragma unroll
        for (int r = 0; r < R; ++r) {
            h0[r] = h1[r];
#pragma unroll
            for (int j = 0; j < VEC; ++j) e0[r][j] = e1[r][j];
        }
        if (w == 0) post_id(p, s_ids, k + 2, next_id, exhausted);
        t1.set(p, get_id<counted_lds_waits<Op>()>(lw, s_ids, k + 2), w);
    }
    record_lds_timeout(p.lb, lw);
    if (w == 0 && lane == 0) retire_workgroup(p);
}

template <class Op, bool EXCL, int BLOCK, int ITEMS, int WAIT>
__global__ __launch_bounds__(BLOCK) void tile_scan_persistent(ScanParams p)
{
    constexpr int kPipeWait = WAIT, kPipeTiles = WAIT + 1;
    static_assert(kPipeSlots >= 2 * kPipeWait + 1, "slot ring too short for the pipeline depth");
    using G = Geometry<Op, BLOCK, ITEMS>;
    using E = typename Op::elem_t;
    using V = typename Op::value_t;
    using C = typename Op::carry_t;
    using Slot = PipeSlot<V, C, G::ND>;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    static_assert(!IsSeg<Op>::value || VEC == 4, "segmented scans use 4-byte elements");
    constexpr bool BLK = UseBlocked<Op>::value;
    constexpr bool BLKH = BLK && IsSeg<Op>::value;
    static_assert(G::K == 1 || BLK, "elements wider than 16 bytes use the blocked layout");

    __shared__ Slot s_slot[kPipeSlots];
    __shared__ TileIdRing s_ids;
    __shared__ uint32_t s_role;
    __shared__ u32x4 s_tr[BLK ? ND : 1][BLK ? tr_slots<R * G::K>() : 1];
    __shared__ uint32_t s_trh[BLKH ? ND : 1][BLKH ? tr_slots<R>() : 1];
    const int lane = lane_id();
    const int w = UniformWaveIndex<Op>::value ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))
                                               : (int)(threadIdx.x >> 6);
    u32x4* tr = BLK ? s_tr[w < ND ? w : 0] : nullptr;
    uint32_t* trh = BLKH ? s_trh[w < ND ? w : 0] : nullptr;
    if (start_workgroup(p, s_slot, &s_ids, &s_role) == 0) {
        if (w == 0) {
            (void)resolve_stream<Op, ResolveSpan<Op>::value>(p.lb, p.lb.status, p.lb.groups, p.num_tiles);
            if (lane == 0) retire_workgroup(p);
        }
        return;
    }
    bool exhausted = false;
    constexpr bool PIECES = FirstPieces<Op>::first > 0 && !ReloadAfterWait<Op>::value;
    if (w == 0) {
        if constexpr (PIECES)
            exhausted = take_first_pieces<kPipeTiles, FirstPieces<Op>::first, FirstPieces<Op>::next>(p, &s_ids);
        else
            exhausted = take_first_batch<kPipeTiles>(p, &s_ids);
    }
    if (w == ND) {
        fetch_prefixes<Op>(p, &s_ids, s_slot);
        return;
    }
    if constexpr (ReloadAfterWait<Op>::value) {
        static_assert(WAIT == 1 && BLK && !IsSeg<Op>::value, "one waiting tile, blocked layout");
        persistent_reload_loop<Op, EXCL, G, Slot>(p, s_slot, &s_ids, tr, w, lane, exhausted);
        return;
    }

    // WAIT + 1 tiles per data wavefront, oldest first: stage 0 waits for its
    // prefix, stages 1 .. WAIT-1 have their totals out, the newest loads.
    E e[kPipeTiles][R][VEC];
    uint32_t h[kPipeTiles][R];
    // each stage's lane prefix from the wavefront scan of its total, kept
    // across the wait by the operators that KeepLanePrefix names (before the
    // one-pass scan from the prefix, FoldCarry, the extra registers cost more
    // than the second wavefront scan: (maximum, count) at 2^27 435 -> 682 us,
    // 2x2 matrices at 2^26 473 -> 905)
    constexpr bool KEEP = BLK && KeepLanePrefix<Op>::value;
    // 16-byte lane loads in the last, partial tile: for the round-order
    // operators only; in the blocked kernels the extra branch (and the same
    // one in their stores) moved the register allocation: (maximum, count) at
    // 2^27 438 -> 471 us, 2x2 matrices at 2^26 476 -> 503-526
    constexpr bool LANE_VEC = !BLK;
    V lx[kPipeTiles];
    WaveTile<G> t[kPipeTiles];
    LdsWait lw(p.lb, &s_ids.abort);
    // the first batch: every tile loaded and its total published up front
    if constexpr (PIECES) {
        // each tile's loads go out as soon as its number is known
#pragma unroll
        for (int q = 0; q < kPipeTiles; ++q) {
            t[q].set(p, get_id<counted_lds_waits<Op>()>(lw, &s_ids, q), w);
            if (t[q].tile < p.num_tiles) issue_loads<Op, R, VEC, LANE_VEC>(p, t[q].base, t[q].vec, lane, e[q], h[q]);
        }
    } else {
#pragma unroll
        for (int q = 0; q < kPipeTiles; ++q) t[q].set(p, get_id<counted_lds_waits<Op>()>(lw, &s_ids, q), w);
#pragma unroll
        for (int q = 0; q < kPipeTiles; ++q)
            if (t[q].tile < p.num_tiles) issue_loads<Op, R, VEC, LANE_VEC>(p, t[q].base, t[q].vec, lane, e[q], h[q]);
    }
#pragma unroll
    for (int q = 0; q < kPipeTiles; ++q)
        if (t[q].tile < p.num_tiles)
            hand_over_slot<Op, Slot, ND>(p, t[q].tile, q, w, lane,
                                         tile_wave_total<Op, R, VEC, BLK>(t[q].base, lane, tr, trh, e[q], h[q], lx[q]),
                                         &s_slot[q % kPipeSlots]);
    for (uint32_t k = 0; t[0].tile < p.num_tiles; ++k) {
        constexpr int NEW = kPipeTiles - 1, PUB = kPipeWait - 1;
        // the tile number for the next iteration goes out before this
        // iteration's loads, so waiting for it never waits for them
        uint32_t next_id = p.num_tiles;
        if (w == 0) next_id = ask_id(p, exhausted);
        // stages still holding the first batch were loaded and published above
        if (k >= 1 && t[NEW].tile < p.num_tiles) issue_loads<Op, R, VEC, LANE_VEC>(p, t[NEW].base, t[NEW].vec, lane, e[NEW], h[NEW]);
        if (k >= 2 && t[PUB].tile < p.num_tiles)
            hand_over_slot<Op, Slot, ND>(p, t[PUB].tile, k + PUB, w, lane,
                                         tile_wave_total<Op, R, VEC, BLK>(t[PUB].base, lane, tr, trh, e[PUB], h[PUB], lx[PUB]),
                                         &s_slot[(k + PUB) % kPipeSlots]);

        Slot* slot = &s_slot[k % kPipeSlots];
        wait_seq<counted_lds_waits<Op>()>(lw, &slot->prefix_seq, k + 1);
        if constexpr (BLK) {
            V wave_prefix = Op::identity();
#pragma unroll
            for (int q = 0; q < ND; ++q)
                if (q < w) wave_prefix = Op::combine(wave_prefix, slot->wave_total[q]);
            scan_store_blocked<Op, EXCL, R, VEC, KEEP>(p, t[0].base, t[0].vec, lane, tr, slot->prefix, wave_prefix,
                                                       e[0], h[0], lx[0], KEEP);
        } else {
            V x[R][VEC], lane_excl[R], round_carry[R + 1];
            uint32_t raw_head[R];
            to_values<Op, R, VEC>(t[0].base, lane, e[0], h[0], x, raw_head);
            scan_wave<Op, R, VEC>(x, lane_excl, round_carry);
            V wave_prefix = Op::identity();
#pragma unroll
            for (int q = 0; q < ND; ++q)
                if (q < w) wave_prefix = Op::combine(wave_prefix, slot->wave_total[q]);
            apply_store<Op, EXCL, R, VEC>(p, t[0].base, t[0].vec, lane, slot->prefix, wave_prefix, x, lane_excl,
                                          round_carry, raw_head);
        }
        // shift the stages down; the newest gets the next tile
#pragma unroll
        for (int q = 0; q + 1 < kPipeTiles; ++q) {
            t[q] = t[q + 1];
            if constexpr (KEEP) lx[q] = lx[q + 1];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                h[q][r] = h[q + 1][r];
#pragma unroll
                for (int j = 0; j < VEC; ++j) e[q][r][j] = e[q + 1][r][j];
            }
        }
        if (w == 0) post_id(p, &s_ids, k + kPipeTiles, next_id, exhausted);
        t[NEW].set(p, get_id<counted_lds_waits<Op>()>(lw, &s_ids, k + kPipeTiles), w);
    }
    record_lds_timeout(p.lb, lw);
    if (w == 0 && lane == 0) retire_workgroup(p);
}

// Persistent compaction.  A tile's kept elements leave as one contiguous run:
// every data wavefront packs its kept elements into a tile buffer in LDS at
// the wavefront's offset within the tile's run, and once all of them have
// packed, all write the run out together in 16-byte chunks aligned in global
// memory, so that partial lines occur only at the two ends of a tile's run
// (wavefront-by-wavefront runs put 15 seams in every tile, whose lines were
// written twice: 1.042x the algorithmic bytes).  The buffer is placed so that
// its chunks line up with the output's 16-byte chunks.  Two tile buffers
// alternate; LDS counters order their reuse (all waits end: every data
// wavefront of the workgroup processes the same tiles, and only waits for the
// others to reach the same point of the same tile).
//
// Kept counts: per round, at most 64 * VEC elements of a wavefront are kept,
// so three rounds' counts fit 10-bit fields of one word, and one wavefront
// scan of that word gives the lane's exclusive count in each of them and, in
// lane 63, the wavefront's round totals (in place of one scan per round).
constexpr int kCountBits = 10, kCountsPerWord = 3;
template <int R>
__device__ __forceinline__ uint32_t count_field(const uint32_t (&w)[(R + kCountsPerWord - 1) / kCountsPerWord], int r)
{
    return (w[r / kCountsPerWord] >> (kCountBits * (r % kCountsPerWord))) & ((1u << kCountBits) - 1u);
}

__device__ __forceinline__ void wait_at_least(uint32_t* c, uint32_t want)
{
    while (__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < want) __builtin_amdgcn_s_sleep(1);
}

template <typename T, int BLOCK, int ITEMS, int WAIT>
__global__ __launch_bounds__(BLOCK) void compact_persistent(ScanParams p)
{
    constexpr int kPipeWait = WAIT, kPipeTiles = WAIT + 1;
    static_assert(kPipeSlots >= 2 * kPipeWait + 1, "slot ring too short for the pipeline depth");
    using Cnt = OpAdd<uint32_t>;
    using Ld = OpMax<T>;  // element loads of T (identity past n: never kept)
    using G = Geometry<Cnt, BLOCK, ITEMS>;
    using Slot = PipeSlot<uint32_t, uint32_t, G::ND>;
    constexpr int R = G::R, VEC = G::VEC, ND = G::ND;
    static_assert(sizeof(T) == 4 && VEC == 4, "4-byte elements, 16-byte chunks");
    static_assert(64 * VEC < (1 << kCountBits), "packed round counts");
    constexpr int CW = (R + kCountsPerWord - 1) / kCountsPerWord;  // words of packed counts
    constexpr int RUN = G::TILE + 4;  // a tile's run and up to 3 elements of alignment
    static_assert(RUN * sizeof(T) % 16 == 0, "the second tile buffer starts 16-byte aligned");

    __shared__ __align__(16) T s_run[2][RUN];
    __shared__ uint32_t s_packed[2], s_written[2];  // arrivals per buffer, over all its uses
    __shared__ Slot s_slot[kPipeSlots];
    __shared__ TileIdRing s_ids;
    __shared__ uint32_t s_role;
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    if (threadIdx.x < 2) {
        s_packed[threadIdx.x] = 0u;
        s_written[threadIdx.x] = 0u;
    }
    if (start_workgroup(p, s_slot, &s_ids, &s_role) == 0) {
        if (w == 0) {
            const uint32_t total = resolve_stream<Cnt, ResolveSpan<Cnt>::value>(p.lb, p.lb.status, p.lb.groups, p.num_tiles);
            if (lane == 0) {
                *p.count = total;
                retire_workgroup(p);
            }
        }
        return;
    }
    bool exhausted = false;
    // first tile numbers in pieces of 1, WAIT - 1 and 1 (take_first_pieces):
    // the totals of stages 0 .. WAIT - 1 go out before the first wait for a
    // prefix, the newest stage's only after it, so the newest stage must be a
    // piece of its own -- one that shares a piece with an earlier stage puts
    // its consecutive numbers behind that stage's prefix: 2^28 pieces of 1 + 3
    // or 2 + 2 270 us, 1 + 2 + 1 257.0-257.5, 2 + 1 + 1 258.8, single numbers
    // one round trip apart 259.7-260.1.
    static_assert(kPipeWait >= 2, "pieces of 1, WAIT - 1 and 1");
    if (w == 0) exhausted = take_first_pieces<kPipeTiles, 1, kPipeWait - 1>(p, &s_ids);
    if (w == ND) {
        fetch_prefixes<Cnt>(p, &s_ids, s_slot);
        return;
    }
    T* __restrict__ out = static_cast<T*>(p.out);
    // the output's offset from a 16-byte boundary, in elements
    const uint32_t out_mis = (uint32_t)(((uintptr_t)out >> 2) & 3u);

    // elements past n were loaded as the lowest value of T, which is never kept
    const auto kept_bits = [&](const T (&e)[R][VEC], uint32_t (&kept)[R]) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t b = 0;
#pragma unroll
            for (int j = 0; j < VEC; ++j) b |= keep(e[r][j]) ? (1u << j) : 0u;
            kept[r] = b;
        }
    };
    // the wavefront's kept count; xcl: the lane's exclusive packed counts, tot: the round totals
    const auto count_wave = [&](const T (&e)[R][VEC], uint32_t (&xcl)[CW], uint32_t (&tot)[CW]) {
        uint32_t kept[R];
        kept_bits(e, kept);
        uint32_t c[CW];
#pragma unroll
        for (int q = 0; q < CW; ++q) c[q] = 0;
#pragma unroll
        for (int r = 0; r < R; ++r)
            c[r / kCountsPerWord] += (uint32_t)__builtin_popcount(kept[r]) << (kCountBits * (r % kCountsPerWord));
        const auto add = [](uint32_t a, uint32_t b) { return a + b; };
        uint32_t sum = 0;
#pragma unroll
        for (int q = 0; q < CW; ++q) {
            const uint32_t incl = wave_inclusive_scan(c[q], 0u, add);
            xcl[q] = incl - c[q];
            tot[q] = read_lane(incl, 63);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) sum += count_field<R>(tot, r);
        return sum;
    };

    T e[kPipeTiles][R][VEC];
    uint32_t xcl[kPipeTiles][CW], tot[kPipeTiles][CW];
    uint32_t hu[R];
    WaveTile<G> t[kPipeTiles];
    LdsWait lw(p.lb, &s_ids.abort);
#pragma unroll
    for (int q = 0; q < kPipeTiles; ++q) t[q].set(p, get_id<false>(lw, &s_ids, q), w);
#pragma unroll
    for (int q = 0; q < kPipeTiles - 1; ++q)
        if (t[q].tile < p.num_tiles) issue_loads<Ld, R, VEC>(p, t[q].base, t[q].vec, lane, e[q], hu);
#pragma unroll
    for (int q = 0; q < kPipeWait - 1; ++q)
        if (t[q].tile < p.num_tiles)
            hand_over_slot<Cnt, Slot, ND>(p, t[q].tile, q, w, lane, count_wave(e[q], xcl[q], tot[q]),
                                          &s_slot[q % kPipeSlots]);
    for (uint32_t k = 0; t[0].tile < p.num_tiles; ++k) {
        constexpr int NEW = kPipeTiles - 1, PUB = kPipeWait - 1;
        uint32_t next_id = p.num_tiles;
        if (w == 0) next_id = ask_id(p, exhausted);
        if (t[NEW].tile < p.num_tiles) issue_loads<Ld, R, VEC>(p, t[NEW].base, t[NEW].vec, lane, e[NEW], hu);
        if (t[PUB].tile < p.num_tiles)
            hand_over_slot<Cnt, Slot, ND>(p, t[PUB].tile, k + PUB, w, lane, count_wave(e[PUB], xcl[PUB], tot[PUB]),
                                          &s_slot[(k + PUB) % kPipeSlots]);
        Slot* slot = &s_slot[k % kPipeSlots];
        wait_seq<false>(lw, &slot->prefix_seq, k + 1);
        uint32_t wave_prefix = 0, run_len = 0;
#pragma unroll
        for (int q = 0; q < ND; ++q) {
            const uint32_t c = slot->wave_total[q];
            if (q < w) wave_prefix += c;
            run_len += c;
        }
        const uint64_t g0 = slot->prefix;  // output index of the tile's first kept element
        const uint32_t shift = (uint32_t)((g0 + out_mis) & 3u);
        const uint32_t b = k & 1u, use = k >> 1;
        T* buf = s_run[b];
        // the buffer's previous tile is out
        wait_at_least(&s_written[b], (uint32_t)ND * use);
        {
            uint32_t kept[R];
            kept_bits(e[0], kept);
            uint32_t base = shift + wave_prefix;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                uint32_t rank = base + count_field<R>(xcl[0], r);
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    if ((kept[r] >> j) & 1u) buf[rank++] = e[0][r][j];
                base += count_field<R>(tot[0], r);
            }
        }
        if (lane == 0) __hip_atomic_fetch_add(&s_packed[b], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        wait_at_least(&s_packed[b], (uint32_t)ND * (use + 1));
        // chunk m of the buffer holds output elements g0 - shift + 4m ... + 3
        if (run_len > 0) {
            const uint32_t chunks = (shift + run_len + 3) / 4;
            T* __restrict__ dst = out + (g0 - shift);
            for (uint32_t m = (uint32_t)w * 64 + lane; m < chunks; m += ND * 64) {
                const uint32_t lo = 4 * m, hi = 4 * m + 4;
                if (lo >= shift && hi <= shift + run_len) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(buf + lo);
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + lo));
                } else {
                    // the run's first or last chunk: its elements one by one, read
                    // from LDS one by one (taking them out of a 16-byte LDS read
                    // here was compiled into four stores of its first word)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (lo + j >= shift && lo + j < shift + run_len)
                            __builtin_nontemporal_store(buf[lo + j], dst + lo + j);
                }
            }
        }
        if (lane == 0) __hip_atomic_fetch_add(&s_written[b], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int q = 0; q + 1 < kPipeTiles; ++q) {
            t[q] = t[q + 1];
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                xcl[q][c] = xcl[q + 1][c];
                tot[q][c] = tot[q + 1][c];
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int j = 0; j < VEC; ++j) e[q][r][j] = e[q + 1][r][j];
        }
        if (w == 0) post_id(p, &s_ids, k + kPipeTiles, next_id, exhausted);
        t[NEW].set(p, get_id<false>(lw, &s_ids, k + kPipeTiles), w);
    }
    record_lds_timeout(p.lb, lw);
    if (w == 0 && lane == 0) retire_workgroup(p);
}

}  // namespace dwpt
