// One pass of a least-significant-digit radix sort: a stable split of uint32
// keys (and, if given, their uint32 values) by the 8-bit digit
// (key >> shift) & 255.  Radix sort is a split by digit followed by a scan
// that gives every element its place; 32-bit keys take four such passes
// ("Lecture 7: 并行模式五 —— 前缀和 / 扫描", concept 2; PMPP chapter 9 notes,
// §9.6: the scan of the digit histogram gives each bucket's start).
//
// Three launches on the caller's stream:
//   1. radix_hist_kernel: counts every digit d in every tile t (T tiles, in
//      groups of kHistTiles consecutive tiles) and stores, digit-major, the
//      count of d in the earlier tiles of t's group at local[d * T + t] and
//      the group's count of d at group[d * G + g] (G groups);
//   2. the library's exclusive add scan of group, in place: group[d * G + g]
//      becomes the output position of group g's first key of digit d (all
//      smaller digits come first, then the same digit in earlier groups);
//   3. radix_scatter_kernel: every key's rank among the keys of its digit in
//      its tile, the tile reordered by digit in LDS, and each digit's run
//      written to its position, group[d * G + g] + local[d * T + t] onward.
// Only the group totals are scanned: 256 words per kHistTiles tiles instead
// of 256 per tile (2^28 keys: a scan of 2^20 words instead of 2^23, which
// took 22 us of the pass).
//
// Ranking inside a wavefront, one round of 64 keys at a time: every lane
// sets its bit in an LDS word kept for its digit and reads the word back,
// which gives the mask of lanes holding the same digit (a round whose keys
// all share one digit skips this).  The bits are set with 32-bit ORs into
// the word's two halves (a 64-bit OR from every lane moves twice the bytes:
// 478 -> 470 us for the scatter at 2^28 keys).  A key's rank is the number of those
// lanes below it plus the wavefront's count of the digit so far, which the
// lowest lane of the group advances by the group's size with one LDS add.
//
// Measured on MI355X with 2^28 keys: eight ballots of the digit bits find
// the same masks with about 40 more vector instructions per round, which
// made the pass 6% slower; LDS adds from many lanes to one word are slow
// (all 64 on one word: five times the time of the loads), hence the counter
// copies of the histogram pass.  Half-wavefront groups (32-bit masks, two
// count adds per round, the lower half's first) were slower: 493 against
// 478 us.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wave_ops.hpp"

namespace dwpt {

#ifndef DWPT_RS_BLOCK
#define DWPT_RS_BLOCK 512
#endif
#ifndef DWPT_RS_ITEMS
#define DWPT_RS_ITEMS 16
#endif
constexpr int kRsBlock = DWPT_RS_BLOCK;        // threads per workgroup
constexpr int kRsItems = DWPT_RS_ITEMS;        // keys per lane
constexpr int kRsWaves = kRsBlock / 64;
constexpr int kRsWaveKeys = 64 * kRsItems;     // wavefront w owns keys [w * kRsWaveKeys, ...) of the tile
constexpr int kRsTile = kRsBlock * kRsItems;   // 8192 keys
constexpr int kRsDigits = 256;
static_assert(kRsBlock >= kRsDigits, "one thread per digit");
static_assert(kRsTile == 8192, "8192-key tiles");

// Number of lanes of mask m below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Tile of workgroup b of T (one tile per workgroup).  Workgroups are dealt
// to the chip's 8 XCDs in turn (workgroup b to XCD b % 8), and each XCD has
// its own L2: XCD x takes the x-th eighth of the tiles, in order.
// Neighbouring tiles then run on one XCD at about the same time, so the
// partial cache lines that they write side by side (a digit's run of one
// tile ends where the next tile's begins) are merged in that XCD's L2
// before they go to memory.
__device__ __forceinline__ uint32_t rs_tile(uint32_t b, uint32_t T)
{
    constexpr uint32_t kXcds = 8;
    const uint32_t x = b % kXcds, i = b / kXcds, q = T / kXcds, r = T % kXcds;
    return x * q + (x < r ? x : r) + i;
}

// Keys of this lane: round v holds key tile_base + w * kRsWaveKeys + v * 64 + lane,
// so the order of (wavefront, round, lane) is the input order.  FULL: the
// whole tile lies below n.
template <bool FULL>
__device__ __forceinline__ void load_keys(const uint32_t* __restrict__ src, uint64_t base, uint64_t n, int lane,
                                          uint32_t (&k)[kRsItems])
{
#pragma unroll
    for (int v = 0; v < kRsItems; ++v) {
        const uint64_t i = base + (uint64_t)v * 64 + lane;
        k[v] = FULL || i < n ? src[i] : 0u;
    }
}

// This lane's keys of tile t.
__device__ __forceinline__ void load_tile(const uint32_t* __restrict__ src, uint32_t t, uint64_t n, int w, int lane,
                                          uint32_t (&k)[kRsItems])
{
    const uint64_t base = (uint64_t)t * kRsTile + (uint64_t)w * kRsWaveKeys;
    if ((uint64_t)(t + 1) * kRsTile <= n)
        load_keys<true>(src, base, n, lane, k);
    else
        load_keys<false>(src, base, n, lane, k);
}

// Histogram counters: every wavefront has its own, kRsCopies copies of each
// digit's counter; lane l adds to copy l % kRsCopies.  LDS adds to one word
// from many lanes of an instruction are slow (measured: 64 lanes on one word
// cost about five times the loads; up to four per word cost nothing
// visible); with 4 copies, all keys of one digit put 16 lanes on a word.  (On
// uniform digits the number of copies made no difference: 1, 2 and 4 copies
// 182.8, 182.8, 182.9 us at 2^28 keys.)
constexpr int kRsCopies = 4;
constexpr int kRsCntRow = kRsCopies * kRsDigits + 1;  // one wavefront's counters (+1: rows start in distinct banks)

// Pass 1: local[d * T + t] = number of keys of digit d in the tiles of t's
// group before t, group[d * G + g] = number of keys of digit d in group g.
// A group is kHistTiles consecutive tiles, one per wavefront of a workgroup:
// each wavefront reads its whole tile (16-byte loads, four keys each, the
// next four loads in flight while it counts; counting does not depend on the
// keys' order) and counts it into its own counters, so the only barrier comes
// at the end, where the group's counts are turned into prefixes and written,
// kHistTiles consecutive words per digit.  Measured at 2^28 keys: 182-183 us;
// a workgroup that counted its tiles one after another, every wavefront an
// eighth of each, with two barriers per tile, 193 us (one tile per workgroup:
// 225; two tiles per wavefront 197, four 241: they spill).  Groups are dealt
// to the XCDs as tiles are by rs_tile (dealt in order: 202 us).
constexpr int kHistTiles = kRsWaves;

__global__ __launch_bounds__(kRsBlock) void radix_hist_kernel(const uint32_t* __restrict__ keys, uint64_t n,
                                                              uint32_t shift, uint32_t T, uint32_t* __restrict__ local,
                                                              uint32_t* __restrict__ group, int vec)
{
    __shared__ uint32_t s_cnt[kRsWaves][kRsCntRow];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const uint32_t G = (T + kHistTiles - 1) / kHistTiles;
    if (blockIdx.x >= G) return;  // a grid of G workgroups is expected; never index past the tiles
    const uint32_t g = rs_tile(blockIdx.x, G);
    const uint32_t t = g * kHistTiles + w;  // this wavefront's tile
    uint32_t* cnt = s_cnt[w];
    for (int i = lane; i < kRsCntRow; i += 64) cnt[i] = 0u;
    uint32_t* my = cnt + (lane % kRsCopies) * kRsDigits;
    if (t < T) {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        if (vec && (uint64_t)(t + 1) * kRsTile <= n) {
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(keys + (uint64_t)t * kRsTile) + lane;
            constexpr int B = 4, NB = kRsTile / 4 / 64 / B;  // loads per batch, batches
            u32x4_t q[B], q2[B];
#pragma unroll
            for (int j = 0; j < B; ++j) q[j] = __builtin_nontemporal_load(src + j * 64);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b + 1 < NB) {
#pragma unroll
                    for (int j = 0; j < B; ++j) q2[j] = __builtin_nontemporal_load(src + ((b + 1) * B + j) * 64);
                }
#pragma unroll
                for (int j = 0; j < B; ++j) {
                    atomicAdd(my + ((q[j].x >> shift) & 255u), 1u);
                    atomicAdd(my + ((q[j].y >> shift) & 255u), 1u);
                    atomicAdd(my + ((q[j].z >> shift) & 255u), 1u);
                    atomicAdd(my + ((q[j].w >> shift) & 255u), 1u);
                }
#pragma unroll
                for (int j = 0; j < B; ++j) q[j] = q2[j];
            }
        } else {  // the partial last tile, or keys not 16-byte aligned: one key per lane and step
            const uint64_t base = (uint64_t)t * kRsTile;
            for (uint32_t i = lane; i < (uint32_t)kRsTile && base + i < n; i += 64)
                atomicAdd(my + ((keys[base + i] >> shift) & 255u), 1u);
        }
    }
    // fold the copies into copy 0 (a wavefront's LDS operations take effect
    // in order, so its adds are all in)
#pragma unroll
    for (int k = 0; k < kRsDigits / 64; ++k) {
        const int d = lane + 64 * k;
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < kRsCopies; ++i) c += cnt[i * kRsDigits + d];
        cnt[d] = c;
    }
    __syncthreads();
    // thread d: the counts of the group's tiles become prefixes in place
    if (threadIdx.x < kRsDigits) {
        const int d = threadIdx.x;
        uint32_t run = 0;
#pragma unroll
        for (int q = 0; q < kHistTiles; ++q) {
            const uint32_t c = s_cnt[q][d];
            s_cnt[q][d] = run;
            run += c;
        }
        group[(uint64_t)d * G + g] = run;
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < kRsDigits * kHistTiles; i += kRsBlock) {
        const uint32_t d = i / kHistTiles, q = i % kHistTiles;
        if (g * kHistTiles + q < T) local[(uint64_t)d * T + g * kHistTiles + q] = s_cnt[q][d];
    }
}

struct RsShared {
    uint32_t cnt[kRsWaves][kRsDigits];  // per wavefront: running count, then the wavefront's first slot of the digit
    uint32_t start[kRsDigits];          // digit's first slot in the reordered tile
    uint32_t base[kRsDigits];           // output position of the tile's first key of the digit, minus start
    uint32_t part[kRsDigits / 64];
    union {
        uint32_t buf[kRsTile];            // the tile reordered by digit: keys, then values
        uint64_t grp[kRsWaves][kRsDigits];  // while ranking: per wavefront, the lanes holding each digit
    };
    uint8_t dig[kRsTile];               // digit of every slot (for the values)
};

// One tile: keys k (values x) of this lane, counters and digit groups clear.
template <bool VALS, bool FULL>
__device__ __forceinline__ void scatter_tile(RsShared& sh, const uint32_t (&k)[kRsItems], const uint32_t (&x)[kRsItems],
                                             uint64_t n, uint32_t shift, uint32_t g, uint64_t tile_base,
                                             uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out)
{
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const uint64_t base = tile_base + (uint64_t)w * kRsWaveKeys;
    const uint32_t cnt = FULL ? (uint32_t)kRsTile : (uint32_t)(n - tile_base);

    // rank of every key among the earlier keys of its digit in this
    // wavefront: the lowest lane of each group of equal digits adds the
    // group's size to the digit's counter and receives the count before it,
    // which the other lanes of the group fetch from it.  The adds of
    // successive rounds need not wait for each other.
    uint32_t rank[kRsItems];
    const uint32_t my_bit = 1u << (lane & 31);
#pragma unroll
    for (int v = 0; v < kRsItems; ++v) {
        const bool valid = FULL || base + (uint64_t)v * 64 + lane < n;
        const uint32_t d = (k[v] >> shift) & 255u;
        // the lanes holding digit d: every lane sets its bit in the digit's
        // word, reads the word back, and the lowest of them clears it again
        // (a wavefront's LDS operations take effect in order).  A round whose
        // keys share one digit skips this.
        const uint64_t vm = wave_ballot(valid);
        const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
        uint64_t m = vm;
        if (wave_ballot(valid && d == d0) != vm) {
            uint64_t* slot = &sh.grp[w][d];
            // lanes 0-31 set bits of the low half, lanes 32-63 of the high half
            if (valid) atomicOr(reinterpret_cast<uint32_t*>(slot) + (lane >> 5), my_bit);
            m = valid ? *slot : 0ull;
            if (valid && lanes_below(m) == 0) *slot = 0ull;
        }
        const uint32_t below = lanes_below(m);
        uint32_t before = 0;
        if (valid && below == 0) before = atomicAdd(&sh.cnt[w][d], (uint32_t)__builtin_popcountll(m));
        const int first = (int)__builtin_ctzll(m | (1ull << 63));  // lowest lane of the group
        rank[v] = (uint32_t)__builtin_amdgcn_ds_bpermute(first << 2, (int)before) + below;
    }
    __syncthreads();

    // per digit: exclusive prefix over the wavefronts, the tile's count, and
    // the exclusive scan of the counts over the digits
    if (threadIdx.x < kRsDigits) {
        const int d = threadIdx.x;
        uint32_t run = 0;
#pragma unroll
        for (int j = 0; j < kRsWaves; ++j) {
            const uint32_t c = sh.cnt[j][d];
            sh.cnt[j][d] = run;
            run += c;
        }
        const auto add = [](uint32_t a, uint32_t b) { return a + b; };
        const uint32_t incl = wave_inclusive_scan(run, 0u, add);
        if (lane == 63) sh.part[w] = incl;
        sh.start[d] = incl - run;  // within this wavefront's 64 digits, completed below
    }
    __syncthreads();
    if (threadIdx.x < kRsDigits) {
        const int d = threadIdx.x;
        uint32_t before = 0;
#pragma unroll
        for (int j = 0; j < kRsDigits / 64; ++j)
            if (j < w) before += sh.part[j];
        const uint32_t start = sh.start[d] + before;
        sh.base[d] = g - start;
#pragma unroll
        for (int j = 0; j < kRsWaves; ++j) sh.cnt[j][d] += start;
    }
    __syncthreads();

    // reorder the tile by digit (stable) in LDS; rank[] becomes the slot
#pragma unroll
    for (int v = 0; v < kRsItems; ++v) {
        const bool valid = FULL || base + (uint64_t)v * 64 + lane < n;
        const uint32_t d = (k[v] >> shift) & 255u;
        rank[v] += sh.cnt[w][d];
        if (valid) {
            sh.buf[rank[v]] = k[v];
            if (VALS) sh.dig[rank[v]] = (uint8_t)d;
        }
    }
    __syncthreads();

    // consecutive slots of a digit go to consecutive output positions
#pragma unroll
    for (int v = 0; v < kRsItems; ++v) {
        const uint32_t j = (uint32_t)v * kRsBlock + threadIdx.x;
        if (FULL || j < cnt) {
            const uint32_t key = sh.buf[j];
            keys_out[sh.base[(key >> shift) & 255u] + j] = key;
        }
    }
    if (VALS) {
        __syncthreads();
#pragma unroll
        for (int v = 0; v < kRsItems; ++v)
            if (FULL || base + (uint64_t)v * 64 + lane < n) sh.buf[rank[v]] = x[v];
        __syncthreads();
#pragma unroll
        for (int v = 0; v < kRsItems; ++v) {
            const uint32_t j = (uint32_t)v * kRsBlock + threadIdx.x;
            if (FULL || j < cnt) vals_out[sh.base[sh.dig[j]] + j] = sh.buf[j];
        }
    }
}

// Pass 3: `local` as pass 1 left it, `group` its group counts after the
// exclusive scan.  Writes the tile's keys (and values) to their places in
// keys_out (vals_out).
//
// Registers: the workgroup's LDS (51 KiB) leaves room for three workgroups
// per CU, which at 512 threads need six wavefronts per SIMD, i.e. at most 80
// VGPRs.  The keys-only kernel is held to that (82 -> 80 VGPRs, no spills;
// 2^28 keys 522 -> 478 us); with values it would spill (100 bytes per lane:
// 440 -> 889 us at 2^27 pairs), so that one keeps two workgroups per CU.
template <bool VALS>
__global__ __launch_bounds__(kRsBlock) __attribute__((amdgpu_waves_per_eu(VALS ? 1 : 6))) void radix_scatter_kernel(const uint32_t* __restrict__ keys,
                                                                 const uint32_t* __restrict__ vals, uint64_t n,
                                                                 uint32_t shift, uint32_t T,
                                                                 const uint32_t* __restrict__ local,
                                                                 const uint32_t* __restrict__ group,
                                                                 uint32_t* __restrict__ keys_out,
                                                                 uint32_t* __restrict__ vals_out)
{
    __shared__ RsShared sh;
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const uint32_t t = rs_tile(blockIdx.x, T);
    uint32_t k[kRsItems], x[kRsItems];
    load_tile(keys, t, n, w, lane, k);
    if (VALS) load_tile(vals, t, n, w, lane, x);
    const uint32_t G = (T + kHistTiles - 1) / kHistTiles;
    const uint32_t g = threadIdx.x < kRsDigits
                           ? group[(uint64_t)threadIdx.x * G + t / kHistTiles] + local[(uint64_t)threadIdx.x * T + t]
                           : 0u;
    for (int i = threadIdx.x; i < kRsWaves * kRsDigits; i += kRsBlock) {
        (&sh.cnt[0][0])[i] = 0u;
        (&sh.grp[0][0])[i] = 0ull;
    }
    __syncthreads();  // counters and groups cleared
    const uint64_t tile_base = (uint64_t)t * kRsTile;
    if (tile_base + kRsTile <= n)
        scatter_tile<VALS, true>(sh, k, x, n, shift, g, tile_base, keys_out, vals_out);
    else
        scatter_tile<VALS, false>(sh, k, x, n, shift, g, tile_base, keys_out, vals_out);
}

}  // namespace dwpt
