// pipeline_model.cpp -- host model of the persistent scan kernel's inter-tile
// protocol, for CPU tests (plain C++17 threads; also built with
// ThreadSanitizer).  Not part of the library: it restates, step by step and
// one std::thread per wavefront, what tile_scan_persistent and its resolver
// do between workgroups, so that schedules the GPU never shows on demand --
// workgroups starting late and in any order, waves delayed at any step --
// can be run by the thousand, and so that a data race on the LDS rings or a
// lost tile total shows up on the CPU instead of as a hang on the GPU.
//
// Modelled, as in the kernel:
//  * roles from a counter (role 0 resolves), tile numbers from a counter: a
//    first batch of WAIT + 1 consecutive numbers per workgroup with one
//    atomic, or in consecutive pieces one round trip apart, later numbers
//    one iteration ahead (ask_id / post_id);
//  * per workgroup: ND data waves with WAIT + 1 tiles in flight, a prefix
//    wave, LDS rings of S slots with sequence numbers (tile-number ring,
//    prefix/arrival ring), the last data wave to hand a tile's total over
//    publishes it;
//  * status words tag << 49 | payload, tag = epoch << 3 | flag << 2 | state,
//    multi-word payloads accepted only when all tags agree, epochs instead of
//    clearing (cleared at the 12-bit wrap);
//  * the streaming resolver (windows of 64 * SPAN totals, publishes every
//    tile's exclusive prefix) and the prefix wave's polls of it;
//  * bounded waits: spin limits, the launch's abort word read every 64 polls
//    by status-word waits, the workgroup's LDS flag, the prefix wave releasing
//    every slot when it gives up, sticky give-ups.
// A wave's 64 lanes are not modelled: wave-wide steps (a wavefront scan, a
// 64-entry window) run as loops in the wave's thread.
//
// Usage: pipeline_model key=value ...   (see Params); prints one line
//   "result ok=<0|1> err=<bits> mismatches=<n> launches=<n> max_launch_ms=<x> full_budgets=<n>"
// and exits 0 when ok (all outputs equal the sequential scan, no error bit),
// 1 otherwise; with lose_tile >= 0 (a total deliberately never published) it
// exits 0 when the launch still finished and reported a timeout.
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <random>
#include <string>
#include <thread>
#include <vector>

namespace {

struct Params {
    int nd = 3;            // data waves per workgroup
    int wait = 3;          // tiles per data wave waiting for their prefix
    int slots = 16;        // LDS ring slots (the kernel: 16 >= 2 * wait)
    int span = 1;          // resolver window: 64 * span tiles
    int first_piece = 0;   // first tile numbers: one batch (0), or a piece of this many, then pieces of next_piece
    int next_piece = 3;
    int wgs = 5;           // workgroups launched (one becomes the resolver)
    int tiles = 300;       // tiles per launch
    int share = 3;         // elements per data wave and tile
    int launches = 3;      // launches on one workspace (epochs advance)
    int op = 1;            // 0: uint32 add (one word), 1: affine maps (two words)
    int delay = 200;       // per-mille chance of a random pause at each step
    int max_pause_us = 30;
    uint64_t spin = 1u << 22;  // spin limit (status-word polls)
    int lose_tile = -1;    // >= 0: that tile's total is never published
    int sticky = 1;        // 0: the earlier, non-sticky budgets (no abort word)
    int epoch_start = 1;   // first epoch (to run across the 12-bit wrap)
    int kernel = 0;        // 0: persistent kernel; 1: one workgroup per tile, two-level look-back
    int resident = 12;     // kernel 1: workgroups alive at once
    unsigned seed = 1;
};

constexpr int kPayloadBits = 49;
constexpr uint64_t kPayloadMask = (1ull << kPayloadBits) - 1;
constexpr uint32_t kEpochLimit = 1u << 12;
enum : uint32_t { kEmpty = 0, kAggregate = 1, kPrefix = 2 };
enum : uint32_t { kErrTimeout = 1 };
constexpr uint64_t kAbortCheck = 64;

// ---------------------------------------------------------------- operators
struct Val {
    uint32_t a, b;  // affine map x -> a x + b; for add only b is used
};
Val identity(int op) { return op ? Val{1u, 0u} : Val{0u, 0u}; }
// earlier (+) later
Val combine(int op, Val e, Val l)
{
    if (op) return {l.a * e.a, l.a * e.b + l.b};
    return {0u, e.b + l.b};
}
int words(int op) { return op ? 2 : 1; }

struct Mem {
    std::vector<std::atomic<uint64_t>> agg, excl;  // tile totals; published prefixes (kernel 1: group statuses)
    std::atomic<uint32_t> tile_ctr{0}, role_ctr{0}, retired{0};
    std::atomic<uint32_t> tile_ctr1{0};  // kernel 1's counter (never reset; the host keeps its base)
    uint32_t ctr_base = 0;
    std::atomic<uint32_t> err{0}, abort_word{0};
    std::atomic<uint64_t> full_budgets{0};  // checks: waits that polled their whole budget
    uint32_t epoch = 0;
    explicit Mem(size_t n) : agg(n), excl(n)
    {
        for (auto& w : agg) w.store(0);
        for (auto& w : excl) w.store(0);
    }
};

uint64_t tag(uint32_t epoch, uint32_t state) { return (uint64_t)((epoch << 3) | state) << kPayloadBits; }

// Status words are release stores and acquire loads here, where the kernel
// uses relaxed agent-scope atomics (the payload travels in the word itself).
// The stronger order stands for what the GPU gives the protocol through
// in-order waves and an LDS without caches: a wave that sees a published word
// also sees the LDS writes its producers made before publishing.  It lets
// ThreadSanitizer check every access to the LDS rings (plain data here, as
// in the kernel) against the protocol's ordering.
void publish(Mem& m, std::vector<std::atomic<uint64_t>>& arr, size_t tile, int op, Val v, uint32_t state)
{
    const uint64_t t = tag(m.epoch, state);
    if (op) {
        arr[2 * tile].store(t | v.a, std::memory_order_release);
        arr[2 * tile + 1].store(t | v.b, std::memory_order_release);
    } else {
        arr[tile].store(t | v.b, std::memory_order_release);
    }
}

// true (and the value) when the words hold this launch's entry of a state in `states`
bool read_entry(Mem& m, std::vector<std::atomic<uint64_t>>& arr, size_t tile, int op, bool prefix_only, Val& out)
{
    const int W = words(op);
    uint64_t raw[2];
    for (int q = 0; q < W; ++q) raw[q] = arr[W * tile + q].load(std::memory_order_acquire);
    const uint32_t t0 = (uint32_t)(raw[0] >> kPayloadBits);
    for (int q = 1; q < W; ++q)
        if ((uint32_t)(raw[q] >> kPayloadBits) != t0) return false;  // torn across words: not yet
    if ((t0 >> 3) != m.epoch) return false;
    const uint32_t state = t0 & 3u;
    if (state == kEmpty || (prefix_only && state != kPrefix)) return false;
    out = op ? Val{(uint32_t)(raw[0] & kPayloadMask), (uint32_t)(raw[1] & kPayloadMask)}
             : Val{0u, (uint32_t)(raw[0] & kPayloadMask)};
    return true;
}

// ---------------------------------------------------------------- schedule noise
struct Noise {
    std::mt19937 rng;
    int permille, max_us;
    Noise(unsigned seed, int p, int mx) : rng(seed), permille(p), max_us(mx) {}
    void step()
    {
        if ((int)(rng() % 1000) >= permille) return;
        const int us = (int)(rng() % (unsigned)(max_us + 1));
        if (us == 0) std::this_thread::yield();
        else std::this_thread::sleep_for(std::chrono::microseconds(us));
    }
};

void poll_pause() { std::this_thread::yield(); }

// ---------------------------------------------------------------- bounded waits
// status-word waits (resolver, prefix wave): budget, abort word every 64 polls
bool give_up(Mem& m, const Params& P, uint64_t& polls)
{
    ++polls;
    if (polls > P.spin) {
        if (polls == P.spin + 1) m.full_budgets.fetch_add(1, std::memory_order_relaxed);
        m.err.fetch_or(kErrTimeout, std::memory_order_relaxed);
        if (P.sticky) m.abort_word.store(m.epoch, std::memory_order_relaxed);
        return true;
    }
    if (P.sticky && polls % kAbortCheck == 0 && m.abort_word.load(std::memory_order_relaxed) == m.epoch) {
        polls = P.spin + 1;
        return true;
    }
    return false;
}

// ---------------------------------------------------------------- workgroup LDS
struct Slot {
    std::atomic<uint32_t> arrived{0};
    std::atomic<uint32_t> prefix_seq{0};
    Val prefix{};
    std::vector<Val> wave_total;  // plain data, ordered by `arrived` and `prefix_seq`
    // checks, not protocol: which of the workgroup's tiles (k) each value belongs to
    uint32_t prefix_k = UINT32_MAX;
    std::vector<uint32_t> wave_total_k;
};
struct Lds {
    std::vector<Slot> slot;
    std::vector<uint32_t> id;  // plain data, ordered by `seq`
    std::vector<std::atomic<uint32_t>> seq;
    std::atomic<uint32_t> abort{0};
    Lds(const Params& P) : slot(P.slots), id(P.slots), seq(P.slots)
    {
        for (auto& s : slot) {
            s.wave_total.assign(P.nd, Val{});
            s.wave_total_k.assign(P.nd, UINT32_MAX);
        }
        for (auto& s : seq) s.store(0);
    }
};

struct LdsWait {
    uint64_t limit;
    std::atomic<uint32_t>* flag;
    bool gave_up = false;
    bool fail_batch(uint64_t& polls)
    {
        polls += kAbortCheck;
        if (polls > limit || flag->load(std::memory_order_relaxed) != 0u) {
            flag->store(1u, std::memory_order_relaxed);
            gave_up = true;
            return true;
        }
        return false;
    }
};

void record_lds_timeout(Mem& m, const Params& P, const LdsWait& lw)
{
    if (!lw.gave_up) return;
    m.err.fetch_or(kErrTimeout, std::memory_order_relaxed);
    if (P.sticky) m.abort_word.store(m.epoch, std::memory_order_relaxed);
}

void wait_seq(LdsWait& lw, std::atomic<uint32_t>& seq, uint32_t want)
{
    uint64_t polls = 0;
    while (true) {
        for (uint64_t i = 0; i < kAbortCheck; ++i) {
            if (seq.load(std::memory_order_acquire) >= want) return;
            poll_pause();
        }
        if (lw.fail_batch(polls)) return;
    }
}

uint32_t get_id(LdsWait& lw, Lds& L, const Params& P, uint32_t k)
{
    uint64_t polls = 0;
    std::atomic<uint32_t>& s = L.seq[k % P.slots];
    while (true) {
        for (uint64_t i = 0; i < kAbortCheck; ++i) {
            if (s.load(std::memory_order_acquire) >= k + 1) return L.id[k % P.slots];
            poll_pause();
        }
        if (lw.fail_batch(polls)) return UINT32_MAX;
    }
}

void put_id(Lds& L, const Params& P, uint32_t k, uint32_t id)
{
    L.id[k % P.slots] = id;
    L.seq[k % P.slots].store(k + 1, std::memory_order_release);
}

// ---------------------------------------------------------------- launch state
struct Launch {
    const Params& P;
    Mem& m;
    const std::vector<Val>& in;
    std::vector<Val>& out;  // each element written by exactly one wave
    uint32_t num_tiles;
    std::atomic<int> lost_published{0};
    // checks: a slot read for tile k held another tile's value (ring reused too early)
    std::atomic<uint64_t> stale_prefix{0}, stale_total{0}, stale_wave_prefix{0};
    std::mutex bar_mu;
};

uint32_t tile_elems(const Params& P) { return (uint32_t)(P.nd * P.share); }

void retire(Launch& Lc, uint32_t grid)
{
    const uint32_t d = Lc.m.retired.fetch_add(1, std::memory_order_relaxed);
    if (d == grid - 1) {
        Lc.m.tile_ctr.store(0, std::memory_order_relaxed);
        Lc.m.role_ctr.store(0, std::memory_order_relaxed);
        Lc.m.retired.store(0, std::memory_order_relaxed);
    }
}

// the streaming resolver (one wave)
void resolve_stream(Launch& Lc, Noise& nz)
{
    const Params& P = Lc.P;
    Mem& m = Lc.m;
    const uint32_t W = 64u * (uint32_t)P.span;
    Val carry = identity(P.op);
    uint64_t polls = 0;
    for (uint64_t B = 0; B < Lc.num_tiles; B += W) {
        const uint32_t want = (uint32_t)std::min<uint64_t>(W, Lc.num_tiles - B);
        std::vector<bool> have(W, false);
        std::vector<Val> val(W, identity(P.op));
        uint32_t done = 0;
        while (true) {
            for (uint32_t j = 0; j < want; ++j)
                if (!have[j]) have[j] = read_entry(m, m.agg, B + j, P.op, false, val[j]);
            uint32_t ready = 0;
            while (ready < want && have[ready]) ++ready;
            if (ready > done) {
                Val run = carry;
                for (uint32_t j = 0; j < ready; ++j) {
                    if (j >= done) publish(m, m.excl, B + j, P.op, run, kPrefix);
                    run = combine(P.op, run, val[j]);
                }
                done = ready;
                nz.step();
                if (done == want) {
                    carry = run;
                    break;
                }
            }
            if (!P.sticky) {
                // the earlier budget: restarted after every give-up
                if (++polls > P.spin) {
                    m.full_budgets.fetch_add(1, std::memory_order_relaxed);
                    m.err.fetch_or(kErrTimeout, std::memory_order_relaxed);
                    for (uint32_t j = 0; j < W; ++j) have[j] = true;
                    polls = 0;
                    continue;
                }
            } else if (give_up(m, P, polls)) {
                for (uint32_t j = 0; j < W; ++j) have[j] = true;
                continue;
            }
            poll_pause();
        }
    }
}

// the prefix wave of a data workgroup
void fetch_prefixes(Launch& Lc, Lds& L, Noise& nz)
{
    const Params& P = Lc.P;
    Mem& m = Lc.m;
    LdsWait lw{P.spin * 16, &L.abort};
    uint64_t polls = 0;
    for (uint32_t k = 0;; ++k) {
        const uint32_t tile = get_id(lw, L, P, k);
        if (tile >= Lc.num_tiles) break;
        if (P.sticky && polls <= P.spin) polls = 0;
        if (!P.sticky) polls = 0;
        Val excl = identity(P.op);
        while (!read_entry(m, m.excl, tile, P.op, true, excl)) {
            if (give_up(m, P, polls)) {
                excl = identity(P.op);
                L.abort.store(1u, std::memory_order_relaxed);
                break;
            }
            poll_pause();
        }
        nz.step();
        Slot& s = L.slot[k % P.slots];
        s.prefix = excl;
        s.prefix_k = k;
        s.prefix_seq.store(k + 1, std::memory_order_release);
    }
    if (lw.gave_up)
        for (auto& s : L.slot) s.prefix_seq.store(UINT32_MAX, std::memory_order_release);
    record_lds_timeout(m, P, lw);
}

struct WaveTile {
    uint32_t tile;
    std::vector<Val> e;  // the wave's share of the tile
};

// a data wave: the persistent loop with WAIT + 1 tiles in flight
void data_wave(Launch& Lc, Lds& L, int w, uint32_t grid, Noise& nz)
{
    const Params& P = Lc.P;
    Mem& m = Lc.m;
    const int NT = P.wait + 1;
    const uint32_t TE = tile_elems(P);
    LdsWait lw{P.spin * 16, &L.abort};
    bool exhausted = false;
    if (w == 0 && P.first_piece <= 0) {
        const uint32_t b = m.tile_ctr.fetch_add((uint32_t)NT, std::memory_order_relaxed);
        for (int q = 0; q < NT; ++q)
            put_id(L, P, (uint32_t)q, (uint64_t)b + q < Lc.num_tiles ? b + q : Lc.num_tiles);
        exhausted = (uint64_t)b + NT >= Lc.num_tiles;
    } else if (w == 0) {
        // the first numbers in consecutive pieces, each taken once the one
        // before has come back (take_first_pieces)
        bool ex = false;
        for (int q = 0; q < NT;) {
            const int want = q == 0 ? P.first_piece : P.next_piece;
            const int mq = want < NT - q ? want : NT - q;
            uint32_t b = Lc.num_tiles;
            if (!ex) b = m.tile_ctr.fetch_add((uint32_t)mq, std::memory_order_relaxed);
            for (int j = 0; j < mq; ++j)
                put_id(L, P, (uint32_t)(q + j), !ex && (uint64_t)b + j < Lc.num_tiles ? b + j : Lc.num_tiles);
            ex = ex || (uint64_t)b + mq >= Lc.num_tiles;
            q += mq;
            nz.step();
        }
        exhausted = ex;
    }
    auto load = [&](WaveTile& t) {
        t.e.assign(P.share, identity(P.op));
        if (t.tile >= Lc.num_tiles) return;
        for (int j = 0; j < P.share; ++j) {
            const uint64_t i = (uint64_t)t.tile * TE + (uint64_t)w * P.share + j;
            t.e[j] = Lc.in[i];
        }
    };
    auto hand_over = [&](const WaveTile& t, uint32_t k) {
        Val tot = identity(P.op);
        for (const Val& v : t.e) tot = combine(P.op, tot, v);
        Slot& s = L.slot[k % P.slots];
        s.wave_total[w] = tot;
        s.wave_total_k[w] = k;
        const uint32_t old = s.arrived.fetch_add(1, std::memory_order_acq_rel);
        if (old != (k / (uint32_t)P.slots) * (uint32_t)P.nd + (uint32_t)(P.nd - 1)) return;
        Val total = identity(P.op);
        for (int q = 0; q < P.nd; ++q) {
            if (s.wave_total_k[q] != k) Lc.stale_total.fetch_add(1);
            total = combine(P.op, total, s.wave_total[q]);
        }
        if ((int)t.tile == P.lose_tile) {
            Lc.lost_published.store(1);
            return;  // deliberately lost
        }
        publish(m, m.agg, t.tile, P.op, total, kAggregate);
    };
    std::vector<WaveTile> t(NT);
    for (int q = 0; q < NT; ++q) t[q].tile = get_id(lw, L, P, (uint32_t)q);
    for (int q = 0; q < NT; ++q) load(t[q]);
    for (int q = 0; q < NT; ++q) {
        nz.step();
        if (t[q].tile < Lc.num_tiles) hand_over(t[q], (uint32_t)q);
    }
    const int NEW = NT - 1, PUB = P.wait - 1;
    for (uint32_t k = 0; t[0].tile < Lc.num_tiles; ++k) {
        uint32_t next_id = Lc.num_tiles;
        if (w == 0 && !exhausted) next_id = m.tile_ctr.fetch_add(1, std::memory_order_relaxed);
        nz.step();
        if (k >= 1 && t[NEW].tile < Lc.num_tiles) load(t[NEW]);
        if (k >= 2 && t[PUB].tile < Lc.num_tiles) hand_over(t[PUB], k + (uint32_t)PUB);
        nz.step();
        Slot& s = L.slot[k % P.slots];
        wait_seq(lw, s.prefix_seq, k + 1);
        Val wave_prefix = identity(P.op);
        for (int q = 0; q < w; ++q) {
            if (s.wave_total_k[q] != k) Lc.stale_wave_prefix.fetch_add(1);
            wave_prefix = combine(P.op, wave_prefix, s.wave_total[q]);
        }
        if (s.prefix_k != k) Lc.stale_prefix.fetch_add(1);
        Val run = combine(P.op, s.prefix, wave_prefix);
        for (int j = 0; j < P.share; ++j) {
            run = combine(P.op, run, t[0].e[j]);
            const uint64_t i = (uint64_t)t[0].tile * TE + (uint64_t)w * P.share + j;
            Lc.out[i] = run;
        }
        nz.step();
        for (int q = 0; q + 1 < NT; ++q) t[q] = t[q + 1];
        if (w == 0) {
            put_id(L, P, k + (uint32_t)NT, next_id);
            exhausted = exhausted || next_id >= Lc.num_tiles;
        }
        t[NEW].tile = get_id(lw, L, P, k + (uint32_t)NT);
    }
    record_lds_timeout(m, P, lw);
    if (w == 0) retire(Lc, grid);
}

// one workgroup: role, then its waves as threads
void workgroup(Launch& Lc, uint32_t grid, unsigned seed)
{
    const Params& P = Lc.P;
    Noise start(seed, 1000, P.max_pause_us);
    if (P.delay) start.step();  // workgroups start late and in any order
    const uint32_t role = Lc.m.role_ctr.fetch_add(1, std::memory_order_relaxed);
    if (role == 0) {
        Noise nz(seed * 7 + 1, P.delay, P.max_pause_us);
        resolve_stream(Lc, nz);
        retire(Lc, grid);
        return;
    }
    Lds L(P);  // cleared before any wave of the workgroup runs (the kernel's barrier)
    std::vector<std::thread> waves;
    for (int w = 0; w < P.nd; ++w)
        waves.emplace_back([&Lc, &L, w, grid, seed, &P] {
            Noise nz(seed * 131 + (unsigned)w, P.delay, P.max_pause_us);
            data_wave(Lc, L, w, grid, nz);
        });
    waves.emplace_back([&Lc, &L, seed, &P] {
        Noise nz(seed * 977 + 5, P.delay, P.max_pause_us);
        fetch_prefixes(Lc, L, nz);
    });
    for (auto& th : waves) th.join();
}


// ---------------------------------------------------------------- kernel 1
// One workgroup per tile: the data waves hand the tile total over in LDS and
// the last one publishes it (AGGREGATE, or PREFIX for tile 0); meanwhile a
// look-back wave folds the earlier tiles of the tile's group of 64, then the
// earlier groups, publishes the group's statuses when the tile closes a group,
// waits for the tile total and publishes the tile's PREFIX.
enum : int { kWinFound = 0, kWinBoundary = 1, kWinNone = 2, kWinTimeout = 3 };

struct Handover {
    std::atomic<uint32_t> arrived{0}, total_ready{0};
    std::vector<Val> wave;  // plain data
    Val total{};
    Val excl{};
    bool known = false;
    std::atomic<uint32_t> at_barrier{0};
};

// Folds entries top-63 .. top of `arr` (entry j < lo: a boundary, the
// identity), starting at the highest terminal entry (PREFIX or boundary),
// once every entry above it is present.
int fold_window(Mem& m, const Params& P, std::vector<std::atomic<uint64_t>>& arr, int64_t top, int64_t lo, Val& out,
                uint64_t& polls)
{
    std::vector<bool> have(64, false), term(64, false);
    std::vector<Val> val(64, identity(P.op));
    for (int l = 0; l < 64; ++l)
        if (top - 63 + l < lo) have[l] = term[l] = true;
    while (true) {
        for (int l = 0; l < 64; ++l) {
            if (have[l]) continue;
            Val v;
            const size_t j = (size_t)(top - 63 + l);
            if (read_entry(m, arr, j, P.op, false, v)) {
                have[l] = true;
                val[l] = v;
                Val dummy;
                term[l] = read_entry(m, arr, j, P.op, true, dummy);  // a PREFIX
                if (term[l]) val[l] = dummy;
            }
        }
        int p = -1;
        for (int l = 63; l >= 0; --l)
            if (term[l]) {
                p = l;
                break;
            }
        bool ready = true;
        for (int l = (p < 0 ? 0 : p); l < 64; ++l)
            if (!have[l]) ready = false;
        if (!ready) {
            if (give_up(m, P, polls)) {
                out = identity(P.op);
                return kWinTimeout;
            }
            poll_pause();
            continue;
        }
        Val acc = identity(P.op);
        for (int l = (p < 0 ? 0 : p); l < 64; ++l) acc = combine(P.op, acc, val[l]);
        out = acc;
        if (p < 0) return kWinNone;
        return (top - 63 + p < lo) ? kWinBoundary : kWinFound;
    }
}

void wait_total(Mem& m, const Params& P, Handover& h)
{
    uint64_t polls = 0;
    while (h.total_ready.load(std::memory_order_acquire) == 0u) {
        if (give_up(m, P, polls)) return;
        poll_pause();
    }
}

void one_tile_workgroup(Launch& Lc, unsigned seed)
{
    const Params& P = Lc.P;
    Mem& m = Lc.m;
    const uint32_t TE = tile_elems(P);
    const uint32_t tile = m.tile_ctr1.fetch_add(1, std::memory_order_relaxed) - m.ctr_base;
    if (tile >= Lc.num_tiles) {
        m.err.fetch_or(2u);
        return;
    }
    Handover h;
    h.wave.assign(P.nd, Val{});
    const int nthreads = P.nd + 1;
    auto barrier = [&h, nthreads]() {
        h.at_barrier.fetch_add(1, std::memory_order_acq_rel);
        while (h.at_barrier.load(std::memory_order_acquire) < (uint32_t)nthreads) std::this_thread::yield();
    };
    std::vector<std::thread> waves;
    for (int w = 0; w < P.nd; ++w)
        waves.emplace_back([&, w] {
            Noise nz(seed * 131 + (unsigned)w, P.delay, P.max_pause_us);
            Val tot = identity(P.op);
            std::vector<Val> e(P.share);
            for (int j = 0; j < P.share; ++j) {
                e[j] = Lc.in[(uint64_t)tile * TE + (uint64_t)w * P.share + j];
                tot = combine(P.op, tot, e[j]);
            }
            nz.step();
            h.wave[w] = tot;
            if (h.arrived.fetch_add(1, std::memory_order_acq_rel) == (uint32_t)(P.nd - 1)) {
                Val total = identity(P.op);
                for (int q = 0; q < P.nd; ++q) total = combine(P.op, total, h.wave[q]);
                h.known = (tile == 0);
                h.total = total;
                if ((int)tile == P.lose_tile) Lc.lost_published.store(1);
                else publish(m, m.agg, tile, P.op, total, h.known ? kPrefix : kAggregate);
                h.total_ready.store(1, std::memory_order_release);
            }
            barrier();
            Val run = h.excl;
            for (int q = 0; q < w; ++q) run = combine(P.op, run, h.wave[q]);
            for (int j = 0; j < P.share; ++j) {
                run = combine(P.op, run, e[j]);
                Lc.out[(uint64_t)tile * TE + (uint64_t)w * P.share + j] = run;
            }
        });
    waves.emplace_back([&] {
        Noise nz(seed * 977 + 5, P.delay, P.max_pause_us);
        const int64_t g = (int64_t)(tile >> 6);
        const bool last_in_group = (tile & 63u) == 63u;
        uint64_t polls = 0;
        Val acc;
        const int r = fold_window(m, P, m.agg, (int64_t)tile - 1, g << 6, acc, polls);
        nz.step();
        if (r == kWinBoundary && g > 0) {
            if (last_in_group) {
                wait_total(m, P, h);
                publish(m, m.excl, (size_t)g, P.op, combine(P.op, acc, h.total), kAggregate);
            }
            Val gacc = identity(P.op);
            if (g == 1) {
                // the second group folds the first group's 64 tile words
                (void)fold_window(m, P, m.agg, 63, 0, gacc, polls);
            } else {
                for (int64_t top = g - 1; top >= 0; top -= 64) {
                    Val wv;
                    const int rr = fold_window(m, P, m.excl, top, 0, wv, polls);
                    gacc = combine(P.op, wv, gacc);
                    if (rr != kWinNone) break;
                }
            }
            acc = combine(P.op, gacc, acc);
        }
        wait_total(m, P, h);
        nz.step();
        const Val incl = combine(P.op, acc, h.total);
        const bool lost = (int)tile == P.lose_tile;  // a tile that never publishes anything
        if (!h.known && !lost) publish(m, m.agg, tile, P.op, incl, kPrefix);
        if (last_in_group && !lost) publish(m, m.excl, (size_t)g, P.op, incl, kPrefix);
        h.excl = acc;
        barrier();
    });
    for (auto& th : waves) th.join();
}

void run_one_tile_launch(Launch& Lc, unsigned seed)
{
    const Params& P = Lc.P;
    // workgroups start in tile-counter order as resources free up: at most
    // `resident` alive at once
    std::vector<std::thread> live;
    std::vector<std::atomic<int>> done(Lc.num_tiles);
    for (auto& d : done) d.store(0);
    std::atomic<int> alive{0};
    std::vector<std::thread> all;
    for (uint32_t i = 0; i < Lc.num_tiles; ++i) {
        while (alive.load() >= P.resident) std::this_thread::yield();
        alive.fetch_add(1);
        all.emplace_back([&Lc, &alive, seed, i] {
            one_tile_workgroup(Lc, seed * 7919 + i);
            alive.fetch_sub(1);
        });
    }
    for (auto& th : all) th.join();
    Lc.m.ctr_base += Lc.num_tiles;
}

}  // namespace

int main(int argc, char** argv)
{
    Params P;
    for (int i = 1; i < argc; ++i) {
        const char* a = argv[i];
        const char* eq = strchr(a, '=');
        if (!eq) continue;
        const std::string k(a, eq - a);
        const long long v = atoll(eq + 1);
        if (k == "nd") P.nd = (int)v;
        else if (k == "wait") P.wait = (int)v;
        else if (k == "slots") P.slots = (int)v;
        else if (k == "span") P.span = (int)v;
        else if (k == "first_piece") P.first_piece = (int)v;
        else if (k == "next_piece") P.next_piece = (int)v;
        else if (k == "wgs") P.wgs = (int)v;
        else if (k == "tiles") P.tiles = (int)v;
        else if (k == "share") P.share = (int)v;
        else if (k == "launches") P.launches = (int)v;
        else if (k == "op") P.op = (int)v;
        else if (k == "delay") P.delay = (int)v;
        else if (k == "max_pause_us") P.max_pause_us = (int)v;
        else if (k == "spin") P.spin = (uint64_t)v;
        else if (k == "lose_tile") P.lose_tile = (int)v;
        else if (k == "sticky") P.sticky = (int)v;
        else if (k == "epoch_start") P.epoch_start = (int)v;
        else if (k == "kernel") P.kernel = (int)v;
        else if (k == "resident") P.resident = (int)v;
        else if (k == "seed") P.seed = (unsigned)v;
    }
    if (P.nd < 1 || P.wait < 1 || P.slots < 1 || P.wgs < 2 || P.tiles < 1 || P.share < 1 || P.span < 1 || P.next_piece < 1) {
        fprintf(stderr, "bad parameters\n");
        return 2;
    }
    const uint32_t TE = tile_elems(P);
    const size_t n = (size_t)P.tiles * TE;
    Mem m((size_t)P.tiles * 2 + 2 * ((size_t)P.tiles / 64 + 1));
    m.epoch = (uint32_t)P.epoch_start - 1;
    std::mt19937 rng(P.seed);
    bool ok = true;
    uint64_t bad_total = 0;
    double max_ms = 0;
    for (int launch = 0; launch < P.launches; ++launch) {
        // next epoch; at the wrap every word could alias it: cleared
        if (++m.epoch >= kEpochLimit) {
            for (auto& wd : m.agg) wd.store(0);
            for (auto& wd : m.excl) wd.store(0);
            m.epoch = 1;
        }
        std::vector<Val> in(n), out(n, Val{0xDEADu, 0xBEEFu});
        for (auto& v : in) v = {(uint32_t)rng() | 1u, (uint32_t)rng()};
        if (P.op == 0)
            for (auto& v : in) v.a = 0;
        Launch Lc{P, m, in, out, (uint32_t)P.tiles};
        const auto t0 = std::chrono::steady_clock::now();
        if (P.kernel == 1) {
            run_one_tile_launch(Lc, P.seed * 1000 + launch);
        } else {
            std::vector<std::thread> wgs;
            for (int g = 0; g < P.wgs; ++g)
                wgs.emplace_back(workgroup, std::ref(Lc), (uint32_t)P.wgs, P.seed * 1000 + launch * 100 + g);
            for (auto& th : wgs) th.join();
        }
        const double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
        if (ms > max_ms) max_ms = ms;
        Val acc = identity(P.op);
        uint64_t bad = 0;
        for (size_t i = 0; i < n; ++i) {
            acc = combine(P.op, acc, in[i]);
            if (out[i].a != acc.a || out[i].b != acc.b) ++bad;
        }
        bad_total += bad;
        if (P.lose_tile < 0 && (bad || m.err.load())) ok = false;
        if (Lc.stale_prefix.load() || Lc.stale_total.load() || Lc.stale_wave_prefix.load()) {
            fprintf(stderr, "launch %d: stale slot reads: prefix %llu, tile total %llu, wave prefix %llu\n", launch,
                    (unsigned long long)Lc.stale_prefix.load(), (unsigned long long)Lc.stale_total.load(),
                    (unsigned long long)Lc.stale_wave_prefix.load());
            ok = false;
        }
        if (m.tile_ctr.load() || m.role_ctr.load() || m.retired.load()) {
            fprintf(stderr, "counters not reset after launch %d\n", launch);
            ok = false;
        }
        if (P.lose_tile >= 0) break;  // one launch is enough to see how it ends
    }
    const uint32_t err = m.err.load();
    if (P.lose_tile >= 0) ok = (err & kErrTimeout) != 0;
    printf("result ok=%d err=%u mismatches=%llu launches=%d max_launch_ms=%.1f full_budgets=%llu\n", ok ? 1 : 0, err,
           (unsigned long long)bad_total, P.launches, max_ms, (unsigned long long)m.full_budgets.load());
    return ok ? 0 : 1;
}
