// scan_api.hip -- C ABI of libdwpt_scan.so: argument checks, the
// (op, dtype, variant) dispatch table, workspace management and launches.
// The kernels are in tile_scan.hpp, reduce_then_scan.hpp and
// csr_offsets.hpp; the ABI is documented in dwpt_scan.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <type_traits>
#include <utility>

#include "csr_offsets.hpp"
#include "dwpt_scan.h"
#include "radix_split.hpp"
#include "reduce_then_scan.hpp"
#include "tile_scan.hpp"

using namespace dwpt;

namespace {

// ------------------------------------------------------------ tile shapes
// Workgroup size, elements per lane and pipeline depth per class of scan
// (defaults: 1024 threads = 15 data wavefronts + 1 prefix wavefront; (maximum,
// count) pairs and 2x2 and 3x3 matrices take 512, whose 8 wavefronts may use
// 256 registers per lane).  ITEMS sets the tile ((BLOCK / 64 - 1) * 64 * ITEMS
// elements); WAIT is the number of tiles per data wavefront that wait on
// their prefix in the persistent kernel.  Each class takes the measured best
// shape: (maximum, count) at 2^27 436 us with 1024 threads x 6 per lane, WAIT
// 3, 365 us with 512 x 16, WAIT 4 (512 x 12/20 at WAIT 3-4: 367-399), and
// since its one-pass scan after the wait 346.4 us with 512 x 16, WAIT 3
// (WAIT 4 348.7, 20/3 350.0, 12/5 395.4; A/B on one machine); 2x2 matrices at 2^26
// 474 -> 413 us with 512 x 8, WAIT 4 (512 x 6 or 12: 469 and more; at 2^25
// with the one-pass scan 8/4 208.7, 10/3 208.5, 8/3 225.0, 6/5 230.5);
// affine and segmented scans were slower at 512 threads (affine 354 against
// 347, segmented 248 against 214 at their best 512 shapes).  The 3x3
// matrices still spill at their fastest measured shape.
// Build-time switches, so that shapes can be compared by measurement.
#ifndef DWPT_BLOCK
#define DWPT_BLOCK 1024
#endif
#ifndef DWPT_ITEMS4            // plain scans of 4-byte values
#define DWPT_ITEMS4 16
#endif
#ifndef DWPT_WAIT4
#define DWPT_WAIT4 3
#endif
#ifndef DWPT_ITEMS8            // 8-byte values (affine pairs)
#define DWPT_ITEMS8 8
#endif
#ifndef DWPT_WAIT8
#define DWPT_WAIT8 3
#endif
#ifndef DWPT_BLOCK_MC          // (max, count) pairs: 512 threads, so up to 256 registers per lane
#define DWPT_BLOCK_MC 512
#endif
#ifndef DWPT_ITEMS_MC
#define DWPT_ITEMS_MC 16
#endif
#ifndef DWPT_WAIT_MC
#define DWPT_WAIT_MC 3
#endif
#ifndef DWPT_ITEMS16           // 16-byte values (2x2 matrices)
#define DWPT_ITEMS16 8
#endif
#ifndef DWPT_WAIT16
#define DWPT_WAIT16 4
#endif
#ifndef DWPT_BLOCK16
#define DWPT_BLOCK16 512
#endif
#ifndef DWPT_BLOCK36           // 36-byte values (3x3 matrices): 512 threads, so 256 registers per lane
#define DWPT_BLOCK36 512
#endif
#ifndef DWPT_ITEMS36
#define DWPT_ITEMS36 8
#endif
#ifndef DWPT_WAIT36
#define DWPT_WAIT36 1
#endif
#ifndef DWPT_ITEMS_SEG         // segmented scans (value + head flag)
#define DWPT_ITEMS_SEG 16
#endif
#ifndef DWPT_WAIT_SEG
#define DWPT_WAIT_SEG 2
#endif
#ifndef DWPT_ITEMS_COMPACT     // stream compaction
#define DWPT_ITEMS_COMPACT 20
#endif
#ifndef DWPT_WAIT_COMPACT
#define DWPT_WAIT_COMPACT 3
#endif
template <class Op>
struct Shape {
    static constexpr bool SEG = IsSeg<Op>::value, WIDE = sizeof(typename Op::elem_t) == 8,
                          WIDE16 = sizeof(typename Op::elem_t) == 16, WIDE36 = sizeof(typename Op::elem_t) == 36;
    static constexpr bool MC = std::is_same<Op, OpMaxCount>::value;
    static constexpr int BLOCK = MC ? DWPT_BLOCK_MC : WIDE36 ? DWPT_BLOCK36 : WIDE16 ? DWPT_BLOCK16 : DWPT_BLOCK;
    static constexpr int ITEMS = SEG      ? DWPT_ITEMS_SEG
                                 : MC     ? DWPT_ITEMS_MC
                                 : WIDE36 ? DWPT_ITEMS36
                                 : WIDE16 ? DWPT_ITEMS16
                                 : WIDE   ? DWPT_ITEMS8
                                          : DWPT_ITEMS4;
    static constexpr int TILE = Geometry<Op, BLOCK, ITEMS>::TILE;
    static constexpr int WAIT = SEG      ? DWPT_WAIT_SEG
                                : MC     ? DWPT_WAIT_MC
                                : WIDE36 ? DWPT_WAIT36
                                : WIDE16 ? DWPT_WAIT16
                                : WIDE   ? DWPT_WAIT8
                                         : DWPT_WAIT4;
};

// ------------------------------------------------------------ settings
std::mutex g_mu;
// n at or below: single-workgroup path.  SCAN_SMALL_N_AUTO: one tile of the
// operator's shape -- measured crossover for int32 exclusive add (one
// workgroup against one workgroup per tile, back to back): 3.8 against 4.5 us
// at 2^12 and 2^13, 5.1 against 4.6 at 2^14 (two tiles).
size_t g_small_n_max = SCAN_SMALL_N_AUTO;
uint32_t g_spin_limit = 1u << 18;     // look-back polls before giving up (a fraction of a second)
int g_multi_mode = 0;  // 0: by size; 1: one tile per workgroup; 2: persistent kernel; 3: reduce-then-scan
// In the automatic mode the persistent kernel takes inputs of at least this
// many tiles per resident data workgroup; below, too few tiles per workgroup
// are left to fill its pipeline and one workgroup per tile is faster
// (measured on int32 max scans: 26 against 30 us at 2^23 elements, 41
// against 36 us at 2^24).
constexpr uint64_t kPersistentTilesPerWorkgroup = 3;

// ------------------------------------------------------------ workspaces
struct Workspace {
    void* mem = nullptr;
    size_t status_words = 0;  // capacity in 64-bit status words
    uint64_t* status = nullptr;
    uint32_t* ctr = nullptr;
    uint32_t* pipe_ctr = nullptr;  // persistent kernel's self-resetting counters (one 128-byte line each)
    uint32_t* err = nullptr;
    uint32_t* abort = nullptr;     // epoch of the last launch that gave up a wait (its own line)
    uint32_t ctr_base = 0;
    uint32_t epoch = 0;
    // reduce-then-scan's plain carries, in memory of their own: status words
    // must only ever hold tagged entries, or a stale carry could pass for a
    // current one
    void* rts = nullptr;
    size_t rts_bytes = 0;
    // radix passes' digit histograms: scanned in place by the library's own
    // scan, so kept apart from both buffers above
    void* hist = nullptr;
    size_t hist_bytes = 0;
};
std::map<std::pair<int, void*>, Workspace> g_ws;
// line 0: err word, tile counter; lines 1-3: persistent-kernel counters; line 4: abort word
constexpr size_t kHeaderBytes = 640;

__global__ void zero_words_kernel(uint64_t* p, size_t nwords)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < nwords;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

hipError_t zero_async(void* p, size_t bytes, hipStream_t s)
{
    const size_t nwords = bytes / 8;
    unsigned grid = (unsigned)((nwords + 255) / 256);
    if (grid > 1024) grid = 1024;
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, s, static_cast<uint64_t*>(p), nwords);
    return hipGetLastError();
}

// Header words and status array of a workspace whose memory starts at mem.
void lay_out(Workspace& ws, void* mem, size_t status_words)
{
    ws.mem = mem;
    ws.status_words = status_words;
    ws.err = static_cast<uint32_t*>(mem);
    ws.ctr = static_cast<uint32_t*>(mem) + 1;
    ws.pipe_ctr = reinterpret_cast<uint32_t*>(static_cast<char*>(mem) + 128);
    ws.abort = reinterpret_cast<uint32_t*>(static_cast<char*>(mem) + 512);
    ws.status = reinterpret_cast<uint64_t*>(static_cast<char*>(mem) + kHeaderBytes);
    ws.ctr_base = 0;
    ws.epoch = 0;
}

// Called with g_mu held: the next call's epoch.  At the wrap every tag of the
// array (and the abort word) could alias the new epoch: they are cleared.
scan_status_t next_epoch(Workspace& ws, hipStream_t s)
{
    ws.epoch += 1;
    if (ws.epoch >= (1u << kEpochBits)) {
        if (zero_async(ws.status, ws.status_words * 8, s) != hipSuccess) return SCAN_ERR_HIP;
        if (zero_async(ws.abort, 128, s) != hipSuccess) return SCAN_ERR_HIP;
        ws.epoch = 1;
    }
    return SCAN_OK;
}

// ------------------------------------------------------------ static scratch
// Device memory of the allocation-free entry point (scan_noalloc): the same
// header and status words as a stream workspace, in a static array that each
// GPU the library runs on holds until the process ends.  In host code the
// array's name is not a device address: each device's address comes from
// hipGetSymbolAddress, once, at that device's first call (with the device
// current), and is kept in g_static; kernels receive that address.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr size_t kScratchStatusWords = (kScratchBytes - kHeaderBytes) / 8;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
struct StaticScratch {
    bool ready = false;
    Workspace ws;
};
StaticScratch g_static[kMaxDevices];

// Called with g_mu held: the current device's scratch (set up and cleared on
// its first call, with a fill kernel on the call's stream), epoch advanced.
scan_status_t static_workspace(hipStream_t s, Workspace** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SCAN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SCAN_ERR_UNSUPPORTED;
    StaticScratch& st = g_static[dev];
    if (!st.ready) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return SCAN_ERR_HIP;
        }
        if (zero_async(ptr, kScratchBytes, s) != hipSuccess) return SCAN_ERR_HIP;
        lay_out(st.ws, ptr, kScratchStatusWords);
        st.ready = true;
    }
    const scan_status_t e = next_epoch(st.ws, s);
    if (e != SCAN_OK) return e;
    *out = &st.ws;
    return SCAN_OK;
}

// Called with g_mu held.  Makes sure the (device, stream) workspace holds at
// least `words` status words and advances its epoch for a new call.
scan_status_t acquire_workspace(hipStream_t s, size_t words, Workspace** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SCAN_ERR_HIP;
    Workspace& ws = g_ws[std::make_pair(dev, (void*)s)];
    if (ws.status_words < words) {
        size_t cap = ws.status_words ? ws.status_words * 2 : (size_t)1 << 16;
        while (cap < words) cap *= 2;
        if (ws.mem) {
            if (hipStreamSynchronize(s) != hipSuccess) return SCAN_ERR_HIP;
            (void)hipFree(ws.mem);
            ws.mem = nullptr;
            ws.status_words = 0;
        }
        void* mem = nullptr;
        const size_t bytes = kHeaderBytes + cap * 8;
        if (hipMalloc(&mem, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return SCAN_ERR_NOMEM;
        }
        if (zero_async(mem, bytes, s) != hipSuccess) {
            (void)hipFree(mem);
            return SCAN_ERR_HIP;
        }
        lay_out(ws, mem, cap);
    }
    const scan_status_t e = next_epoch(ws, s);
    if (e != SCAN_OK) return e;
    *out = &ws;
    return SCAN_OK;
}

// Grows the plain device buffer *p (capacity *have bytes) to at least
// `bytes`, after the stream has finished with the old one.
scan_status_t grow_buffer(hipStream_t s, void** p, size_t* have, size_t bytes)
{
    if (*have >= bytes) return SCAN_OK;
    size_t cap = *have ? *have * 2 : (size_t)1 << 16;
    while (cap < bytes) cap *= 2;
    if (*p) {
        if (hipStreamSynchronize(s) != hipSuccess) return SCAN_ERR_HIP;
        (void)hipFree(*p);
        *p = nullptr;
        *have = 0;
    }
    if (hipMalloc(p, cap) != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        return SCAN_ERR_NOMEM;
    }
    *have = cap;
    return SCAN_OK;
}

// Called with g_mu held, after acquire_workspace: at least `bytes` of
// reduce-then-scan memory in the workspace.
scan_status_t acquire_rts(hipStream_t s, Workspace& ws, size_t bytes)
{
    return grow_buffer(s, &ws.rts, &ws.rts_bytes, bytes);
}

// Called with g_mu held: at least `bytes` of histogram memory in the
// (device, stream) workspace.
scan_status_t acquire_hist(hipStream_t s, size_t bytes, void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SCAN_ERR_HIP;
    Workspace& ws = g_ws[std::make_pair(dev, (void*)s)];
    const scan_status_t st = grow_buffer(s, &ws.hist, &ws.hist_bytes, bytes);
    *out = ws.hist;
    return st;
}

// ------------------------------------------------------------ launches
struct Call {
    const void* in;
    void* out;
    const uint8_t* heads;
    uint32_t* count;
    size_t n;
    hipStream_t stream;
    bool noalloc = false;  // status words in the static scratch; nothing allocated
};

bool is_aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Compute units of the current device (cached in a fixed table, so that no
// call allocates host memory either; called with g_mu held).
int device_cus()
{
    static int cache[kMaxDevices];  // 0: not asked yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (dev >= 0 && dev < kMaxDevices && cache[dev] > 0) return cache[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        cus = 1;
    }
    if (dev >= 0 && dev < kMaxDevices) cache[dev] = cus;
    return cus;
}

// Resident workgroups of kernel `f` on the current device (cached in a fixed
// open-addressing table keyed by device and kernel; called with g_mu held).
int resident_capacity(const void* f, int block)
{
    struct Entry {
        const void* f;
        int dev;
        int cap;
    };
    constexpr int kEntries = 1024;
    static Entry cache[kEntries];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const size_t h = ((uintptr_t)f >> 4) * 31u + (size_t)dev;
    int slot = -1;
    for (int i = 0; i < kEntries; ++i) {
        Entry& e = cache[(h + i) % kEntries];
        if (e.f == f && e.dev == dev) return e.cap;
        if (e.f == nullptr) {
            slot = (int)((h + i) % kEntries);
            break;
        }
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, block, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        per_cu = 0;
    }
    const int cap = per_cu * cus;
    if (slot >= 0) cache[slot] = Entry{f, dev, cap};
    return cap;
}

// The three kernels of the reduce-then-scan variant, for carries of type C.
template <class C>
struct RtsKernels {
    void (*reduce)(ScanParams, C*);
    void (*carries)(const C*, C*, uint32_t, C*);
    void (*seeded)(ScanParams, const C*);
};

// Fills params and launches the single-workgroup kernel (small n), else the
// persistent pipelined kernel (as many workgroups as fit, plus none beyond
// one per tile and the resolver), the one-tile-per-workgroup kernel or the
// three reduce-then-scan kernels, as the mode and the number of tiles
// select.  TILE is the tile size and kWords the status words per tile;
// `grand` receives the fold of all tiles in reduce-then-scan (compaction's
// count), or nullptr.  rts_ok == false makes reduce-then-scan mode take the
// single-pass kernels instead (in-place compaction: its last pass writes a
// tile's kept elements below the tile, where earlier tiles of the same launch
// may not have read theirs yet).
template <int BLOCK, int TILE, int kWords, class C>
scan_status_t launch(void (*ks)(ScanParams), void (*km)(ScanParams), void (*kp)(ScanParams),
                     const RtsKernels<C>& rts, C* grand, const Call& c, bool vec_ok, bool rts_ok = true)
{
    ScanParams p{};
    p.in = c.in;
    p.out = c.out;
    p.heads = c.heads;
    p.count = c.count;
    p.n = c.n;
    const uint64_t tiles = (c.n + TILE - 1) / TILE;
    if (tiles > 0xFFFFFFFFull) return SCAN_ERR_INVALID;
    p.num_tiles = (uint32_t)tiles;
    p.vec_ok = vec_ok ? 1 : 0;
    // per tile: its status (AGG_PAD entries apart), then a second array for group statuses
    // (one-tile-per-workgroup kernel) or the resolver's published prefixes (persistent
    // kernel, PREFIX_PAD entries apart: one prefix per 128-byte line)
    const size_t words = (size_t)tiles * kWords * (DWPT_AGG_PAD + DWPT_PREFIX_PAD);
    if (c.noalloc && words > kScratchStatusWords) return SCAN_ERR_INVALID;  // beyond the static scratch

    std::lock_guard<std::mutex> lock(g_mu);
    if (c.n <= (g_small_n_max == SCAN_SMALL_N_AUTO ? (size_t)TILE : g_small_n_max)) {
        hipLaunchKernelGGL(ks, dim3(1), dim3(BLOCK), 0, c.stream, p);
        return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
    }
    Workspace* ws = nullptr;
    const scan_status_t st = c.noalloc ? static_workspace(c.stream, &ws) : acquire_workspace(c.stream, words, &ws);
    if (st != SCAN_OK) return st;
    // reduce-then-scan needs a carry buffer: not on the allocation-free path
    if (g_multi_mode == 3 && rts_ok && !c.noalloc) {
        // 2T + 1 plain carries: the tile totals, the grand total, the prefixes
        const scan_status_t sr = acquire_rts(c.stream, *ws, (2 * (size_t)tiles + 1) * sizeof(C));
        if (sr != SCAN_OK) return sr;
        C* totals = static_cast<C*>(ws->rts);
        C* excl = totals + tiles + 1;
        const uint32_t T = (uint32_t)tiles;
        hipLaunchKernelGGL(rts.reduce, dim3(T), dim3(BLOCK), 0, c.stream, p, totals);
        hipLaunchKernelGGL(rts.carries, dim3(1), dim3(BLOCK), 0, c.stream, (const C*)totals, excl, T,
                           grand ? grand : totals + tiles);
        hipLaunchKernelGGL(rts.seeded, dim3(T), dim3(BLOCK), 0, c.stream, p, (const C*)excl);
        return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
    }
    p.tile_ctr = ws->ctr;
    p.ctr_base = ws->ctr_base;
    p.pipe_ctr = ws->pipe_ctr;
    p.lb.status = ws->status;
    p.lb.groups = ws->status + (size_t)tiles * kWords * DWPT_AGG_PAD;
    p.lb.err = ws->err;
    p.lb.abort = ws->abort;
    p.lb.epoch = ws->epoch;
    p.lb.spin_limit = g_spin_limit;
    if (g_multi_mode != 1) {
        const int cap = resident_capacity((const void*)kp, BLOCK);
        const bool big = tiles >= kPersistentTilesPerWorkgroup * (uint64_t)(cap > 1 ? cap - 1 : 1);
        if (cap > 1 && (g_multi_mode == 2 || big)) {
            // the first workgroup to start resolves prefixes; the others scan tiles
            const unsigned grid = 1u + (unsigned)std::min<uint64_t>((uint64_t)cap - 1, tiles);
            hipLaunchKernelGGL(kp, dim3(grid), dim3(BLOCK), 0, c.stream, p);
            return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
        }
    }
    hipLaunchKernelGGL(km, dim3(p.num_tiles), dim3(BLOCK), 0, c.stream, p);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    ws->ctr_base += p.num_tiles;  // every workgroup takes exactly one tile number
    return SCAN_OK;
}

template <class Op, bool EXCL>
scan_status_t run_scan(const Call& c, bool vec_ok)
{
    using S = Shape<Op>;
    using C = typename Op::carry_t;
    const RtsKernels<C> rts{tile_reduce_kernel<Op, S::BLOCK, S::ITEMS>, carry_scan_kernel<Op, S::BLOCK>,
                            tile_scan_seeded_kernel<Op, EXCL, S::BLOCK, S::ITEMS>};
    return launch<S::BLOCK, S::TILE, Op::kWords, C>(tile_scan_kernel<Op, EXCL, S::BLOCK, S::ITEMS, true>,
                                                    tile_scan_kernel<Op, EXCL, S::BLOCK, S::ITEMS, false>,
                                                    tile_scan_persistent<Op, EXCL, S::BLOCK, S::ITEMS, S::WAIT>, rts,
                                                    (C*)nullptr, c, vec_ok);
}

template <typename T>
scan_status_t run_compact(const Call& c, bool vec_ok)
{
    constexpr int BLOCK = DWPT_BLOCK, ITEMS = DWPT_ITEMS_COMPACT;
    const RtsKernels<uint32_t> rts{tile_count_kernel<T, BLOCK, ITEMS>, carry_scan_kernel<OpAdd<uint32_t>, BLOCK>,
                                   compact_seeded_kernel<T, BLOCK, ITEMS>};
    return launch<BLOCK, Geometry<OpAdd<uint32_t>, BLOCK, ITEMS>::TILE, 1, uint32_t>(
        compact_kernel<T, BLOCK, ITEMS, true>, compact_kernel<T, BLOCK, ITEMS, false>,
        compact_persistent<T, BLOCK, ITEMS, DWPT_WAIT_COMPACT>, rts, c.count, c, vec_ok, c.in != (const void*)c.out);
}

typedef scan_status_t (*Runner)(const Call&, bool);

// Dispatch tables: [op][dtype] for plain scans (inclusive, exclusive) and
// segmented scans (inclusive, exclusive); nullptr = unsupported.
template <bool EXCL>
Runner plain_runner(int op, int dt)
{
    static const Runner table[3][3] = {
        {run_scan<OpAdd<int32_t>, EXCL>, run_scan<OpAdd<uint32_t>, EXCL>, run_scan<OpAdd<float>, EXCL>},
        {run_scan<OpMax<int32_t>, EXCL>, run_scan<OpMax<uint32_t>, EXCL>, run_scan<OpMax<float>, EXCL>},
        {run_scan<OpMin<int32_t>, EXCL>, run_scan<OpMin<uint32_t>, EXCL>, run_scan<OpMin<float>, EXCL>},
    };
    if (op <= SCAN_OP_MIN && dt <= SCAN_F32) return table[op][dt];
    if (op == SCAN_OP_AFFINE && dt == SCAN_U32X2) return run_scan<OpAffine, EXCL>;
    if (op == SCAN_OP_MAX_COUNT && dt == SCAN_I32_U32) return run_scan<OpMaxCount, EXCL>;
    if (op == SCAN_OP_MAT2 && dt == SCAN_U32X4) return run_scan<OpMat2, EXCL>;
    if (op == SCAN_OP_MAT3 && dt == SCAN_U32X9) return run_scan<OpMat3, EXCL>;
    if (op == SCAN_OP_AND && dt == SCAN_I32) return run_scan<OpAnd<int32_t>, EXCL>;
    if (op == SCAN_OP_AND && dt == SCAN_U32) return run_scan<OpAnd<uint32_t>, EXCL>;
    if (op == SCAN_OP_OR && dt == SCAN_I32) return run_scan<OpOr<int32_t>, EXCL>;
    if (op == SCAN_OP_OR && dt == SCAN_U32) return run_scan<OpOr<uint32_t>, EXCL>;
    return nullptr;
}

template <bool EXCL>
Runner seg_runner(int op, int dt)
{
    static const Runner table[3][3] = {
        {run_scan<OpSeg<OpAdd<int32_t>>, EXCL>, run_scan<OpSeg<OpAdd<uint32_t>>, EXCL>,
         run_scan<OpSeg<OpAdd<float>>, EXCL>},
        {run_scan<OpSeg<OpMax<int32_t>>, EXCL>, run_scan<OpSeg<OpMax<uint32_t>>, EXCL>,
         run_scan<OpSeg<OpMax<float>>, EXCL>},
        {run_scan<OpSeg<OpMin<int32_t>>, EXCL>, run_scan<OpSeg<OpMin<uint32_t>>, EXCL>,
         run_scan<OpSeg<OpMin<float>>, EXCL>},
    };
    return table[op][dt];
}

// Element size in bytes.
size_t elem_size(int dt)
{
    switch (dt) {
        case SCAN_U32X2:
        case SCAN_I32_U32: return 8;
        case SCAN_U32X4: return 16;
        case SCAN_U32X9: return 36;
        default: return 4;
    }
}

// Alignment an array of the type needs: its size, except 4 bytes for the
// 36-byte matrices (arrays of uint32).
size_t elem_align(int dt) { return dt == SCAN_U32X9 ? 4 : elem_size(dt); }

bool ranges_partially_overlap(const void* a, const void* b, size_t bytes_a, size_t bytes_b)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    if (a0 == b0) return false;
    return a0 < b0 + bytes_b && b0 < a0 + bytes_a;
}

scan_status_t plain_scan(bool excl, scan_op_t op, scan_dtype_t dt, const void* in, void* out, size_t n,
                         void* stream, bool noalloc = false)
{
    if ((unsigned)op > SCAN_OP_OR || (unsigned)dt > SCAN_U32X9) return SCAN_ERR_UNSUPPORTED;
    const Runner r = excl ? plain_runner<true>(op, dt) : plain_runner<false>(op, dt);
    if (!r) return SCAN_ERR_UNSUPPORTED;
    if (n == 0) return SCAN_OK;
    const size_t es = elem_size(dt);
    if (!in || !out) return SCAN_ERR_INVALID;
    if (!is_aligned(in, elem_align(dt)) || !is_aligned(out, elem_align(dt))) return SCAN_ERR_INVALID;
    if (n > ((size_t)1 << 40)) return SCAN_ERR_INVALID;
    if (ranges_partially_overlap(in, out, n * es, n * es)) return SCAN_ERR_INVALID;
    const Call c{in, out, nullptr, nullptr, n, static_cast<hipStream_t>(stream), noalloc};
    return r(c, is_aligned(in, 16) && is_aligned(out, 16));
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

scan_status_t scan_inclusive(scan_op_t op, scan_dtype_t dtype, const void* in, void* out, size_t n,
                             void* stream)
{
    try {
        return plain_scan(false, op, dtype, in, out, n, stream);
    } catch (const std::bad_alloc&) {
        return SCAN_ERR_NOMEM;
    }
}

scan_status_t scan_exclusive(scan_op_t op, scan_dtype_t dtype, const void* in, void* out, size_t n,
                             void* stream)
{
    try {
        return plain_scan(true, op, dtype, in, out, n, stream);
    } catch (const std::bad_alloc&) {
        return SCAN_ERR_NOMEM;
    }
}

scan_status_t scan_noalloc(scan_op_t op, scan_dtype_t dtype, const void* in, void* out, size_t n, int exclusive,
                          void* stream)
{
    try {
        return plain_scan(exclusive != 0, op, dtype, in, out, n, stream, true);
    } catch (const std::bad_alloc&) {
        return SCAN_ERR_NOMEM;
    }
}

scan_status_t segmented_scan(scan_op_t op, scan_dtype_t dtype, const void* in, const uint8_t* head_flags,
                             void* out, size_t n, int exclusive, void* stream)
{
    try {
        if ((unsigned)op > SCAN_OP_MIN || (unsigned)dtype > SCAN_F32) return SCAN_ERR_UNSUPPORTED;
        const Runner r = exclusive ? seg_runner<true>(op, dtype) : seg_runner<false>(op, dtype);
        if (n == 0) return SCAN_OK;
        if (!in || !out || !head_flags) return SCAN_ERR_INVALID;
        if (!is_aligned(in, 4) || !is_aligned(out, 4)) return SCAN_ERR_INVALID;
        if (n > ((size_t)1 << 40)) return SCAN_ERR_INVALID;
        if (ranges_partially_overlap(in, out, n * 4, n * 4)) return SCAN_ERR_INVALID;
        if (ranges_partially_overlap(head_flags, out, n, n * 4) || (const void*)head_flags == out)
            return SCAN_ERR_INVALID;
        const Call c{in, out, head_flags, nullptr, n, static_cast<hipStream_t>(stream)};
        return r(c, is_aligned(in, 16) && is_aligned(out, 16) && is_aligned(head_flags, 4));
    } catch (const std::bad_alloc&) {
        return SCAN_ERR_NOMEM;
    }
}

scan_status_t csr_row_offsets(const uint32_t* row_idx, size_t nnz, uint32_t n_rows, uint32_t* row_ptr,
                              void* stream)
{
    try {
        const size_t np = (size_t)n_rows + 1;
        if (!row_ptr || !is_aligned(row_ptr, 4)) return SCAN_ERR_INVALID;
        if (nnz > 0 && (!row_idx || !is_aligned(row_idx, 4))) return SCAN_ERR_INVALID;
        if (nnz >= ((size_t)1 << 32)) return SCAN_ERR_INVALID;  // offsets are uint32
        if (nnz > 0) {
            const uintptr_t a = (uintptr_t)row_idx, b = (uintptr_t)row_ptr;
            if (a < b + np * 4 && b < a + nnz * 4) return SCAN_ERR_INVALID;  // any overlap
        }
        const hipStream_t s = static_cast<hipStream_t>(stream);
        // counts of every row into row_ptr[0 .. n_rows), row_ptr[n_rows] = 0
        const unsigned zgrid = (unsigned)std::min<size_t>((np + kCsrBlock - 1) / kCsrBlock, 4096);
        hipLaunchKernelGGL(zero_u32_kernel, dim3(zgrid), dim3(kCsrBlock), 0, s, row_ptr, (uint64_t)np);
        if (nnz > 0) {
            const size_t chunks = (nnz + 64 * kCsrSteps - 1) / (64 * kCsrSteps);  // one per wavefront
            int cus = 1;
            {
                std::lock_guard<std::mutex> lock(g_mu);
                cus = device_cus();
            }
            if (n_rows <= kCsrSmallBins && is_aligned(row_idx, 16)) {
                // one workgroup per CU, every index counted in LDS
                const size_t c4 = (nnz / 4 + kCsrLdsBlock - 1) / kCsrLdsBlock;
                const unsigned grid = (unsigned)std::max<size_t>(1, std::min<size_t>(c4, (size_t)cus));
                hipLaunchKernelGGL(csr_count_small_kernel, dim3(grid), dim3(kCsrLdsBlock),
                                   (size_t)kCsrCopies * (n_rows + 1) * 4, s, row_idx, (uint64_t)nnz, n_rows, row_ptr);
            } else if (n_rows <= kCsrLdsBins) {
                // at most one workgroup per CU: each adds its n_rows counts to memory once
                const unsigned grid = (unsigned)std::min<size_t>((chunks + kCsrLdsBlock / 64 - 1) / (kCsrLdsBlock / 64),
                                                                 (size_t)cus);
                hipLaunchKernelGGL(csr_count_lds_kernel, dim3(grid), dim3(kCsrLdsBlock), (size_t)n_rows * 4, s,
                                   row_idx, (uint64_t)nnz, n_rows, row_ptr);
            } else {
                const unsigned grid =
                    (unsigned)std::min<size_t>((chunks + kCsrBlock / 64 - 1) / (kCsrBlock / 64), 4096);
                hipLaunchKernelGGL(csr_count_kernel, dim3(grid), dim3(kCsrBlock), 0, s, row_idx, (uint64_t)nnz,
                                   n_rows, row_ptr);
            }
        }
        if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
        // row_ptr = exclusive scan of the counts, in place
        const Call c{row_ptr, row_ptr, nullptr, nullptr, np, s};
        return run_scan<OpAdd<uint32_t>, true>(c, is_aligned(row_ptr, 16));
    } catch (const std::bad_alloc&) {
        return SCAN_ERR_NOMEM;
    }
}

scan_status_t radix_split(const uint32_t* keys, const uint32_t* vals, size_t n, uint32_t shift,
                          uint32_t* keys_out, uint32_t* vals_out, void* stream)
{
    try {
        if (shift > 31) return SCAN_ERR_INVALID;
        if (n == 0) return SCAN_OK;
        if ((vals == nullptr) != (vals_out == nullptr)) return SCAN_ERR_INVALID;
        if (n >= ((size_t)1 << 32)) return SCAN_ERR_INVALID;  // positions are uint32
        if (!keys || !keys_out || !is_aligned(keys, 4) || !is_aligned(keys_out, 4)) return SCAN_ERR_INVALID;
        if (vals && (!is_aligned(vals, 4) || !is_aligned(vals_out, 4))) return SCAN_ERR_INVALID;
        const size_t b = n * 4;
        const auto overlap = [b](const void* x, const void* y) {
            return x && y && (uintptr_t)x < (uintptr_t)y + b && (uintptr_t)y < (uintptr_t)x + b;
        };
        // outputs are written while other tiles still read the inputs
        if (overlap(keys_out, keys) || overlap(keys_out, vals) || overlap(keys_out, vals_out) ||
            overlap(vals_out, keys) || overlap(vals_out, vals))
            return SCAN_ERR_INVALID;
        const hipStream_t s = static_cast<hipStream_t>(stream);
        const uint32_t T = (uint32_t)((n + kRsTile - 1) / kRsTile);
        const uint32_t G = (T + kHistTiles - 1) / kHistTiles;
        // per (digit, tile): count in the earlier tiles of the tile's group;
        // then per (digit, group): the group's count
        const size_t nl = (size_t)kRsDigits * T, ng = (size_t)kRsDigits * G;
        void* hist = nullptr;
        {
            std::lock_guard<std::mutex> lock(g_mu);
            const scan_status_t st = acquire_hist(s, (nl + ng) * 4, &hist);
            if (st != SCAN_OK) return st;
        }
        uint32_t* local = static_cast<uint32_t*>(hist);
        uint32_t* group = local + nl;
        hipLaunchKernelGGL(radix_hist_kernel, dim3(G), dim3(kRsBlock), 0,
                           s, keys, (uint64_t)n, shift, T, local, group, is_aligned(keys, 16) ? 1 : 0);
        if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
        // each (digit, group) count -> the output position of the group's first key of the digit
        const Call c{group, group, nullptr, nullptr, ng, s};
        const scan_status_t st = run_scan<OpAdd<uint32_t>, true>(c, true);
        if (st != SCAN_OK) return st;
        if (vals)
            hipLaunchKernelGGL(radix_scatter_kernel<true>,
                               dim3(T), dim3(kRsBlock), 0, s,
                               keys, vals, (uint64_t)n, shift, T, (const uint32_t*)local, (const uint32_t*)group,
                               keys_out, vals_out);
        else
            hipLaunchKernelGGL(radix_scatter_kernel<false>,
                               dim3(T), dim3(kRsBlock), 0, s,
                               keys, vals, (uint64_t)n, shift, T, (const uint32_t*)local, (const uint32_t*)group,
                               keys_out, vals_out);
        return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
    } catch (const std::bad_alloc&) {
        return SCAN_ERR_NOMEM;
    }
}

scan_status_t compact(scan_dtype_t dtype, const void* in, void* out, uint32_t* d_count, size_t n, void* stream)
{
    try {
        if ((unsigned)dtype > SCAN_F32) return SCAN_ERR_UNSUPPORTED;
        if (!d_count || !is_aligned(d_count, 4)) return SCAN_ERR_INVALID;
        // n == 0 still launches one single-workgroup pass so that *d_count becomes 0
        if (n > 0 && (!in || !out)) return SCAN_ERR_INVALID;
        if (n > 0 && (!is_aligned(in, 4) || !is_aligned(out, 4))) return SCAN_ERR_INVALID;
        if (n >= ((size_t)1 << 32)) return SCAN_ERR_INVALID;
        if (n > 0 && ranges_partially_overlap(in, out, n * 4, n * 4)) return SCAN_ERR_INVALID;
        if (ranges_partially_overlap(d_count, out, 4, n * 4) || (void*)d_count == out) return SCAN_ERR_INVALID;
        if (n > 0 && (ranges_partially_overlap(d_count, in, 4, n * 4) || (const void*)d_count == in))
            return SCAN_ERR_INVALID;
        const Call c{in, out, nullptr, d_count, n, static_cast<hipStream_t>(stream)};
        const bool vec_ok = is_aligned(in, 16);
        switch (dtype) {
            case SCAN_I32: return run_compact<int32_t>(c, vec_ok);
            case SCAN_U32: return run_compact<uint32_t>(c, vec_ok);
            case SCAN_F32: return run_compact<float>(c, vec_ok);
            default: return SCAN_ERR_UNSUPPORTED;
        }
    } catch (const std::bad_alloc&) {
        return SCAN_ERR_NOMEM;
    }
}

const char* scan_status_string(scan_status_t s)
{
    switch (s) {
        case SCAN_OK: return "ok";
        case SCAN_ERR_INVALID: return "invalid argument";
        case SCAN_ERR_UNSUPPORTED: return "unsupported op/dtype combination";
        case SCAN_ERR_NOMEM: return "out of device memory for the workspace";
        case SCAN_ERR_HIP: return "HIP runtime error";
        case SCAN_ERR_TIMEOUT: return "look-back wait timed out on the device";
    }
    return "unknown status";
}

scan_status_t scan_get_device_error(void* stream)
{
    try {
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if (hipStreamSynchronize(s) != hipSuccess) return SCAN_ERR_HIP;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return SCAN_ERR_HIP;
        std::lock_guard<std::mutex> lock(g_mu);
        // the stream's workspace and the device's static scratch (scan_noalloc calls)
        uint32_t* words[2] = {nullptr, nullptr};
        auto it = g_ws.find(std::make_pair(dev, (void*)s));
        if (it != g_ws.end() && it->second.mem) words[0] = it->second.err;
        if (dev >= 0 && dev < kMaxDevices && g_static[dev].ready) {
            // its calls may sit on any stream of the device
            if (hipDeviceSynchronize() != hipSuccess) return SCAN_ERR_HIP;
            words[1] = g_static[dev].ws.err;
        }
        uint32_t err = 0;
        for (uint32_t* w : words) {
            if (!w) continue;
            uint32_t e = 0;
            if (hipMemcpy(&e, w, 4, hipMemcpyDeviceToHost) != hipSuccess) return SCAN_ERR_HIP;
            if (e) {
                const uint32_t zero = 0;
                if (hipMemcpy(w, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return SCAN_ERR_HIP;
            }
            err |= e;
        }
        if (err & kErrTimeout) return SCAN_ERR_TIMEOUT;
        return err ? SCAN_ERR_HIP : SCAN_OK;
    } catch (const std::bad_alloc&) {
        return SCAN_ERR_NOMEM;
    }
}

scan_status_t scan_release_workspace(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    scan_status_t st = SCAN_OK;
    for (auto& kv : g_ws) {
        if (!kv.second.mem && !kv.second.rts && !kv.second.hist) continue;
        if (hipSetDevice(kv.first.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            st = SCAN_ERR_HIP;
        if (kv.second.mem && hipFree(kv.second.mem) != hipSuccess) st = SCAN_ERR_HIP;
        if (kv.second.rts && hipFree(kv.second.rts) != hipSuccess) st = SCAN_ERR_HIP;
        if (kv.second.hist && hipFree(kv.second.hist) != hipSuccess) st = SCAN_ERR_HIP;
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
    return st;
}

size_t scan_set_small_n_max(size_t n_max)
{
    std::lock_guard<std::mutex> lock(g_mu);
    const size_t old = g_small_n_max;
    g_small_n_max = n_max;
    return old;
}

int scan_set_multi_tile_mode(int mode)
{
    std::lock_guard<std::mutex> lock(g_mu);
    const int old = g_multi_mode;
    g_multi_mode = (mode >= 1 && mode <= 3) ? mode : 0;
    return old;
}

uint32_t scan_set_spin_limit(uint32_t polls)
{
    std::lock_guard<std::mutex> lock(g_mu);
    const uint32_t old = g_spin_limit;
    g_spin_limit = polls;
    return old;
}

}  // extern "C"

// ------------------------------------------------------------ copy probe
namespace {
// One 16-byte vector per lane, streaming loads, and stores with the same
// cache policy as the scan's whole-tile stores: the fastest plain copy
// measured on MI355X (about 6.5 TB/s for 1 GiB each way), i.e. the practical
// ceiling of a one-read-one-write kernel.
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out,
                                                          size_t nvec)
{
    for (size_t b = blockIdx.x * (size_t)256; b < nvec; b += (size_t)gridDim.x * 256) {
        const size_t i = b + threadIdx.x;
        if (i < nvec)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_nontemporal_load(in + i), wave_rsrc(out + b),
                                                   threadIdx.x * 16u, 0, DWPT_STORE_POLICY);
    }
}
}  // namespace

extern "C" scan_status_t scan_copy_probe(const void* in, void* out, size_t nbytes, void* stream)
{
    if (nbytes == 0) return SCAN_OK;
    if (!in || !out || nbytes % 16 || !is_aligned(in, 16) || !is_aligned(out, 16)) return SCAN_ERR_INVALID;
    const size_t nvec = nbytes / 16;
    size_t grid = (nvec + 255) / 256;
    if (grid > 65536 * 4) grid = 65536 * 4;
    hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(in), static_cast<u32x4*>(out), nvec);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}
