/*
 * dwpt_scan.h -- C ABI of the MI355X (gfx950) device-wide prefix scan library
 * (libdwpt_scan.so).
 *
 * Pages cited:
 *   [L7]    "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
 *           (UIUC ECE408 course notes, runguoli.com)
 *   [PMPP9] "第9章并行模式：前缀和 - Scan算法" (PMPP chapter 9 notes, bittern.cn)
 *   [YLY]   "CUDA编程并行前缀和扫描详解" (tutorial, m.youleyou.com)
 *
 * Conventions shared by every entry point:
 *   - `in`, `out`, `head_flags` and `d_count` are DEVICE pointers owned by the
 *     caller (hipMalloc'd or torch CUDA tensors on the current device).  The
 *     library never frees or keeps them past the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work: they return before the GPU has finished, and
 *     results (and device-side errors, see scan_get_device_error) are visible
 *     after the stream is synchronised.
 *   - n is an element count (pairs for the U32X2 and I32_U32 dtypes,
 *     matrices for U32X4 and U32X9).  n == 0 returns SCAN_OK and launches
 *     nothing.
 *   - Pointers must be aligned to the element size (4 bytes for the 36-byte
 *     U32X9 matrices, which are arrays of uint32); 16-byte alignment selects
 *     the vector path, anything else a slower scalar path with the same
 *     results.  `out` may equal `in` (in-place); partial overlap is rejected.
 *   - Errors are returned, never raised: argument errors (null pointer with
 *     n > 0, misalignment, partial overlap, n too large) give
 *     SCAN_ERR_INVALID before anything is launched; an op/dtype pair outside
 *     the table below gives SCAN_ERR_UNSUPPORTED; a failed HIP call gives
 *     SCAN_ERR_HIP (hipGetLastError has the HIP code); failure to get
 *     workspace memory gives SCAN_ERR_NOMEM.
 *   - Workspace: the multi-tile path keeps a status array (17 eight-byte
 *     words per tile of 3584-15360 elements and per status word of its
 *     carry: 1 for 32-bit carries and the float32 sum, 2 for AFFINE and
 *     MAX_COUNT, 4 for MAT2, 9 for MAT3) and counters per (device, stream); reduce-then-scan and the radix
 *     pass add a plain buffer each (the tile carries; 256 uint32 counts per
 *     8192-key tile).  Each is allocated on first use, grown when needed
 *     (after the stream has drained) and reused across calls without
 *     clearing.  Calls on one stream are serialised by the stream; calls on
 *     different streams use different workspaces.
 *   - Host threads: entry points may be called from several threads, but
 *     calls on one stream must come from one thread at a time (a call may
 *     grow that stream's workspace while the previous call's kernels are
 *     still queued on it, which is safe only in stream order).
 *
 * Valid combinations:
 *   scan_inclusive / scan_exclusive: ADD, MAX, MIN with I32, U32, F32;
 *                                    AFFINE with U32X2; MAX_COUNT with
 *                                    I32_U32; MAT2 with U32X4; MAT3 with
 *                                    U32X9; AND, OR with I32, U32.
 *   segmented_scan:                  ADD, MAX, MIN with I32, U32, F32.
 *   compact:                         I32, U32, F32.
 * Integer ADD wraps modulo 2^32.  F32 ADD results may differ from an exact
 * sum by rounding (any association is allowed); the prefix carried between
 * tiles is kept in double so the error stays well inside
 * 1e-5 * sum_{k<=i} |x_k| + 1e-6.  MAX/MIN keep the earlier value on ties
 * (for F32: of +0 and -0, whichever comes first).  F32 MAX/MIN inputs must
 * not hold NaN: NaN is unordered, the operator is then not associative, and
 * results would depend on the kernel path (unsupported, unspecified).
 *
 * Bounded waits: tiles wait for one another on the device.  Every such wait
 * gives up after a poll budget (scan_set_spin_limit); the first one that does
 * records SCAN_ERR_TIMEOUT (see scan_get_device_error) and makes every other
 * wait of the same call give up at its next check, so a call always finishes.
 */
#ifndef DWPT_SCAN_H
#define DWPT_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SCAN_OK = 0,
    SCAN_ERR_INVALID = 1,
    SCAN_ERR_UNSUPPORTED = 2,
    SCAN_ERR_NOMEM = 3,
    SCAN_ERR_HIP = 4,
    SCAN_ERR_TIMEOUT = 5
} scan_status_t;

typedef enum {
    SCAN_OP_ADD = 0,
    SCAN_OP_MAX = 1,
    SCAN_OP_MIN = 2,
    SCAN_OP_AFFINE = 3,    /* x -> a*x + b maps composed, later map applied after */
    SCAN_OP_MAX_COUNT = 4, /* (maximum, number of occurrences) composite */
    SCAN_OP_MAT2 = 5,      /* 2x2 matrix product, later factor on the left */
    SCAN_OP_MAT3 = 6,      /* 3x3 matrix product, later factor on the left */
    SCAN_OP_AND = 7,       /* bitwise AND */
    SCAN_OP_OR = 8         /* bitwise OR */
} scan_op_t;

typedef enum {
    SCAN_I32 = 0,
    SCAN_U32 = 1,
    SCAN_F32 = 2,
    SCAN_U32X2 = 3,   /* (a, b) pairs of uint32, 8 bytes per element */
    SCAN_I32_U32 = 4, /* (int32 value, uint32 count) pairs, 8 bytes per element */
    SCAN_U32X4 = 5,   /* 2x2 uint32 matrices [[a, b], [c, d]] stored a, b, c, d: 16 bytes */
    SCAN_U32X9 = 6    /* 3x3 uint32 matrices stored row-major: 36 bytes, 4-byte aligned */
} scan_dtype_t;

/*
 * Inclusive scan: out[i] = in[0] (+) in[1] (+) ... (+) in[i].
 * [L7 concept 1 "扫描（Scan / Prefix Sum）：inclusive 与 exclusive";
 *  PMPP9 §9.1; YLY §2.1]  The operator must be associative; operand order is
 * kept (earlier element on the left), commutativity is never assumed.
 * For AFFINE, element i of the result is the composition of maps 0..i:
 * (a2,b2) o (a1,b1) = (a2*a1, a2*b1 + b2) mod 2^32, i.e. its b component is
 * the recurrence y_i = a_i*y_{i-1} + b_i with y_{-1} = 0 [L7 concept 1,
 * recurrences as scans].
 * MAX_COUNT and MAT2 are the composite and matrix operators [L7 concept 1,
 * operator generalisation]: (v1,c1) (+) (v2,c2) keeps the larger value and,
 * on a tie, adds the counts (mod 2^32) -- fed (x_i, 1) it gives the maximum
 * so far and how often it occurred; MAT2 and MAT3 multiply 2x2 and 3x3
 * matrices mod 2^32 with the later factor on the left (affine maps are
 * [[a, b], [0, 1]]; 2x2 matrices A are the 3x3 [[A, 0], [0, 1]]).
 * AND and OR are the bitwise operators, also named as scan operators there.
 */
scan_status_t scan_inclusive(scan_op_t op, scan_dtype_t dtype, const void* in, void* out,
                             size_t n, void* stream);

/*
 * Exclusive scan: out[0] = identity, out[i] = in[0] (+) ... (+) in[i-1].
 * [L7 concept 1; PMPP9 §9.1 (identity table); YLY §2.2]  Identities: ADD 0,
 * MAX the type's lowest value (-inf for F32), MIN its highest (+inf),
 * AFFINE (1, 0), MAX_COUNT (INT32_MIN, 0), MAT2 and MAT3 the identity
 * matrix, AND all bits set, OR no bits set.
 */
scan_status_t scan_exclusive(scan_op_t op, scan_dtype_t dtype, const void* in, void* out,
                             size_t n, void* stream);

/*
 * Segmented scan: the scan restarts at every element whose head flag is
 * nonzero; element 0 always starts a segment whatever its flag.
 * `head_flags` is a device array of n bytes.  Inclusive (exclusive == 0):
 * out[i] = fold of in[s..i]; exclusive: out[i] = fold of in[s..i-1], the
 * identity at every head, where s is the head of i's segment.
 * [L7 concept 2 "扫描的典型应用", radix-sort placement as a segmented scan]
 */
scan_status_t segmented_scan(scan_op_t op, scan_dtype_t dtype, const void* in,
                             const uint8_t* head_flags, void* out, size_t n, int exclusive,
                             void* stream);

/*
 * Stream compaction: writes the elements with in[i] > 0, in input order, to
 * out[0 .. count) and the count (uint32) to *d_count (device memory).
 * out[count .. n) is left untouched.  The write position of a kept element
 * is the exclusive scan of the 0/1 predicate flags [L7 concept 2 compaction
 * figure; PMPP9 §9.6 array compaction; YLY §2.2 flag/pos example].  -0.0
 * and NaN are not kept.  Requires n < 2^32.  out may equal in (in place);
 * d_count must overlap neither in nor out (SCAN_ERR_INVALID).  In place, the
 * reduce-then-scan mode (scan_set_multi_tile_mode(3)) is not used: its last
 * pass would write a tile's kept elements over input that earlier tiles of
 * the same launch may not have read yet, so the call runs the single-pass
 * kernels instead.
 */
scan_status_t compact(scan_dtype_t dtype, const void* in, void* out, uint32_t* d_count, size_t n,
                      void* stream);

/*
 * CSR row offsets from COO row indices: row_ptr[r] = the number of entries
 * i with row_idx[i] < r, for r = 0 .. n_rows (n_rows + 1 values, so
 * row_ptr[n_rows] is the number of entries counted).  Entries whose row
 * index is n_rows or more are not counted.  The counts of every row go to
 * row_ptr, and an exclusive add scan of them in place gives the offsets:
 * building the CSR format is among the uses of a prefix sum that [YLY]
 * lists in its introduction, and the row pointer array has N + 1 entries
 * ("UIUC ECE 408 应用并行编程", L09).  row_idx (nnz uint32, any order) and
 * row_ptr (n_rows + 1 uint32, caller-owned) are device arrays aligned to 4
 * bytes that must not overlap; nnz < 2^32.  Sorted indices cost about one
 * atomic add per row, unsorted ones up to one per entry.
 */
scan_status_t csr_row_offsets(const uint32_t* row_idx, size_t nnz, uint32_t n_rows, uint32_t* row_ptr,
                              void* stream);

/*
 * One pass of a least-significant-digit radix sort: a stable split of the
 * uint32 keys by the 8-bit digit (key >> shift) & 255.  keys_out receives
 * the keys ordered by digit, keys of one digit in their input order; if
 * vals is given, vals_out receives each key's value at the key's new place.
 * Four passes with shift = 0, 8, 16, 24 sort 32-bit keys.  Radix sort is a
 * split by digit plus a scan that places every element [L7 concept 2,
 * radix sort]; the scan of the digit histogram gives each bucket's first
 * position [PMPP9 §9.6 radix sort].
 *
 * keys, keys_out (and vals, vals_out) are device arrays of n uint32 aligned
 * to 4 bytes; vals and vals_out are both NULL or both non-NULL.  No output
 * may overlap an input or the other output (the split is out of place).
 * shift <= 31; n < 2^32.  n == 0 does nothing.  The digit histograms (256
 * uint32 per 8192 keys, and 256 per 65536 keys) live in the library's
 * per-stream workspace.
 */
scan_status_t radix_split(const uint32_t* keys, const uint32_t* vals, size_t n, uint32_t shift,
                          uint32_t* keys_out, uint32_t* vals_out, void* stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the plain
 * inclusive (exclusive == 0) or exclusive scan, as scan_inclusive /
 * scan_exclusive (same operators, types, results, alignment and overlap
 * rules), that allocates nothing.  The tiles' status words and counters live
 * in a static device array of the library, 16 MiB on each GPU it runs on,
 * held until the process ends (set up and cleared on a GPU's first call, with
 * a fill kernel on that call's stream).  Inputs whose status words do not fit
 * are rejected with SCAN_ERR_INVALID before anything is launched: tiles *
 * words * 17 * 8 bytes must fit in 16 MiB - 640 bytes, with tiles = ceil(n /
 * tile) and (tile, words) = (15360, 1) for ADD, MAX, MIN, AND, OR over
 * I32, U32 and F32, (7680, 2) AFFINE, (7168, 2) MAX_COUNT, (3584, 4) MAT2,
 * (3584, 9) MAT3 -- e.g. n up to 1,894,763,520 for the 4-byte types.  Every call on a GPU shares that
 * GPU's array (the last call's contents stay in it): calls that overlap in
 * time on one GPU, e.g. on two streams, race and give wrong results; calls
 * in one stream's order, or separated by synchronisation, are safe.  The
 * reduce-then-scan mode (scan_set_multi_tile_mode(3)) is not used here (the
 * automatic choice runs instead).  Device errors of these calls are reported
 * by scan_get_device_error on the same device.
 */
scan_status_t scan_noalloc(scan_op_t op, scan_dtype_t dtype, const void* in, void* out, size_t n,
                           int exclusive, void* stream);

/* Static text for a status code (never NULL). */
const char* scan_status_string(scan_status_t s);

/*
 * Synchronises `stream`, then reads and clears the device error word of its
 * workspace (and, once scan_noalloc has run on the current device, after
 * synchronising the device, that of its static array): SCAN_ERR_TIMEOUT if a
 * look-back wait gave up since the last check (the results of that call are
 * then wrong), SCAN_ERR_HIP if a workgroup found the tile counter out of
 * step with its launch (it then skipped its tile), SCAN_OK otherwise.
 */
scan_status_t scan_get_device_error(void* stream);

/* Frees every workspace of the calling process (synchronises the device). */
scan_status_t scan_release_workspace(void);

/*
 * Tuning and test knobs (process-wide, thread-safe; each returns the old value).
 * scan_set_small_n_max: inputs with n at or below this size run on one
 *   workgroup that walks the tiles in order (no workspace, no atomics); larger
 *   inputs use the multi-tile look-back kernel.  Default SCAN_SMALL_N_AUTO:
 *   one tile of the operation's shape (15360 four-byte elements, 7680 affine
 *   pairs, ...), where one workgroup stops being faster than one workgroup
 *   per tile.
 * scan_set_multi_tile_mode: selects the kernel for inputs above the
 *   small-n size.  2 runs the persistent pipelined kernel (one launch of as
 *   many workgroups as fit on the GPU, each taking tile numbers from a
 *   counter until the input is done); 1 runs one workgroup per tile; 0 (the
 *   default) takes the persistent kernel from 3 tiles per resident
 *   workgroup up (about 1.2e7 four-byte elements on 256 compute units) and
 *   one workgroup per tile below.  3 runs reduce-then-scan: three launches
 *   (tile totals, one workgroup scanning them, every tile scanned again
 *   from its prefix), which reads the input twice but never makes a tile
 *   wait for another, and fixes the association of float sums by n alone.
 *   Other values select 0.
 * scan_set_spin_limit: number of look-back polls after which a waiting tile
 *   gives up, records SCAN_ERR_TIMEOUT (see scan_get_device_error) and
 *   finishes with a wrong prefix instead of waiting forever.  Default 2^18.
 */
#define SCAN_SMALL_N_AUTO ((size_t)-1)
size_t scan_set_small_n_max(size_t n_max);
int scan_set_multi_tile_mode(int mode);
uint32_t scan_set_spin_limit(uint32_t polls);

/*
 * Measurement helper, not part of the scan: copies nbytes (a multiple of 16,
 * 16-byte aligned pointers) from in to out with a plain streaming kernel
 * (its stores carry the same cache policy as the scan's whole-tile stores), to
 * calibrate achievable HBM bandwidth and the traffic counters.  Returns
 * SCAN_ERR_INVALID for null pointers, misalignment or a size not a multiple
 * of 16; nbytes == 0 does nothing.
 */
scan_status_t scan_copy_probe(const void* in, void* out, size_t nbytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DWPT_SCAN_H */
