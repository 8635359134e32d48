// CSR row offsets from COO row indices: row_ptr[r] = number of entries with
// row index < r, for r = 0 .. n_rows.  Building the CSR sparse format is one
// of the uses of a prefix sum listed in the introduction of
// "CUDA编程并行前缀和扫描详解"; the row pointer array has N + 1 entries
// ("UIUC ECE 408 应用并行编程", L09).  Two steps: count the entries of every
// row into row_ptr (csr_count_kernel, csr_count_lds_kernel for up to 16384
// rows, csr_count_small_kernel for up to 1023 rows and 16-byte aligned
// indices, after row_ptr is zeroed), then an exclusive add scan of the n_rows + 1
// counts in place (the library's scan).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wave_ops.hpp"

namespace dwpt {

constexpr int kCsrBlock = 256;
constexpr int kCsrSteps = 16;  // 64-entry windows per wavefront and chunk

__global__ __launch_bounds__(kCsrBlock) void zero_u32_kernel(uint32_t* p, uint64_t n)
{
    for (uint64_t i = blockIdx.x * (uint64_t)kCsrBlock + threadIdx.x; i < n; i += (uint64_t)gridDim.x * kCsrBlock)
        p[i] = 0u;
}

// Every wavefront takes chunks of kCsrSteps windows of 64 consecutive
// entries, one entry per lane (coalesced 4-byte loads, all issued before any
// is used).  In a window, a lane whose row differs from its left neighbour's
// starts a run; the ballot of run starts gives each run's length, and the
// lane that starts it adds the whole run with one add(row, length).  Sorted
// input thus costs about one add per row and window, unsorted input one per
// entry at worst; both count exactly.  Rows >= n_rows are skipped.
template <int BLOCK, class Add>
__device__ __forceinline__ void count_runs(const uint32_t* __restrict__ rows, uint64_t nnz, uint32_t n_rows, Add add)
{
    const int lane = lane_id();
    const uint64_t wave = (blockIdx.x * (uint64_t)BLOCK + threadIdx.x) >> 6;
    const uint64_t waves = (gridDim.x * (uint64_t)BLOCK) >> 6;
    constexpr uint64_t kChunk = 64 * kCsrSteps;
    for (uint64_t base = wave * kChunk; base < nnz; base += waves * kChunk) {
        uint32_t r[kCsrSteps];
#pragma unroll
        for (int s = 0; s < kCsrSteps; ++s) {
            const uint64_t i = base + (uint64_t)s * 64 + lane;
            r[s] = i < nnz ? rows[i] : 0xFFFFFFFFu;  // past the end: never a valid row
        }
#pragma unroll
        for (int s = 0; s < kCsrSteps; ++s) {
            const uint32_t prev = wave_shift_up(r[s], ~r[s]);  // lane 0: a value unequal to its own
            const bool start = r[s] != prev;
            const uint64_t starts = wave_ballot(start);
            // the next run start above this lane, or the end of the window
            const uint64_t above = lane == 63 ? 0ull : starts & (~0ull << (lane + 1));
            const uint32_t len = (uint32_t)((above ? __builtin_ctzll(above) : 64) - lane);
            if (start && r[s] < n_rows) add(r[s], len);
        }
    }
}

// Any number of rows: the runs are added to the counts in memory with
// device-wide atomics.
__global__ __launch_bounds__(kCsrBlock) void csr_count_kernel(const uint32_t* __restrict__ rows, uint64_t nnz,
                                                              uint32_t n_rows, uint32_t* counts)
{
    count_runs<kCsrBlock>(rows, nnz, n_rows, [&](uint32_t row, uint32_t len) {
        __hip_atomic_fetch_add(&counts[row], len, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    });
}

// Up to kCsrLdsBins rows (a histogram of few bins): each workgroup counts
// into its own copy of the counts in LDS (n_rows words of dynamic LDS) and
// adds its nonzero counts to memory once at the end.  With many entries per
// bin the device-wide atomics would otherwise be one per entry for unsorted
// input, all on a few addresses; here they are at most n_rows per workgroup.
constexpr uint32_t kCsrLdsBins = 16384;  // 64 KiB of counts
constexpr int kCsrLdsBlock = 1024;       // one workgroup per CU, 16 wavefronts

__global__ __launch_bounds__(kCsrLdsBlock) void csr_count_lds_kernel(const uint32_t* __restrict__ rows, uint64_t nnz,
                                                                     uint32_t n_rows, uint32_t* counts)
{
    extern __shared__ uint32_t s_cnt[];  // n_rows words
    for (uint32_t i = threadIdx.x; i < n_rows; i += kCsrLdsBlock) s_cnt[i] = 0u;
    __syncthreads();
    count_runs<kCsrLdsBlock>(rows, nnz, n_rows, [&](uint32_t row, uint32_t len) {
        __hip_atomic_fetch_add(&s_cnt[row], len, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    });
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n_rows; i += kCsrLdsBlock) {
        const uint32_t c = s_cnt[i];
        if (c) __hip_atomic_fetch_add(&counts[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Up to kCsrSmallBins rows (a histogram of few bins), indices 16-byte
// aligned: no run detection, every index is counted with one LDS add into
// one of kCsrCopies copies of the counts (lane l into copy l mod kCsrCopies,
// so that at most four lanes of an instruction ever share a word, even when
// every index names the same bin), four indices per lane and 16-byte load.
// The workgroups take 16-byte chunks in grid order, so that at any moment
// the chip reads one contiguous stretch of the indices.  At the end each
// workgroup folds its copies and adds its nonzero counts to memory.
constexpr uint32_t kCsrSmallBins = 1023;  // 64 KiB of counts in all
constexpr int kCsrCopies = 16;
constexpr int kCsrSmallUnroll = 2;  // 16-byte loads in flight per lane (1 or 3 are slower)

__global__ __launch_bounds__(kCsrLdsBlock) void csr_count_small_kernel(const uint32_t* __restrict__ rows, uint64_t nnz,
                                                                       uint32_t n_rows, uint32_t* counts)
{
    extern __shared__ uint32_t s_cnt[];  // kCsrCopies rows of n_rows + 1 words
    const uint32_t stride = n_rows + 1;  // copies start in different banks
    for (uint32_t i = threadIdx.x; i < kCsrCopies * stride; i += kCsrLdsBlock) s_cnt[i] = 0u;
    __syncthreads();
    uint32_t* my = s_cnt + (lane_id() % kCsrCopies) * stride;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(rows);
    const uint64_t n4 = nnz / 4;
    const uint64_t step = (uint64_t)gridDim.x * kCsrLdsBlock;
    for (uint64_t c = blockIdx.x * (uint64_t)kCsrLdsBlock + threadIdx.x; c < n4; c += step * kCsrSmallUnroll) {
        u32x4_t q[kCsrSmallUnroll];
#pragma unroll
        for (int u = 0; u < kCsrSmallUnroll; ++u) {
            const uint64_t j = c + (uint64_t)u * step;
            q[u] = j < n4 ? __builtin_nontemporal_load(src + j) : u32x4_t{~0u, ~0u, ~0u, ~0u};
        }
#pragma unroll
        for (int u = 0; u < kCsrSmallUnroll; ++u) {
            if (q[u].x < n_rows) atomicAdd(my + q[u].x, 1u);
            if (q[u].y < n_rows) atomicAdd(my + q[u].y, 1u);
            if (q[u].z < n_rows) atomicAdd(my + q[u].z, 1u);
            if (q[u].w < n_rows) atomicAdd(my + q[u].w, 1u);
        }
    }
    // the last nnz mod 4 indices
    if (blockIdx.x == 0 && threadIdx.x < (uint32_t)(nnz % 4)) {
        const uint32_t r = rows[n4 * 4 + threadIdx.x];
        if (r < n_rows) atomicAdd(my + r, 1u);
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n_rows; i += kCsrLdsBlock) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < kCsrCopies; ++k) c += s_cnt[k * stride + i];
        if (c) __hip_atomic_fetch_add(&counts[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace dwpt
