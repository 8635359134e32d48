// wave_ops.hpp -- 64-lane wavefront scan built from DPP lane shifts (gfx950).
//
// Pages cited:
//   [L7] "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
//        (UIUC ECE408 course notes, runguoli.com)
//
// The shift-and-combine steps are the Hillis-Steele pattern [L7 concept 3
// "Hillis-Steele（Kogge-Stone）扫描算法"] applied to registers across the
// lanes of one wavefront, as the lecture suggests doing with warp shuffles
// for the levels inside a warp [L7 concept 7, bank-conflict remedies].  On
// CDNA the lanes of a 64-wide wavefront exchange data through DPP: four
// in-row shifts (rows of 16 lanes) and two row broadcasts give an inclusive
// scan in six steps, with no LDS and no barrier.  The shifted value always
// comes from a lower lane, i.e. an earlier element, and is the left operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_ops.hpp"

namespace dwpt {

// DPP control codes (GFX9 encoding).
enum : int {
    kDppRowShr1 = 0x111,
    kDppRowShr2 = 0x112,
    kDppRowShr4 = 0x114,
    kDppRowShr8 = 0x118,
    kDppWaveShr1 = 0x138,
    kDppRowBcast15 = 0x142,
    kDppRowBcast31 = 0x143,
};

// Lane-shifted copy of v; lanes with no source lane (or in rows outside
// ROW_MASK) receive `old`.  Works for any type made of 32-bit words.
template <int CTRL, int ROW_MASK, typename V>
__device__ __forceinline__ V dpp_move(V v, V old)
{
    constexpr int W = sizeof(V) / 4;
    uint32_t s[W], o[W], r[W];
    to_words(v, s);
    to_words(old, o);
#pragma unroll
    for (int i = 0; i < W; ++i)
        r[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)o[i], (int)s[i], CTRL, ROW_MASK, 0xF, false);
    return from_words<V>(r);
}

template <typename V>
__device__ __forceinline__ V read_lane(V v, int lane)
{
    constexpr int W = sizeof(V) / 4;
    uint32_t s[W], r[W];
    to_words(v, s);
#pragma unroll
    for (int i = 0; i < W; ++i) r[i] = (uint32_t)__builtin_amdgcn_readlane((int)s[i], lane);
    return from_words<V>(r);
}

// Inclusive scan over the 64 lanes of the wavefront: lane l receives
// v_0 (+) v_1 (+) ... (+) v_l.  `comb(earlier, later)` is the operator.
template <typename V, typename Comb>
__device__ __forceinline__ V wave_inclusive_scan(V v, V ident, Comb comb)
{
    v = comb(dpp_move<kDppRowShr1, 0xF>(v, ident), v);
    v = comb(dpp_move<kDppRowShr2, 0xF>(v, ident), v);
    v = comb(dpp_move<kDppRowShr4, 0xF>(v, ident), v);
    v = comb(dpp_move<kDppRowShr8, 0xF>(v, ident), v);
    // lane 15 of row r goes to all of row r+1, for rows 1 and 3
    v = comb(dpp_move<kDppRowBcast15, 0xA>(v, ident), v);
    // lane 31 goes to all of rows 2 and 3
    v = comb(dpp_move<kDppRowBcast31, 0xC>(v, ident), v);
    return v;
}

// Float32 add: the same six steps, but the two row broadcasts as single
// v_add_f32 DPP instructions.  The compiler fuses a DPP move into the add
// only when the masked-off rows' "old" value is an identity it knows, and it
// knows none for float add (-0.0 would be one), so the generic version costs a
// register fill, a DPP move and a separate add per broadcast step.  Here the
// disabled rows are simply not written (destination = source), which keeps
// their value exactly.  The s_nop gives the two wait states a DPP read needs
// after a VALU write of its source register.
#ifndef DWPT_FADD_DPP
#define DWPT_FADD_DPP 1
#endif
__device__ __forceinline__ float wave_inclusive_scan_fadd(float v)
{
    const auto add = [](float a, float b) { return a + b; };
    v = add(dpp_move<kDppRowShr1, 0xF>(v, 0.0f), v);
    v = add(dpp_move<kDppRowShr2, 0xF>(v, 0.0f), v);
    v = add(dpp_move<kDppRowShr4, 0xF>(v, 0.0f), v);
    v = add(dpp_move<kDppRowShr8, 0xF>(v, 0.0f), v);
#if DWPT_FADD_DPP
    asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf" : "+v"(v));
    asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf" : "+v"(v));
#else
    v = add(dpp_move<kDppRowBcast15, 0xA>(v, 0.0f), v);
    v = add(dpp_move<kDppRowBcast31, 0xC>(v, 0.0f), v);
#endif
    return v;
}

// Value of the next lower lane (identity in lane 0): turns an inclusive
// wavefront scan into an exclusive one without needing an inverse.
template <typename V>
__device__ __forceinline__ V wave_shift_up(V v, V ident)
{
    return dpp_move<kDppWaveShr1, 0xF>(v, ident);
}

__device__ __forceinline__ uint64_t wave_ballot(bool p)
{
    return __builtin_amdgcn_ballot_w64(p);
}

__device__ __forceinline__ int lane_id()
{
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

}  // namespace dwpt
