// scan_ops.hpp -- associative operators of the device-wide scan (gfx950).
//
// Pages cited:
//   [L7]    "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
//           (UIUC ECE408 course notes, runguoli.com)
//   [PMPP9] "第9章并行模式：前缀和 - Scan算法" (PMPP chapter 9 notes, bittern.cn)
//
// A scan needs only associativity; operand order is fixed, the earlier
// value is always the left argument [L7 concept 1, operator generalisation].
// Identities follow the table of [PMPP9 §9.1]: + -> 0, max -> -inf,
// min -> +inf; for 32-bit integers the extreme values of the type stand for
// -inf/+inf, and the affine map's identity is (1, 0).
//
// Each operator trait exposes:
//   elem_t            element type in memory
//   value_t           value scanned inside a tile (registers)
//   carry_t           inter-tile prefix type (wider for float32 add)
//   prep_t            a carry made ready to be applied per element
//   identity(), combine(earlier, later)            on value_t
//   carry_identity(), to_carry(v), combine_carry(earlier, later)
//   prepare(carry) -> prep_t, apply(prep, local) -> value_t   (= carry (+) local)
//   kWords, pack(carry, payloads, flag), unpack(payloads, flag)
//                     status-word codec: kWords payloads of at most 49 bits
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dwpt {

struct Affine {
    uint32_t a, b;
};
struct MaxCount {
    int32_t m;   // the largest value so far
    uint32_t c;  // the summed counts of the elements that carry it
};
struct Mat2 {
    uint32_t a, b, c, d;  // [[a, b], [c, d]], row-major
};
struct Mat3 {
    uint32_t m[9];  // row-major: m[3 * r + c] is row r, column c
};

// ---------------------------------------------------------------- helpers
template <typename V>
__device__ __forceinline__ void to_words(const V& v, uint32_t* w)
{
    static_assert(sizeof(V) % 4 == 0, "32-bit multiple");
    __builtin_memcpy(w, &v, sizeof(V));
}
template <typename V>
__device__ __forceinline__ V from_words(const uint32_t* w)
{
    V v;
    __builtin_memcpy(&v, w, sizeof(V));
    return v;
}

// Common part for operators whose carry is their own value type.
template <typename T, typename Derived>
struct SameCarry {
    using elem_t = T;
    using value_t = T;
    using carry_t = T;
    using prep_t = T;
    static constexpr int kWords = sizeof(T) / 4;
    __device__ __forceinline__ static carry_t carry_identity() { return Derived::identity(); }
    __device__ __forceinline__ static carry_t to_carry(value_t v) { return v; }
    __device__ __forceinline__ static carry_t combine_carry(carry_t a, carry_t b) { return Derived::combine(a, b); }
    __device__ __forceinline__ static prep_t prepare(carry_t c) { return c; }
    __device__ __forceinline__ static value_t apply(prep_t c, value_t local) { return Derived::combine(c, local); }
    __device__ __forceinline__ static void pack(carry_t c, uint64_t* w, uint32_t& flag)
    {
        uint32_t t[kWords];
        to_words(c, t);
#pragma unroll
        for (int k = 0; k < kWords; ++k) w[k] = t[k];
        flag = 0;
    }
    __device__ __forceinline__ static carry_t unpack(const uint64_t* w, uint32_t)
    {
        uint32_t t[kWords];
#pragma unroll
        for (int k = 0; k < kWords; ++k) t[k] = (uint32_t)w[k];
        return from_words<carry_t>(t);
    }
};

// ---------------------------------------------------------------- add
template <typename T> struct OpAdd;

// int32 add wraps modulo 2^32 (done in uint32 to keep it defined).
template <> struct OpAdd<int32_t> : SameCarry<int32_t, OpAdd<int32_t>> {
    __device__ __forceinline__ static int32_t identity() { return 0; }
    __device__ __forceinline__ static int32_t combine(int32_t a, int32_t b)
    {
        return (int32_t)((uint32_t)a + (uint32_t)b);
    }
};

template <> struct OpAdd<uint32_t> : SameCarry<uint32_t, OpAdd<uint32_t>> {
    __device__ __forceinline__ static uint32_t identity() { return 0u; }
    __device__ __forceinline__ static uint32_t combine(uint32_t a, uint32_t b) { return a + b; }
};

// float32 add: tiles are summed in float32, but the prefix carried from tile
// to tile is a double.  Each lane rounds the double prefix of its elements
// (carry plus the in-tile prefix before them) to float once, and each output
// is that float plus the element's in-lane float partial: two roundings per
// output instead of one (a float pair hi + (lo + local) would round once),
// well inside the tolerance, and one float32 add per element instead of two
// (measured: 340.5 -> 339.2 us at 2^28 with identical worst error/tolerance).
// The error that grows with n -- the carry's -- stays in double.
struct F32Split {
    float hi, lo;
};
template <> struct OpAdd<float> {
    using elem_t = float;
    using value_t = float;
    using carry_t = double;
    using prep_t = F32Split;
    static constexpr int kWords = 1;
    __device__ __forceinline__ static float identity() { return 0.0f; }
    __device__ __forceinline__ static float combine(float a, float b) { return a + b; }
    __device__ __forceinline__ static double carry_identity() { return 0.0; }
    __device__ __forceinline__ static double to_carry(float v) { return (double)v; }
    __device__ __forceinline__ static double combine_carry(double a, double b) { return a + b; }
#ifndef DWPT_F32_APPLY_HI
#define DWPT_F32_APPLY_HI 1  // 0: the single-rounding hi + (lo + local)
#endif
    __device__ __forceinline__ static F32Split prepare(double c)
    {
        float hi = (float)c;
#if DWPT_F32_APPLY_HI
        return {hi, 0.0f};
#else
        float lo = (float)(c - (double)hi);
        return {hi, lo};
#endif
    }
#if DWPT_F32_APPLY_HI
    __device__ __forceinline__ static float apply(F32Split c, float local) { return c.hi + local; }
#else
    __device__ __forceinline__ static float apply(F32Split c, float local) { return c.hi + (c.lo + local); }
#endif
    // One 49-bit status payload: the double's sign, exponent and a 37-bit
    // mantissa, rounded to nearest (relative error below 2^-38).  Tile totals
    // are floats and pass exactly; a published prefix is rounded once -- the
    // streaming resolver keeps its running carry in full double, and the
    // carries are rounded to float before they are applied anyway.
    __device__ __forceinline__ static void pack(double c, uint64_t* w, uint32_t& flag)
    {
        const uint64_t b = __builtin_bit_cast(uint64_t, c);
        const uint64_t mag = ((b & 0x7FFFFFFFFFFFFFFFull) + (1ull << 14)) >> 15;  // 48 bits: exponent, mantissa
        w[0] = ((b >> 63) << 48) | mag;
        flag = 0;
    }
    __device__ __forceinline__ static double unpack(const uint64_t* w, uint32_t)
    {
        const uint64_t b = ((w[0] >> 48) << 63) | ((w[0] & 0xFFFFFFFFFFFFull) << 15);
        return __builtin_bit_cast(double, b);
    }
};

// ---------------------------------------------------------------- max / min
// A later value replaces the running one only when strictly greater
// (smaller); the earlier value wins ties, which keeps the operator
// associative for floats with +0/-0 and makes results bit-exact.
template <typename T> struct Limits;
template <> struct Limits<int32_t> {
    __device__ __forceinline__ static int32_t lowest() { return INT32_MIN; }
    __device__ __forceinline__ static int32_t highest() { return INT32_MAX; }
};
template <> struct Limits<uint32_t> {
    __device__ __forceinline__ static uint32_t lowest() { return 0u; }
    __device__ __forceinline__ static uint32_t highest() { return UINT32_MAX; }
};
template <> struct Limits<float> {
    __device__ __forceinline__ static float lowest() { return -__builtin_inff(); }
    __device__ __forceinline__ static float highest() { return __builtin_inff(); }
};

template <typename T> struct OpMax : SameCarry<T, OpMax<T>> {
    __device__ __forceinline__ static T identity() { return Limits<T>::lowest(); }
    __device__ __forceinline__ static T combine(T a, T b) { return (b > a) ? b : a; }
};
template <typename T> struct OpMin : SameCarry<T, OpMin<T>> {
    __device__ __forceinline__ static T identity() { return Limits<T>::highest(); }
    __device__ __forceinline__ static T combine(T a, T b) { return (b < a) ? b : a; }
};

// ---------------------------------------------------------------- bitwise
// Bitwise AND / OR, also scan operators [L7 concept 1, operator
// generalisation]; identities: all bits set / no bits set.
template <typename T> struct OpAnd : SameCarry<T, OpAnd<T>> {
    __device__ __forceinline__ static T identity() { return (T)~0u; }
    __device__ __forceinline__ static T combine(T a, T b) { return a & b; }
};
template <typename T> struct OpOr : SameCarry<T, OpOr<T>> {
    __device__ __forceinline__ static T identity() { return (T)0; }
    __device__ __forceinline__ static T combine(T a, T b) { return a | b; }
};

// ---------------------------------------------------------------- affine
// Composition of maps x -> a*x + b over uint32 (mod 2^32).  The later map is
// applied after the earlier one: (a2,b2) o (a1,b1) = (a2*a1, a2*b1 + b2).
// This is the matrix-product case of a non-commutative scan operator.
struct OpAffine : SameCarry<Affine, OpAffine> {
    __device__ __forceinline__ static Affine identity() { return {1u, 0u}; }
    __device__ __forceinline__ static Affine combine(Affine e, Affine l)
    {
        return {l.a * e.a, l.a * e.b + l.b};
    }
};

// ---------------------------------------------------------------- (max, count)
// The "(maximum, number of occurrences)" composite operator [L7 concept 1,
// operator generalisation]: keep the larger value; on a tie add the counts
// (mod 2^32).  Identity (INT32_MIN, 0).
struct OpMaxCount : SameCarry<MaxCount, OpMaxCount> {
    __device__ __forceinline__ static MaxCount identity() { return {INT32_MIN, 0u}; }
    __device__ __forceinline__ static MaxCount combine(MaxCount e, MaxCount l)
    {
        if (l.m > e.m) return l;
        if (l.m == e.m) return {e.m, e.c + l.c};
        return e;
    }
};

// ---------------------------------------------------------------- commutativity
// Operators whose result does not depend on the order of the operands, bit
// for bit: integer add/max/min/and/or, float add (exact per operation; only the
// rounding of a longer sum depends on its association, which the float
// tolerance already allows) and (maximum, count).  Not float max/min (the
// earlier of +0 and -0 wins), affine maps, matrices or segmented pairs.  A
// tile's total may then be folded lane by lane over all its rounds first.
template <class Op> struct IsCommutative { static constexpr bool value = false; };
template <> struct IsCommutative<OpAdd<int32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpAdd<uint32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpAdd<float>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpMax<int32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpMax<uint32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpMin<int32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpMin<uint32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpMaxCount> { static constexpr bool value = true; };
template <> struct IsCommutative<OpAnd<int32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpAnd<uint32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpOr<int32_t>> { static constexpr bool value = true; };
template <> struct IsCommutative<OpOr<uint32_t>> { static constexpr bool value = true; };

// ---------------------------------------------------------------- 2x2 matrices
// Matrix multiplication [L7 concept 1] over uint32 (mod 2^32), the later
// factor on the left: X_e (+) X_l = X_l * X_e, as for the affine maps, which
// are the matrices [[a, b], [0, 1]].  Identity: the identity matrix.
struct OpMat2 : SameCarry<Mat2, OpMat2> {
    __device__ __forceinline__ static Mat2 identity() { return {1u, 0u, 0u, 1u}; }
    __device__ __forceinline__ static Mat2 combine(Mat2 e, Mat2 l)
    {
        return {l.a * e.a + l.b * e.c, l.a * e.b + l.b * e.d, l.c * e.a + l.d * e.c, l.c * e.b + l.d * e.d};
    }
};

// ---------------------------------------------------------------- 3x3 matrices
// The same product one size up: X_e (+) X_l = X_l * X_e mod 2^32, 27
// multiplies per combine.  Identity: the identity matrix.
struct OpMat3 : SameCarry<Mat3, OpMat3> {
    __device__ __forceinline__ static Mat3 identity() { return {{1u, 0u, 0u, 0u, 1u, 0u, 0u, 0u, 1u}}; }
    __device__ __forceinline__ static Mat3 combine(Mat3 e, Mat3 l)
    {
        Mat3 r;
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                r.m[3 * i + j] = l.m[3 * i] * e.m[j] + l.m[3 * i + 1] * e.m[3 + j] + l.m[3 * i + 2] * e.m[6 + j];
        return r;
    }
};

// ---------------------------------------------------------------- segmented
// Segmented scan as a scan of (flag, value) pairs: a set flag marks that the
// span contains a segment head, and a head discards everything before it:
//   (f1, v1) (+) (f2, v2) = (f1 | f2, f2 ? v2 : v1 (+) v2).
// The pair operator is associative and not commutative.
template <typename V>
struct SegPair {
    uint32_t f;
    V v;
};

template <class Base>
struct OpSeg {
    using elem_t = typename Base::elem_t;
    using bvalue_t = typename Base::value_t;
    using bcarry_t = typename Base::carry_t;
    using value_t = SegPair<bvalue_t>;
    using carry_t = SegPair<bcarry_t>;
    using prep_t = typename Base::prep_t;
    static constexpr int kWords = Base::kWords;
    __device__ __forceinline__ static value_t identity() { return {0u, Base::identity()}; }
    __device__ __forceinline__ static value_t combine(value_t a, value_t b)
    {
        return {a.f | b.f, b.f ? b.v : Base::combine(a.v, b.v)};
    }
    __device__ __forceinline__ static carry_t carry_identity() { return {0u, Base::carry_identity()}; }
    __device__ __forceinline__ static carry_t to_carry(value_t v) { return {v.f, Base::to_carry(v.v)}; }
    __device__ __forceinline__ static carry_t combine_carry(carry_t a, carry_t b)
    {
        return {a.f | b.f, b.f ? b.v : Base::combine_carry(a.v, b.v)};
    }
    // The carry's flag never matters when it is applied: only the local flag does.
    __device__ __forceinline__ static prep_t prepare(carry_t c) { return Base::prepare(c.v); }
    __device__ __forceinline__ static value_t apply(prep_t c, value_t local)
    {
        return {local.f, local.f ? local.v : Base::apply(c, local.v)};
    }
    __device__ __forceinline__ static void pack(carry_t c, uint64_t* w, uint32_t& flag)
    {
        uint32_t unused;
        Base::pack(c.v, w, unused);
        flag = c.f ? 1u : 0u;
    }
    __device__ __forceinline__ static carry_t unpack(const uint64_t* w, uint32_t flag)
    {
        return {flag, Base::unpack(w, 0u)};
    }
};

}  // namespace dwpt
