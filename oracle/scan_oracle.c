/*
 * scan_oracle.c -- the plain, sequential CPU oracle for the device-wide
 * prefix scan.  TEST INFRASTRUCTURE ONLY: it is built and called by the
 * tests, by the smoke check and by the CPU-baseline leg of the benchmark,
 * never by the GPU library, and it shares no code, header or table with it.
 *
 * Every routine is the textbook definition written out as one left-to-right
 * loop: no blocking, no reordering, no parallelism.  Floating-point sums are
 * accumulated in double.  Integers wrap modulo 2^32.
 *
 * Pages cited (by title and section):
 *   [L7]    "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
 *           (UIUC ECE408 course notes, runguoli.com)
 *   [YLY]   "CUDA编程并行前缀和扫描详解" (tutorial, m.youleyou.com)
 *   [PMPP9] "第9章并行模式：前缀和 - Scan算法 (Parallel Patterns: Prefix Sum -
 *           Scan Algorithms)" (PMPP chapter 9 notes, bittern.cn)
 *   [ECE408] "UIUC ECE 408 应用并行编程" (course index, runguoli.com)
 *
 * Definitions followed:
 *   inclusive  y[i] = x[0] (+) ... (+) x[i]
 *              [L7 concept 1 "inclusive 与 exclusive"; PMPP9 §9.1; YLY §2.1]
 *   exclusive  y[0] = identity, y[i] = x[0] (+) ... (+) x[i-1]
 *              [L7 concept 1; PMPP9 §9.1; YLY §2.2]
 *   The operator only has to be associative; the order of the operands is
 *   kept, earlier element on the left [L7 concept 1, operator generalisation].
 *   Identities: + -> 0, max -> -inf, min -> +inf [PMPP9 §9.1 identity table];
 *   for 32-bit integers -inf/+inf read as the smallest/largest value of the
 *   type, and the identity of the affine map is (a, b) = (1, 0).
 *   A recurrence out[j] = out[j-1] (+) f(j) is a scan [L7 concept 1]; the
 *   affine recurrence y_i = a_i * y_{i-1} + b_i composes maps
 *   (a2,b2) o (a1,b1) = (a2*a1, a2*b1 + b2), applied after the earlier one.
 *   Stream compaction keeps x > 0 in order, at the positions given by an
 *   exclusive scan of the 0/1 flags [L7 concept 2 "扫描的典型应用";
 *   PMPP9 §9.6 array compaction; YLY §2.2 flag/pos example].
 *   Segmented scan restarts the fold at every head flag [L7 concept 2, radix
 *   sort remark]; index 0 always starts a segment.
 *   Composite and matrix operators [L7 concept 1, operator generalisation,
 *   which names matrix multiplication and a user-defined "(maximum, number
 *   of occurrences)" operator]: (v1,c1) (+) (v2,c2) keeps the larger value
 *   and adds the counts on a tie, empty fold (INT32_MIN, 0); 2x2 and 3x3
 *   matrices multiply with the later factor on the left, empty product the
 *   identity.
 *   CSR row offsets are the exclusive scan of the per-row entry counts.
 *   A radix-sort pass places every key by an exclusive scan of the digit
 *   counts [L7 concept 2, radix sort; PMPP9 §9.6 radix sort], keeping the
 *   input order within a digit; 32-bit keys take four 8-bit passes.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define OP_ADD 0
#define OP_MAX 1
#define OP_MIN 2
#define OP_AND 3 /* bitwise AND and OR [L7 concept 1, operator generalisation]; */
#define OP_OR 4  /* identities: all bits set, no bits set                        */

/* ------------------------------------------------------------------ */
/* int32: add wraps modulo 2^32 (two's complement); max/min as usual.  */
/* ------------------------------------------------------------------ */
static int32_t i32_identity(int op)
{
    if (op == OP_MAX) return INT32_MIN;
    if (op == OP_MIN) return INT32_MAX;
    if (op == OP_AND) return -1; /* all 32 bits set */
    return 0;
}

static int32_t i32_combine(int op, int32_t earlier, int32_t later)
{
    if (op == OP_MAX) return (later > earlier) ? later : earlier;
    if (op == OP_MIN) return (later < earlier) ? later : earlier;
    if (op == OP_AND) return earlier & later;
    if (op == OP_OR) return earlier | later;
    return (int32_t)((uint32_t)earlier + (uint32_t)later);
}

void oracle_scan_i32(int op, int exclusive, const int32_t *x, int32_t *y, int64_t n)
{
    int32_t acc = i32_identity(op);
    for (int64_t i = 0; i < n; ++i) {
        if (exclusive) {
            y[i] = acc;
            acc = i32_combine(op, acc, x[i]);
        } else {
            acc = i32_combine(op, acc, x[i]);
            y[i] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* uint32                                                              */
/* ------------------------------------------------------------------ */
static uint32_t u32_identity(int op)
{
    if (op == OP_MIN || op == OP_AND) return UINT32_MAX;
    return 0; /* add: 0, max: smallest value 0, or: no bits */
}

static uint32_t u32_combine(int op, uint32_t earlier, uint32_t later)
{
    if (op == OP_MAX) return (later > earlier) ? later : earlier;
    if (op == OP_MIN) return (later < earlier) ? later : earlier;
    if (op == OP_AND) return earlier & later;
    if (op == OP_OR) return earlier | later;
    return earlier + later;
}

void oracle_scan_u32(int op, int exclusive, const uint32_t *x, uint32_t *y, int64_t n)
{
    uint32_t acc = u32_identity(op);
    for (int64_t i = 0; i < n; ++i) {
        if (exclusive) {
            y[i] = acc;
            acc = u32_combine(op, acc, x[i]);
        } else {
            acc = u32_combine(op, acc, x[i]);
            y[i] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* float32 add: the reference value is accumulated in double, as the    */
/* pages' CPU references do; s[i] is the matching prefix of |x|, which  */
/* sets the tolerance of a float32 result.                              */
/* ------------------------------------------------------------------ */
void oracle_scan_f32_add(int exclusive, const float *x, double *y, double *s, int64_t n)
{
    double acc = 0.0, abs_acc = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        if (exclusive) {
            y[i] = acc;
            s[i] = abs_acc;
            acc += (double)x[i];
            abs_acc += fabs((double)x[i]);
        } else {
            acc += (double)x[i];
            abs_acc += fabs((double)x[i]);
            y[i] = acc;
            s[i] = abs_acc;
        }
    }
}

/* float32 max/min: a later value replaces the running one only when it is
 * strictly greater (smaller), so the earlier value wins ties (+0 vs -0).  */
void oracle_scan_f32_minmax(int op, int exclusive, const float *x, float *y, int64_t n)
{
    float acc = (op == OP_MAX) ? -INFINITY : INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        float next;
        if (op == OP_MAX) next = (x[i] > acc) ? x[i] : acc;
        else              next = (x[i] < acc) ? x[i] : acc;
        if (exclusive) {
            y[i] = acc;
            acc = next;
        } else {
            acc = next;
            y[i] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Affine-map composition over uint32 pairs stored as (a0,b0,a1,b1,...).  */
/* y_i = a_i * y_{i-1} + b_i with y_{-1} = 0 is the b component; the a    */
/* component is the running product of the multipliers.  All mod 2^32.   */
/* ------------------------------------------------------------------ */
void oracle_scan_affine(int exclusive, const uint32_t *ab, uint32_t *y, int64_t n)
{
    uint32_t A = 1u, B = 0u;
    for (int64_t i = 0; i < n; ++i) {
        uint32_t a = ab[2 * i], b = ab[2 * i + 1];
        if (exclusive) {
            y[2 * i] = A;
            y[2 * i + 1] = B;
        }
        B = a * B + b;
        A = a * A;
        if (!exclusive) {
            y[2 * i] = A;
            y[2 * i + 1] = B;
        }
    }
}

/* ------------------------------------------------------------------ */
/* The "(maximum, number of occurrences)" composite operator that [L7]  */
/* concept 1 names among user-defined scan operators, over pairs stored */
/* as (v0,c0,v1,c1,...) with int32 values and uint32 counts: the fold   */
/* keeps the largest value seen and adds up the counts of the elements  */
/* that carry it (mod 2^32).  The empty fold is (INT32_MIN, 0).          */
/* ------------------------------------------------------------------ */
void oracle_scan_maxcount(int exclusive, const int32_t *vc, int32_t *y, int64_t n)
{
    int32_t M = INT32_MIN;
    uint32_t C = 0u;
    for (int64_t i = 0; i < n; ++i) {
        int32_t v = vc[2 * i];
        uint32_t c = (uint32_t)vc[2 * i + 1];
        if (exclusive) {
            y[2 * i] = M;
            y[2 * i + 1] = (int32_t)C;
        }
        if (v > M) {
            M = v;
            C = c;
        } else if (v == M) {
            C = C + c;
        }
        if (!exclusive) {
            y[2 * i] = M;
            y[2 * i + 1] = (int32_t)C;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Products of 2x2 uint32 matrices (row-major a,b,c,d per element), the */
/* matrix-multiplication operator of [L7] concept 1, mod 2^32: element  */
/* i of an inclusive result is X_i * X_{i-1} * ... * X_0 (the later     */
/* factor on the left, as for affine maps, which are the matrices       */
/* [[a,b],[0,1]]).  The empty product is the identity matrix.           */
/* ------------------------------------------------------------------ */
void oracle_scan_mat2(int exclusive, const uint32_t *x, uint32_t *y, int64_t n)
{
    uint32_t P[4] = {1u, 0u, 0u, 1u};
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t *X = x + 4 * i;
        uint32_t Q[4];
        if (exclusive) {
            y[4 * i + 0] = P[0];
            y[4 * i + 1] = P[1];
            y[4 * i + 2] = P[2];
            y[4 * i + 3] = P[3];
        }
        /* Q = X * P */
        Q[0] = X[0] * P[0] + X[1] * P[2];
        Q[1] = X[0] * P[1] + X[1] * P[3];
        Q[2] = X[2] * P[0] + X[3] * P[2];
        Q[3] = X[2] * P[1] + X[3] * P[3];
        P[0] = Q[0];
        P[1] = Q[1];
        P[2] = Q[2];
        P[3] = Q[3];
        if (!exclusive) {
            y[4 * i + 0] = P[0];
            y[4 * i + 1] = P[1];
            y[4 * i + 2] = P[2];
            y[4 * i + 3] = P[3];
        }
    }
}

/* ------------------------------------------------------------------ */
/* Products of 3x3 uint32 matrices (row-major, 9 words per element),    */
/* the same operator one size up: element i of an inclusive result is  */
/* X_i * X_{i-1} * ... * X_0 mod 2^32, the later factor on the left;    */
/* the empty product is the identity matrix.                            */
/* ------------------------------------------------------------------ */
void oracle_scan_mat3(int exclusive, const uint32_t *x, uint32_t *y, int64_t n)
{
    uint32_t P[9] = {1u, 0u, 0u, 0u, 1u, 0u, 0u, 0u, 1u};
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t *X = x + 9 * i;
        uint32_t Q[9];
        if (exclusive)
            for (int k = 0; k < 9; ++k) y[9 * i + k] = P[k];
        /* Q = X * P: row r of X times column c of P */
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) {
                uint32_t acc = 0u;
                for (int k = 0; k < 3; ++k) acc += X[3 * r + k] * P[3 * k + c];
                Q[3 * r + c] = acc;
            }
        for (int k = 0; k < 9; ++k) P[k] = Q[k];
        if (!exclusive)
            for (int k = 0; k < 9; ++k) y[9 * i + k] = P[k];
    }
}

/* ------------------------------------------------------------------ */
/* CSR row offsets from COO row indices: building the CSR sparse format */
/* is among the uses of a prefix sum that [YLY] lists in its            */
/* introduction, and [ECE408] (L09) gives the layout, rowPtr[N+1].      */
/* Count the entries of every row, then row_ptr = exclusive scan of the */
/* counts, n_rows + 1 values; row_ptr[n_rows] = the entries counted.    */
/* Entries whose row index is n_rows or more are not counted.            */
/* ------------------------------------------------------------------ */
void oracle_csr_offsets(const uint32_t *rows, int64_t nnz, uint32_t n_rows, uint32_t *row_ptr)
{
    for (uint32_t r = 0; r <= n_rows; ++r) row_ptr[r] = 0u;
    for (int64_t i = 0; i < nnz; ++i)
        if (rows[i] < n_rows) row_ptr[rows[i]] += 1u;
    uint32_t acc = 0u;
    for (uint32_t r = 0; r <= n_rows; ++r) {
        uint32_t c = row_ptr[r];
        row_ptr[r] = acc;
        acc += c;
    }
}

/* ------------------------------------------------------------------ */
/* One pass of a radix sort: a stable split of uint32 keys (and their    */
/* values, if any) by the 8-bit digit (key >> shift) & 255.  Radix sort */
/* splits by digit and places every element with a scan of the digit    */
/* histogram [L7 concept 2; PMPP9 §9.6]; 32-bit keys take four passes.  */
/* Written out: count every digit, exclusive scan of the 256 counts,     */
/* then each element in input order to the next free place of its digit.*/
/* ------------------------------------------------------------------ */
void oracle_radix_split(const uint32_t *keys, const uint32_t *vals, int64_t n, uint32_t shift,
                        uint32_t *keys_out, uint32_t *vals_out)
{
    int64_t start[256];
    int64_t count[256];
    for (int d = 0; d < 256; ++d) count[d] = 0;
    for (int64_t i = 0; i < n; ++i) count[(keys[i] >> shift) & 255u] += 1;
    int64_t acc = 0;
    for (int d = 0; d < 256; ++d) {
        start[d] = acc;
        acc += count[d];
    }
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t d = (keys[i] >> shift) & 255u;
        const int64_t at = start[d]++;
        keys_out[at] = keys[i];
        if (vals) vals_out[at] = vals[i];
    }
}

/* ------------------------------------------------------------------ */
/* Segmented scans: head[i] != 0 (or i == 0) starts a new segment; the  */
/* exclusive form puts the identity at every head.                      */
/* ------------------------------------------------------------------ */
void oracle_segscan_i32(int op, int exclusive, const int32_t *x, const uint8_t *head,
                        int32_t *y, int64_t n)
{
    int32_t acc = i32_identity(op);
    for (int64_t i = 0; i < n; ++i) {
        if (i == 0 || head[i]) acc = i32_identity(op);
        if (exclusive) {
            y[i] = acc;
            acc = i32_combine(op, acc, x[i]);
        } else {
            acc = i32_combine(op, acc, x[i]);
            y[i] = acc;
        }
    }
}

void oracle_segscan_u32(int op, int exclusive, const uint32_t *x, const uint8_t *head,
                        uint32_t *y, int64_t n)
{
    uint32_t acc = u32_identity(op);
    for (int64_t i = 0; i < n; ++i) {
        if (i == 0 || head[i]) acc = u32_identity(op);
        if (exclusive) {
            y[i] = acc;
            acc = u32_combine(op, acc, x[i]);
        } else {
            acc = u32_combine(op, acc, x[i]);
            y[i] = acc;
        }
    }
}

void oracle_segscan_f32_add(int exclusive, const float *x, const uint8_t *head,
                            double *y, double *s, int64_t n)
{
    double acc = 0.0, abs_acc = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        if (i == 0 || head[i]) {
            acc = 0.0;
            abs_acc = 0.0;
        }
        if (exclusive) {
            y[i] = acc;
            s[i] = abs_acc;
            acc += (double)x[i];
            abs_acc += fabs((double)x[i]);
        } else {
            acc += (double)x[i];
            abs_acc += fabs((double)x[i]);
            y[i] = acc;
            s[i] = abs_acc;
        }
    }
}

void oracle_segscan_f32_minmax(int op, int exclusive, const float *x, const uint8_t *head,
                               float *y, int64_t n)
{
    const float ident = (op == OP_MAX) ? -INFINITY : INFINITY;
    float acc = ident;
    for (int64_t i = 0; i < n; ++i) {
        float next;
        if (i == 0 || head[i]) acc = ident;
        if (op == OP_MAX) next = (x[i] > acc) ? x[i] : acc;
        else              next = (x[i] < acc) ? x[i] : acc;
        if (exclusive) {
            y[i] = acc;
            acc = next;
        } else {
            acc = next;
            y[i] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Stream compaction, predicate x > 0.  pos[i] is the exclusive scan of  */
/* the 0/1 flags (the write index of element i when it is kept); kept    */
/* elements go to out[pos[i]] in input order; returns the count.         */
/* ------------------------------------------------------------------ */
int64_t oracle_compact_i32(const int32_t *x, int32_t *out, uint32_t *pos, int64_t n)
{
    uint32_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        pos[i] = c;
        if (x[i] > 0) out[c++] = x[i];
    }
    return (int64_t)c;
}

int64_t oracle_compact_u32(const uint32_t *x, uint32_t *out, uint32_t *pos, int64_t n)
{
    uint32_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        pos[i] = c;
        if (x[i] > 0u) out[c++] = x[i];
    }
    return (int64_t)c;
}

int64_t oracle_compact_f32(const float *x, float *out, uint32_t *pos, int64_t n)
{
    uint32_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        pos[i] = c;
        if (x[i] > 0.0f) out[c++] = x[i];
    }
    return (int64_t)c;
}
