/*
 * oracle.c -- plain, serial CPU reference for prefix scan and stream compaction.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the test-suite, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no source, header, table or constant with the HIP library.
 *
 * Every routine is the textbook definition, evaluated one element after another,
 * in the order the definition states.  No blocking, no reordering, no vectorised
 * tricks: a reader can check each loop against the definitions by eye.
 *
 * Citations name the source page and its section:
 *   [Scan3]  geek-doc.cn, "并行前缀和 scan: Hillis-Steele、Blelloch 与 warp shuffle
 *            三种写法" (parallel prefix scan, three ways); sections 一..五 and the
 *            pitfall list ("常见坑").
 *   [Blog2]  lpnh.cn/news/2866224, parallel scan / prefix sum overview; sections 1..7.
 *   [SIMT3]  pgsm.cn/news/414823, "SIMT数据依赖与并行前缀和：从原理到流压缩实战";
 *            sections 1..5.
 *
 * Codes used below (defined here, independently of the library's header):
 *   dtype: 0 = int32, 1 = uint32, 2 = float32
 *   op:    0 = sum,   1 = max,    2 = xor,  3 = min,  4 = and,  5 = or,
 *          6 = product,  7 = affine-map composition (uint32 only)
 *   cmp:   0 = <, 1 = <=, 2 = >, 3 = >=, 4 = ==, 5 = !=
 * Readings of points the pages leave open (operator identities, integer wrap,
 * tie rule of the float max) are stated at each routine.
 */
#include <stdint.h>
#include <string.h>

#define OR_INT32 0
#define OR_UINT32 1
#define OR_FLOAT32 2

#define OR_SUM 0
#define OR_MAX 1
#define OR_XOR 2
#define OR_MIN 3
#define OR_AND 4
#define OR_OR 5
#define OR_PROD 6
#define OR_AFFINE 7

/* ---- the binary operators ------------------------------------------------
 * [Scan3] §一 (last paragraph) and §三: scan is defined for any associative
 * operator; the default is addition, and max and xor are named examples.
 * Integer addition wraps modulo 2^32 (two's complement), computed on uint32_t so
 * that C has no undefined behaviour; the pages never overflow, so any wrapping
 * rule agrees with them, and this one is what 32-bit hardware addition does. */
/* [Blog2] §3.3 (generic operators) adds to these the product, min and the
 * logical AND / OR; the integer product wraps modulo 2^32 like the sum.
 *
 * Affine-map composition ([Scan3] §三, last paragraph: any associative operator
 * may be scanned, matrix chain products included, and a non-commutative one must
 * keep its left-right order).  A uint32 element (a << 16) | b stands for the map
 * v -> a*v + b (mod 2^16), i.e. the 2x2 matrix [[a, b], [0, 1]] acting on the
 * column (v, 1).  Scanning applies the earlier map first: the element for
 * x[0..i] is M_i * ... * M_1 * M_0, and combining an earlier e = (a1, b1) with a
 * later f = (a2, b2) gives the map v -> a2*(a1*v + b1) + b2, i.e.
 * (a2*a1, a2*b1 + b2), all mod 2^16.  Not commutative, so any slip in the order
 * of a combination shows. */
static uint32_t affine_then(uint32_t earlier, uint32_t later)
{
    uint32_t a1 = earlier >> 16, b1 = earlier & 0xffffu;
    uint32_t a2 = later >> 16, b2 = later & 0xffffu;
    uint32_t a = (a2 * a1) & 0xffffu;
    uint32_t b = (a2 * b1 + b2) & 0xffffu;
    return (a << 16) | b;
}

/* op(earlier, later): the scan's accumulator is always the left operand. */
static uint32_t op_u32(int dtype, int op, uint32_t a, uint32_t b)
{
    switch (op) {
    case OR_SUM:
        return a + b; /* wraps mod 2^32 */
    case OR_XOR:
        return a ^ b;
    case OR_MAX:
        if (dtype == OR_INT32)
            return ((int32_t)a > (int32_t)b) ? a : b;
        return (a > b) ? a : b;
    case OR_MIN:
        if (dtype == OR_INT32)
            return ((int32_t)a < (int32_t)b) ? a : b;
        return (a < b) ? a : b;
    case OR_AND:
        return a & b;
    case OR_OR:
        return a | b;
    case OR_PROD:
        return a * b; /* wraps mod 2^32; the low 32 bits are the same for int32 */
    case OR_AFFINE:
        return affine_then(a, b);
    }
    return 0;
}

/* Identity of each operator: the value an exclusive scan puts in its first cell.
 * [Scan3] §一 fixes z[0] = 0 for addition; for max and xor the same role is
 * played by the operator's identity (0 for xor and or, the smallest value for
 * max, the largest for min, all ones for and, 1 for the product, the identity
 * map for affine maps). */
static uint32_t identity_u32(int dtype, int op)
{
    switch (op) {
    case OR_MAX:
        return dtype == OR_INT32 ? 0x80000000u : 0u; /* smallest value */
    case OR_MIN:
        return dtype == OR_INT32 ? 0x7fffffffu : 0xffffffffu; /* largest value */
    case OR_AND:
        return 0xffffffffu;
    case OR_PROD:
        return 1u;
    case OR_AFFINE:
        return 0x00010000u; /* v -> 1*v + 0 */
    }
    return 0u; /* sum, xor, or */
}

/* ---- integer scans (int32 / uint32; every operator above) -------------------
 * Inclusive: y[i] = x[0] (+) ... (+) x[i]            [Scan3] §一, first formula
 * ((+) is any of the operators above, earlier operand on the left)
 * Exclusive: z[0] = identity, z[i] = x[0] (+) ... (+) x[i-1]   [Scan3] §一
 * Serial evaluation: one accumulator carried left to right, exactly the serial
 * loop of [Scan3] §一 and [Blog2] §2.1.  The total (the value no exclusive cell
 * holds, [Scan3] §一) is written to *total when total != NULL.
 * Returns 0, or -1 on an unknown code. */
int oracle_scan_u32(const uint32_t *x, uint32_t *y, int64_t n, int dtype, int op,
                    int inclusive, uint32_t *total)
{
    if ((dtype != OR_INT32 && dtype != OR_UINT32) || op < OR_SUM || op > OR_AFFINE)
        return -1;
    if (op == OR_AFFINE && dtype != OR_UINT32)
        return -1;
    uint32_t acc = identity_u32(dtype, op);
    if (inclusive) {
        /* y[0] = x[0]; y[i] = y[i-1] (+) x[i] */
        for (int64_t i = 0; i < n; ++i) {
            acc = (i == 0) ? x[0] : op_u32(dtype, op, acc, x[i]);
            y[i] = acc;
        }
    } else {
        /* z[0] = identity; z[i] = z[i-1] (+) x[i-1] */
        for (int64_t i = 0; i < n; ++i) {
            y[i] = acc;
            acc = op_u32(dtype, op, acc, x[i]);
        }
    }
    if (total)
        *total = acc;
    return 0;
}

/* ---- float32 sum, accumulated in double ------------------------------------
 * Same definition as above with real addition.  The accumulator is a double, so
 * the result is the exact prefix up to double rounding.  bound[i] receives
 * sum_{j<=i} |x[j]| (also in double; for the exclusive scan too, i.e. the bound
 * includes x[i]) -- the scale of the float32 tolerance that a parallel order of
 * additions must meet ([Scan3] pitfall list: float addition is not associative,
 * so a parallel result may differ in the last bits).  bound may be NULL. */
void oracle_scan_f32_sum(const float *x, double *y, double *bound, int64_t n, int inclusive,
                         double *total)
{
    double acc = 0.0;
    double mag = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i];
        mag += (v < 0.0) ? -v : v;
        if (inclusive) {
            acc = (i == 0) ? v : acc + v;
            y[i] = acc;
        } else {
            y[i] = acc;
            acc += v;
        }
        if (bound)
            bound[i] = mag;
    }
    if (total)
        *total = acc;
}

/* ---- float32 max ------------------------------------------------------------
 * max(a, b) = (a > b) ? a : b, evaluated in float32.  On a tie (equal values,
 * including -0 against +0) it keeps the right operand, so a prefix holds the
 * right-most of its largest elements; this rule is associative for non-NaN data,
 * hence any association order yields the same bits.  Identity: -infinity.
 * NaN inputs are outside the defined domain. */
static float fmax_right(float a, float b)
{
    return (a > b) ? a : b;
}

void oracle_scan_f32_max(const float *x, float *y, int64_t n, int inclusive, float *total)
{
    uint32_t ninf_bits = 0xff800000u;
    float acc;
    memcpy(&acc, &ninf_bits, sizeof acc);
    for (int64_t i = 0; i < n; ++i) {
        if (inclusive) {
            acc = (i == 0) ? x[0] : fmax_right(acc, x[i]);
            y[i] = acc;
        } else {
            y[i] = acc;
            acc = fmax_right(acc, x[i]);
        }
    }
    if (total)
        *total = acc;
}

/* ---- float32 min ------------------------------------------------------------
 * min(a, b) = (a < b) ? a : b in float32: like the max, a tie (including -0
 * against +0) keeps the right operand, so the rule is associative on non-NaN data
 * and every association order gives the same bits.  Identity: +infinity. */
static float fmin_right(float a, float b)
{
    return (a < b) ? a : b;
}

void oracle_scan_f32_min(const float *x, float *y, int64_t n, int inclusive, float *total)
{
    uint32_t pinf_bits = 0x7f800000u;
    float acc;
    memcpy(&acc, &pinf_bits, sizeof acc);
    for (int64_t i = 0; i < n; ++i) {
        if (inclusive) {
            acc = (i == 0) ? x[0] : fmin_right(acc, x[i]);
            y[i] = acc;
        } else {
            y[i] = acc;
            acc = fmin_right(acc, x[i]);
        }
    }
    if (total)
        *total = acc;
}

/* ---- float32 product, accumulated in double ---------------------------------
 * The running product of the elements ([Blog2] §3.3), carried in a double.  A
 * float32 product of k factors evaluated in any association has a relative error
 * of at most about (k-1) * 2^-24 (one rounding per multiplication), so the
 * double result is the reference and the tolerance is relative. */
void oracle_scan_f32_prod(const float *x, double *y, int64_t n, int inclusive, double *total)
{
    double acc = 1.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i];
        if (inclusive) {
            acc = (i == 0) ? v : acc * v;
            y[i] = acc;
        } else {
            y[i] = acc;
            acc *= v;
        }
    }
    if (total)
        *total = acc;
}

/* ---- the compaction predicate ----------------------------------------------
 * element (cmp) threshold, compared in the element's own type: signed for int32,
 * unsigned for uint32, IEEE float comparison (C semantics) for float32. */
static int pred_holds(int dtype, int cmp, uint32_t vbits, uint32_t tbits)
{
    int lt, eq;
    if (dtype == OR_FLOAT32) {
        float v, t;
        memcpy(&v, &vbits, sizeof v);
        memcpy(&t, &tbits, sizeof t);
        switch (cmp) {
        case 0: return v < t;
        case 1: return v <= t;
        case 2: return v > t;
        case 3: return v >= t;
        case 4: return v == t;
        case 5: return v != t;
        }
        return 0;
    }
    if (dtype == OR_INT32) {
        lt = (int32_t)vbits < (int32_t)tbits;
    } else {
        lt = vbits < tbits;
    }
    eq = vbits == tbits;
    switch (cmp) {
    case 0: return lt;
    case 1: return lt || eq;
    case 2: return !lt && !eq;
    case 3: return !lt;
    case 4: return eq;
    case 5: return !eq;
    }
    return 0;
}

/* ---- stream compaction, serial form -----------------------------------------
 * Keep, in input order, every element whose predicate holds; return how many
 * were kept.  [Scan3] §一 (the 8-element compaction example) and [SIMT3] §4.1
 * (inputs copied to the front of the output, in order, plus a count).
 * out must hold n elements; cells at and beyond the count are not written.
 * Returns the count, or -1 on an unknown code. */
int64_t oracle_compact(const uint32_t *x, uint32_t *out, int64_t n, int dtype, int cmp,
                       uint32_t thr_bits)
{
    if (dtype < OR_INT32 || dtype > OR_FLOAT32 || cmp < 0 || cmp > 5)
        return -1;
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (pred_holds(dtype, cmp, x[i], thr_bits))
            out[c++] = x[i];
    }
    return c;
}

/* ---- stream compaction, flag / exclusive-scan / scatter form ----------------
 * The three steps of [Scan3] §一 and [SIMT3] §4.2: (1) flag[i] = 1 if the
 * predicate holds, else 0; (2) exclusive sum scan of the flags gives each kept
 * element its output index; (3) every kept element writes out[index[i]] = x[i];
 * the count is index[n-1] + flag[n-1].  Computed with its own arrays so that it
 * is an independent check of the serial form above.  flags and index are caller
 * scratch of n elements each.  Returns the count, or -1 on an unknown code. */
int64_t oracle_compact_via_scan(const uint32_t *x, uint32_t *out, int64_t n, int dtype, int cmp,
                                uint32_t thr_bits, int64_t *flags, int64_t *index)
{
    if (dtype < OR_INT32 || dtype > OR_FLOAT32 || cmp < 0 || cmp > 5)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        flags[i] = pred_holds(dtype, cmp, x[i], thr_bits) ? 1 : 0;
    int64_t run = 0;
    for (int64_t i = 0; i < n; ++i) {
        index[i] = run;
        run += flags[i];
    }
    for (int64_t i = 0; i < n; ++i) {
        if (flags[i])
            out[index[i]] = x[i];
    }
    return n > 0 ? index[n - 1] + flags[n - 1] : 0;
}

/* ---- batched row scan -------------------------------------------------------
 * rows x cols, row-major and contiguous; each row is scanned on its own, with no
 * carry from one row into the next: the single-array definition applied to every
 * row.  This is the uniform-length case of the segmented scan that [Blog2] §7.2
 * mentions.  For float32 sum, y/bound are double arrays of rows*cols. */
int oracle_batched_u32(const uint32_t *x, uint32_t *y, int64_t rows, int64_t cols, int dtype,
                       int op, int inclusive)
{
    for (int64_t r = 0; r < rows; ++r) {
        int rc = oracle_scan_u32(x + r * cols, y + r * cols, cols, dtype, op, inclusive, 0);
        if (rc)
            return rc;
    }
    return 0;
}

void oracle_batched_f32_sum(const float *x, double *y, double *bound, int64_t rows, int64_t cols,
                            int inclusive)
{
    for (int64_t r = 0; r < rows; ++r)
        oracle_scan_f32_sum(x + r * cols, y + r * cols, bound ? bound + r * cols : 0, cols,
                            inclusive, 0);
}

void oracle_batched_f32_max(const float *x, float *y, int64_t rows, int64_t cols, int inclusive)
{
    for (int64_t r = 0; r < rows; ++r)
        oracle_scan_f32_max(x + r * cols, y + r * cols, cols, inclusive, 0);
}

void oracle_batched_f32_min(const float *x, float *y, int64_t rows, int64_t cols, int inclusive)
{
    for (int64_t r = 0; r < rows; ++r)
        oracle_scan_f32_min(x + r * cols, y + r * cols, cols, inclusive, 0);
}

void oracle_batched_f32_prod(const float *x, double *y, int64_t rows, int64_t cols, int inclusive)
{
    for (int64_t r = 0; r < rows; ++r)
        oracle_scan_f32_prod(x + r * cols, y + r * cols, cols, inclusive, 0);
}

/* ---- segmented scan ---------------------------------------------------------
 * [Blog2] §7.2 names segmented scans (scans that restart at segment boundaries);
 * read plainly: the array is cut into consecutive segments, each marked by a head
 * flag on its first element (element 0 always starts one), and every segment is
 * scanned on its own with the definitions above, no value crossing a boundary:
 *   inclusive: y[i] = x[i] if i starts a segment, else y[i-1] (+) x[i]
 *   exclusive: z[i] = identity if i starts a segment, else z[i-1] (+) x[i-1]
 * heads[i] != 0 marks a head.  The batched row scan above is the case of a head
 * every cols elements.  Returns 0, or -1 on an unknown code. */
int oracle_segmented_u32(const uint32_t *x, uint32_t *y, const uint8_t *heads, int64_t n,
                         int dtype, int op, int inclusive)
{
    if ((dtype != OR_INT32 && dtype != OR_UINT32) || op < OR_SUM || op > OR_AFFINE)
        return -1;
    if (op == OR_AFFINE && dtype != OR_UINT32)
        return -1;
    uint32_t prev_y = 0, prev_x = 0;
    for (int64_t i = 0; i < n; ++i) {
        int head = (i == 0) || heads[i] != 0;
        if (inclusive)
            y[i] = head ? x[i] : op_u32(dtype, op, prev_y, x[i]);
        else
            y[i] = head ? identity_u32(dtype, op) : op_u32(dtype, op, prev_y, prev_x);
        prev_y = y[i];
        prev_x = x[i];
    }
    return 0;
}

/* float32 sum: double accumulation; bound[i] = sum of |x[j]| over the segment up
 * to and including x[i] (the tolerance scale, as for the plain scan). */
void oracle_segmented_f32_sum(const float *x, double *y, double *bound, const uint8_t *heads,
                              int64_t n, int inclusive)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i];
        if (i == 0 || heads[i] != 0) {
            acc = 0.0;
            mag = 0.0;
        }
        mag += (v < 0.0) ? -v : v;
        if (inclusive) {
            acc += v;
            y[i] = acc;
        } else {
            y[i] = acc;
            acc += v;
        }
        if (bound)
            bound[i] = mag;
    }
}

/* float32 max (is_min == 0) or min (is_min != 0), with the tie rule above (the
 * later element wins) and identity -inf / +inf. */
void oracle_segmented_f32_minmax(const float *x, float *y, const uint8_t *heads, int64_t n,
                                 int inclusive, int is_min)
{
    uint32_t id_bits = is_min ? 0x7f800000u : 0xff800000u;
    float id, acc = 0.0f;
    memcpy(&id, &id_bits, sizeof id);
    for (int64_t i = 0; i < n; ++i) {
        if (i == 0 || heads[i] != 0)
            acc = id;
        if (inclusive) {
            acc = is_min ? fmin_right(acc, x[i]) : fmax_right(acc, x[i]);
            y[i] = acc;
        } else {
            y[i] = acc;
            acc = is_min ? fmin_right(acc, x[i]) : fmax_right(acc, x[i]);
        }
    }
}

/* float32 product in double (relative tolerance, as for the plain product). */
void oracle_segmented_f32_prod(const float *x, double *y, const uint8_t *heads, int64_t n,
                               int inclusive)
{
    double acc = 1.0;
    for (int64_t i = 0; i < n; ++i) {
        if (i == 0 || heads[i] != 0)
            acc = 1.0;
        if (inclusive) {
            acc *= (double)x[i];
            y[i] = acc;
        } else {
            y[i] = acc;
            acc *= (double)x[i];
        }
    }
}

/* Segments given as offsets (the CSR row-offset array that [Scan3] §一 lists among
 * scan's uses): segment k covers [offsets[k], offsets[k+1]); offsets[0] = 0,
 * offsets[nseg] = n, non-decreasing; an empty segment marks nothing.  Writes the
 * equivalent head flags (heads[] must hold n bytes).  Returns 0, or -1 when the
 * offsets break those rules. */
int oracle_heads_from_offsets(const int64_t *offsets, int64_t nseg, uint8_t *heads, int64_t n)
{
    if (nseg < 0 || offsets[0] != 0 || offsets[nseg] != n)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        heads[i] = 0;
    for (int64_t k = 0; k < nseg; ++k) {
        if (offsets[k + 1] < offsets[k])
            return -1;
        if (offsets[k] < n)
            heads[offsets[k]] = 1;
    }
    return 0;
}

/* ---- radix-sort order and stable sort --------------------------------------
 * The radix sort of the pages ([Scan3] 一: each round places keys by the scan of
 * a digit predicate; [Blog2] 4.2: per-digit histograms, their prefix sums, and a
 * reordering) orders keys by their bits once mapped to unsigned integers whose
 * order is the key type's order:
 *   uint32  the key itself
 *   int32   key with the sign bit flipped (two's complement order)
 *   float32 negative (sign set): all bits flipped; else sign bit set.  This is
 *           the IEEE total order: -NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN.
 * The sort is stable: equal keys keep their input order (and so do their values).
 * The oracle sorts by that order with a plain top-down merge sort (stable because
 * ties take the left run first).  tmp_k / tmp_v are caller scratch of n elements. */
uint32_t oracle_sort_order_key(int dtype, uint32_t k)
{
    if (dtype == OR_INT32)
        return k ^ 0x80000000u;
    if (dtype == OR_FLOAT32)
        return (k & 0x80000000u) ? ~k : (k | 0x80000000u);
    return k;
}

static void merge_sort_rec(uint32_t *k, uint32_t *v, uint32_t *tk, uint32_t *tv, int64_t lo,
                           int64_t hi, int dtype, int with_values)
{
    if (hi - lo < 2)
        return;
    int64_t mid = lo + (hi - lo) / 2;
    merge_sort_rec(k, v, tk, tv, lo, mid, dtype, with_values);
    merge_sort_rec(k, v, tk, tv, mid, hi, dtype, with_values);
    int64_t i = lo, j = mid, o = lo;
    while (i < mid || j < hi) {
        int take_left;
        if (i >= mid)
            take_left = 0;
        else if (j >= hi)
            take_left = 1;
        else  /* ties: left first -> stable */
            take_left = oracle_sort_order_key(dtype, k[i]) <= oracle_sort_order_key(dtype, k[j]);
        if (take_left) {
            tk[o] = k[i];
            if (with_values)
                tv[o] = v[i];
            ++i;
        } else {
            tk[o] = k[j];
            if (with_values)
                tv[o] = v[j];
            ++j;
        }
        ++o;
    }
    for (int64_t t = lo; t < hi; ++t) {
        k[t] = tk[t];
        if (with_values)
            v[t] = tv[t];
    }
}

/* Sorts keys (and values, when vals != NULL) in place.  Returns 0, or -1 on a bad code. */
int oracle_stable_sort(uint32_t *keys, uint32_t *vals, int64_t n, int dtype, uint32_t *tmp_k,
                       uint32_t *tmp_v)
{
    if (dtype < OR_INT32 || dtype > OR_FLOAT32)
        return -1;
    merge_sort_rec(keys, vals, tmp_k, tmp_v, 0, n, dtype, vals != 0);
    return 0;
}

/* ---- compaction by a flag array, and index selection --------------------------
 * [SIMT3] 4.1-4.2: the input comes with a validity mask; every element whose flag
 * is set is copied to the output front, in order, and the count is reported.
 * Index selection keeps the positions i instead of the values -- the output index
 * of the compaction's scatter step read the other way round ([Scan3] 一).
 * flags: one byte per element, nonzero = keep.  out holds n elements.
 * Return the count (or -1 on an unknown code). */
int64_t oracle_compact_flags(const uint32_t *x, const uint8_t *flags, uint32_t *out, int64_t n)
{
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (flags[i] != 0)
            out[c++] = x[i];
    }
    return c;
}

int64_t oracle_indices_flags(const uint8_t *flags, uint32_t *out, int64_t n)
{
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (flags[i] != 0)
            out[c++] = (uint32_t)i;
    }
    return c;
}

int64_t oracle_indices_if(const uint32_t *x, uint32_t *out, int64_t n, int dtype, int cmp,
                          uint32_t thr_bits)
{
    if (dtype < OR_INT32 || dtype > OR_FLOAT32 || cmp < 0 || cmp > 5)
        return -1;
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (pred_holds(dtype, cmp, x[i], thr_bits))
            out[c++] = (uint32_t)i;
    }
    return c;
}
