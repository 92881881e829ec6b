/*
 * libscan.h -- device-wide prefix scan and stream compaction for AMD MI355X (gfx950).
 *
 * C ABI: plain pointers and sizes, no C++ or framework types.  Unless marked
 * "host", every pointer is a device pointer (memory from hipMalloc or an
 * allocator built on it) on the device that is current when the call is made.
 *
 * Sources of the operations (page title and section):
 *   [Scan3]  geek-doc.cn, "并行前缀和 scan: Hillis-Steele、Blelloch 与 warp shuffle
 *            三种写法": section 一 (inclusive and exclusive scan, the total, and
 *            compaction by an exclusive scan of predicate flags), 四 (scans larger
 *            than one block), 五 (warp-level scan), pitfall list.
 *   [Blog2]  lpnh.cn/news/2866224, parallel scan overview: section 3.3 (a generic
 *            parallel_scan(in, out, n, op) over any associative operator), 4.1
 *            (compaction: flags, scan, scatter), 5.3 (work issued on streams),
 *            7.2 (segmented scans).
 *   [SIMT3]  pgsm.cn/news/414823, "SIMT数据依赖与并行前缀和：从原理到流压缩实战":
 *            section 4.2 (compaction writes the kept elements in order and a count
 *            computed on the device).
 *
 * Common rules for every entry point
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t passed
 *     as void*; NULL = the null stream) and the call returns without waiting.
 *     Faults during execution surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     non-LS_OK status nothing has been enqueued and no output is written.
 *   - The caller owns every buffer.  The library allocates and frees nothing
 *     and never synchronises.
 *   - Element buffers must be 4-byte aligned.  16-byte alignment of `in` and
 *     `out` enables 128-bit loads and stores; other alignments are accepted and
 *     run a slower path.
 *   - Concurrent calls must use distinct workspaces; calls that share a
 *     workspace on different streams race.
 *
 * Workspaces
 *   The scans, segmented scans, compactions and the radix sort take a caller's
 *   device workspace of at least the size that the matching *_workspace_bytes
 *   query returns.  Inside a call, tiles hand their results on through tile
 *   status words in the workspace ([Scan3] 四: blocks passing their totals on
 *   through flags in global memory; [SIMT3] 5.1: flags published with fences).
 *   - Status workspaces, of the single-pass scans (scan_inclusive,
 *     scan_exclusive, scan_ex with a single-pass scheme), segmented scans and
 *     compactions: zero-filled once before first use, by ls_workspace_init (or
 *     any zero fill of the whole buffer).  Every call leaves the workspace ready
 *     for the next, so calls enqueue no clearing work of their own.  Between
 *     calls its contents must not change, and it must serve no other purpose: a
 *     status workspace used by a radix sort or a three-phase scan_ex, or written
 *     in any other way, must be initialised again.  Apart from that it may serve
 *     any sequence of these calls, of any sizes it is large enough for, up to
 *     2^26 calls: the words carry the call's epoch, compared modulo 2^26, so
 *     initialise it again before that many calls (the Python binding does so
 *     every 2^25).
 *   - The radix sort and the three-phase scan_ex schemes use their workspace as
 *     plain scratch: its contents on entry do not matter.  (For the sort's error
 *     word to be meaningful, initialise its workspace once.)
 *   Each wait for another tile is bounded in time.  The single-pass scans
 *   (except the deterministic scheme) and the compactions take tiles by block
 *   index: a tile that has waited about a millisecond computes what it waited
 *   for from the input itself, and the result stays exact.  The deterministic
 *   scan and the segmented scans take tile ids in the order blocks start: a
 *   wait there gives up after about one second, the call's output is then
 *   incomplete, and the workspace records the fact; so does a call whose last
 *   tile waits more than about ten seconds for the other blocks to start.
 *   ls_workspace_check reports it.  In a correct run no wait lasts more than
 *   microseconds.
 */
#ifndef LIBSCAN_H
#define LIBSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LS_ABI_VERSION 5

/* Largest element count of the scans, segmented scans and the radix sort (tile ids
 * are 32 bits), and of the compaction family (its counts travel in 36 bits). */
#define LS_MAX_N (1LL << 40)
#define LS_COMPACT_MAX_N ((1LL << 36) - 1)

typedef enum ls_status {
    LS_OK = 0,
    LS_ERR_INVALID_ARG = 1, /* bad size, NULL, alignment, enum value, or overlap */
    LS_ERR_UNSUPPORTED = 2, /* an operator not defined for the element type (see ls_op) */
    LS_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the size query returned */
    LS_ERR_HIP = 4,         /* the HIP runtime reported an error when enqueuing */
    LS_ERR_INCOMPLETE = 5   /* ls_workspace_check: a call on the workspace gave up a wait */
} ls_status;

/* Element types.  All are 32 bits wide. */
typedef enum ls_dtype { LS_INT32 = 0, LS_UINT32 = 1, LS_FLOAT32 = 2 } ls_dtype;

/* Associative operators ([Scan3] 一 and 三; [Blog2] 3.3), combined as
 * op(earlier, later), left to right.
 *   LS_SUM     int32/uint32: addition modulo 2^32 (two's complement wrap);
 *              float32: IEEE addition; association order is the library's, so
 *              results may differ from a serial sum in the last bits ([Scan3]
 *              pitfall list).  The order depends only on n and the scheme, so
 *              they are the same bits on every run.
 *   LS_MAX     int32 signed, uint32 unsigned, float32 (a > b) ? a : b, which on a
 *              tie keeps the later element; bit-exact and run-to-run identical
 *              for data without NaN.  NaN inputs give unspecified results.
 *   LS_XOR     int32/uint32 bitwise; float32 -> LS_ERR_UNSUPPORTED.
 *   LS_MIN     as LS_MAX with (a < b) ? a : b (ties keep the later element).
 *   LS_AND, LS_OR  int32/uint32 bitwise ([Blog2] 3.3: logical AND/OR);
 *              float32 -> LS_ERR_UNSUPPORTED.
 *   LS_PROD    int32/uint32: multiplication modulo 2^32; float32: IEEE product
 *              (relative error up to about (i+1) * 2^-24 at element i, any
 *              association; [Blog2] 3.3).
 *   LS_AFFINE  uint32 only: element (a << 16) | b is the map v -> a*v + b mod
 *              2^16 (the 2x2 matrix [[a, b], [0, 1]]); the scan composes the maps,
 *              earlier applied first.  Not commutative, so it shows that results
 *              keep their left-right order ([Scan3] 三, matrix chain products).
 *              int32/float32 -> LS_ERR_UNSUPPORTED.
 * Identity (first exclusive cell, value for n = 0): 0 for sum, xor and or
 * (+0.0f for float32); INT32_MIN / 0u / -infinity for max; INT32_MAX /
 * 0xFFFFFFFF / +infinity for min; all ones for and; 1 (1.0f) for prod; the
 * identity map 0x00010000 for affine. */
typedef enum ls_op {
    LS_SUM = 0,
    LS_MAX = 1,
    LS_XOR = 2,
    LS_MIN = 3,
    LS_AND = 4,
    LS_OR = 5,
    LS_PROD = 6,
    LS_AFFINE = 7
} ls_op;

/* Compaction predicates: keep x when (x CMP threshold), compared in the element
 * type (signed, unsigned, or IEEE float with C semantics: NaN satisfies only NE). */
typedef enum ls_cmp { LS_LT = 0, LS_LE = 1, LS_GT = 2, LS_GE = 3, LS_EQ = 4, LS_NE = 5 } ls_cmp;

/* Device-wide schemes for scan_ex (the default entry points use the single pass).
 *   LS_SCHEME_SINGLE_PASS          one launch; each tile publishes its total, one
 *                                  resident wave turns the published totals into
 *                                  full prefixes in tile order, and each tile reads
 *                                  its predecessor's (the in-kernel hand-off through
 *                                  flags in global memory that [Scan3] 四 mentions;
 *                                  [SIMT3] 5.1).  Moves 2*n*4 bytes.
 *   LS_SCHEME_REDUCE_THEN_SCAN     tile totals, a scan of the totals, a seeded tile
 *                                  scan: three launches, 3*n*4 bytes ([Scan3] 四).
 *   LS_SCHEME_SCAN_THEN_PROPAGATE  tile scans with totals, a scan of the totals, an
 *                                  offset pass over the output: 4*n*4 bytes
 *                                  ([Scan3] 四, the three kernels as listed there).
 *   LS_SCHEME_SINGLE_PASS_DETERMINISTIC  the single pass with a fixed order of
 *                                  combination: tiles form groups of 64, the last
 *                                  tile of a group publishes a full prefix, and a
 *                                  tile combines it with its group's earlier totals
 *                                  in a fixed order.  Float sums and products are
 *                                  then the same bits on every run ([Scan3]
 *                                  pitfall list: a reproducible float result needs
 *                                  a fixed order).  Moves 2*n*4 bytes.
 * The three-phase schemes scan the tile totals recursively when they exceed one
 * tile, as [Scan3] 四 describes for very large arrays.  Their order of combination
 * depends only on n, so they too give the same bits on every run.  So does
 * LS_SCHEME_SINGLE_PASS: its resident wave combines the tile totals in groups of
 * 64 tiles aligned to tile 0, in an order fixed by the tile index. */
typedef enum ls_scheme {
    LS_SCHEME_SINGLE_PASS = 0,
    LS_SCHEME_REDUCE_THEN_SCAN = 1,
    LS_SCHEME_SCAN_THEN_PROPAGATE = 2,
    LS_SCHEME_SINGLE_PASS_DETERMINISTIC = 3
} ls_scheme;

/* Block-level scan used by batched_row_scan_ex for rows of more than 64 elements
 * (one block of 256 threads per row, 4 elements per thread per 1024-element chunk).
 *   LS_BLOCK_WAVE_DPP               64-lane DPP scans, wave totals through LDS, one
 *                                   barrier ([Scan3] 五, the two-level block scan)
 *   LS_BLOCK_HILLIS_STEELE          LDS Hillis-Steele, read / barrier / write /
 *                                   barrier per step ([Scan3] 二)
 *   LS_BLOCK_HILLIS_STEELE_DOUBLE   LDS Hillis-Steele with two buffers, one barrier
 *                                   per step ([Scan3] 二)
 *   LS_BLOCK_BLELLOCH               LDS up-sweep / down-sweep with padded indices
 *                                   ([Scan3] 三; [SIMT3] 5.4)
 * All four give identical results for integers and for max. */
typedef enum ls_block_scan {
    LS_BLOCK_WAVE_DPP = 0,
    LS_BLOCK_HILLIS_STEELE = 1,
    LS_BLOCK_HILLIS_STEELE_DOUBLE = 2,
    LS_BLOCK_BLELLOCH = 3
} ls_block_scan;

/* Returns LS_ABI_VERSION of the loaded library. */
int ls_abi_version(void);

/* A static, human-readable string for a status code (never NULL). */
const char *ls_status_string(ls_status s);

/* Zero-fills a workspace before its first use (or after ls_workspace_check
 * reported LS_ERR_INCOMPLETE): a fill kernel enqueued on `stream` (so the call
 * may be captured in a graph).
 *   ws        device workspace, 16-byte aligned.
 *   ws_bytes  its size: at least 256 and a multiple of 16.
 * Errors: LS_ERR_INVALID_ARG for NULL, misaligned or too small a workspace or a
 * size that is not a multiple of 16; LS_ERR_HIP when the launch fails. */
ls_status ls_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Reports whether a call on this workspace gave up a bounded wait since the
 * workspace was last initialised.  Unlike the other entry points this call
 * waits: it copies the workspace's error word to the host on `stream` and
 * synchronises the stream.
 *   flags (host, out, nullable): the error bits (1 = a wait gave up; 2 = a tile id
 *         beyond the call's tiles was handed out, i.e. the workspace was not
 *         initialised or calls sharing it overlapped).
 * Returns LS_OK when no bit is set, LS_ERR_INCOMPLETE when one is (the outputs of
 * the calls since the last initialisation may be incomplete; initialise the
 * workspace again before further use), LS_ERR_INVALID_ARG for a NULL or
 * misaligned ws, LS_ERR_HIP when the copy fails. */
ls_status ls_workspace_check(const void *ws, uint32_t *flags, void *stream);

/* Workspace size for scan_inclusive / scan_exclusive.
 *   bytes (host, out): size of the device workspace a call with these arguments
 *   needs (never 0).  Errors: LS_ERR_INVALID_ARG for n < 0, bytes == NULL or an
 *   unknown enum; LS_ERR_UNSUPPORTED for an operator not defined on t (see ls_op). */
ls_status ls_scan_workspace_bytes(int64_t n, ls_dtype t, ls_op op, size_t *bytes);

/* Inclusive scan: out[i] = in[0] (+) in[1] (+) ... (+) in[i].     [Scan3] 一
 * Exclusive scan: out[0] = identity, out[i] = in[0] (+) ... (+) in[i-1].
 *
 *   in, out   n elements of type t.  out == in (exact aliasing, in place) is
 *             allowed; any other overlap is LS_ERR_INVALID_ARG.
 *   n         element count, 0 <= n <= LS_MAX_N.  n == 0 writes only *total
 *             (= identity).
 *   t, op     element type and operator (see ls_op).
 *   total     nullable; receives one element: the reduction of all n inputs,
 *             i.e. the value that no exclusive cell holds ([Scan3] 一).
 *   ws        device workspace of ws_bytes >= ls_scan_workspace_bytes(...),
 *             16-byte aligned (else LS_ERR_INVALID_ARG), not overlapping any
 *             other argument, zero-filled before its first use (see
 *             "Workspaces" above).
 *   stream    hipStream_t as void*, or NULL.
 * One pass over the data: each element is read once and written once. */
ls_status scan_inclusive(const void *in, void *out, int64_t n, ls_dtype t, ls_op op, void *total,
                         void *ws, size_t ws_bytes, void *stream);
ls_status scan_exclusive(const void *in, void *out, int64_t n, ls_dtype t, ls_op op, void *total,
                         void *ws, size_t ws_bytes, void *stream);

/* Workspace size for scan_ex with the given scheme (rules as above). */
ls_status ls_scan_ex_workspace_bytes(int64_t n, ls_dtype t, ls_op op, ls_scheme scheme,
                                     size_t *bytes);

/* scan_inclusive / scan_exclusive with an explicit device-wide scheme.
 *   exclusive  nonzero: exclusive scan; zero: inclusive.
 *   scheme     see ls_scheme; an unknown value is LS_ERR_INVALID_ARG.
 *   ws         at least ls_scan_ex_workspace_bytes(n, t, op, scheme) bytes.
 * Other arguments, results and errors as for scan_inclusive. */
ls_status scan_ex(const void *in, void *out, int64_t n, ls_dtype t, ls_op op, int exclusive,
                  ls_scheme scheme, void *total, void *ws, size_t ws_bytes, void *stream);

/* Largest n that scan_noalloc accepts. */
#define LS_SCAN_NOALLOC_MAX_N 402653184LL

/* scan_inclusive / scan_exclusive for callers that cannot allocate device memory
 * at the point of the call: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace: the library keeps a
 * fixed 8 MiB array in device memory per GPU (held until the process ends) and
 * uses it as the single-pass scan's workspace; the call itself allocates and frees
 * nothing.  The first call on a device looks the array up and enqueues its zero
 * fill on `stream` ahead of the scan; every 2^25-th call after that enqueues the
 * fill again (the array's status words compare epochs modulo 2^26).
 *   exclusive  nonzero: exclusive scan; zero: inclusive.
 *   n          0 <= n <= LS_SCAN_NOALLOC_MAX_N; a larger n returns
 *              LS_ERR_WORKSPACE and enqueues nothing.
 * Other arguments, results and errors as for scan_inclusive / scan_exclusive.
 * Every call on one GPU shares that GPU's array: calls whose execution may
 * overlap on one GPU (on different streams without an ordering between them, or
 * from several host threads) race and give wrong results.  Calls on one stream,
 * or ordered by events, are safe. */
ls_status scan_noalloc(const void *in, void *out, int64_t n, ls_dtype t, ls_op op, int exclusive,
                       void *total, void *stream);

/* Workspace size for compact_if (same rules as ls_scan_workspace_bytes). */
ls_status ls_compact_workspace_bytes(int64_t n, ls_dtype t, size_t *bytes);

/* Stable stream compaction ([Scan3] 一; [Blog2] 4.1; [SIMT3] 4.2):
 * every in[i] with (in[i] CMP threshold) is copied to out, in input order, and
 * the number kept is written to *count on the device.
 *
 *   in             n elements of type t.
 *   out            capacity n elements; must not overlap `in`.  Cells at index
 *                  >= *count are not written.
 *   n              0 <= n <= LS_COMPACT_MAX_N.
 *   count          device int64_t, written with the number of kept elements
 *                  (0 when n == 0).  Must not overlap in/out.
 *   threshold_bits the 32-bit pattern of the threshold in type t.
 *   ws, ws_bytes   as for the scans (ls_compact_workspace_bytes).
 * Uses no atomics on the data path; each element is read once and each kept
 * element written once. */
ls_status compact_if(const void *in, void *out, int64_t *count, int64_t n, ls_dtype t, ls_cmp cmp,
                     uint32_t threshold_bits, void *ws, size_t ws_bytes, void *stream);

/* Stable compaction by a flag array ([SIMT3] 4.1-4.2: the input comes with a
 * per-element validity mask; kept elements go to the front of the output in
 * order and the count is computed on the device).
 *   in, out   n 32-bit elements (any type; bits are copied); must not overlap.
 *   flags     n bytes, nonzero = keep; any alignment; must not overlap out.
 *   count     device int64_t, written with the number kept.
 *   ws        >= ls_compact_workspace_bytes(n, LS_UINT32, ...) bytes.
 * Cells of out at index >= *count are not written. */
ls_status compact_flags(const void *in, const uint8_t *flags, void *out, int64_t *count, int64_t n,
                        void *ws, size_t ws_bytes, void *stream);

/* Index selection: the positions i (uint32, ascending) of the elements that
 * compact_if would keep, i.e. the output index of the compaction's scatter
 * read the other way round ([Scan3] 一).  n < 2^32.  Other arguments as for
 * compact_if; out_indices holds n uint32 and must not overlap in. */
ls_status select_indices_if(const void *in, uint32_t *out_indices, int64_t *count, int64_t n,
                            ls_dtype t, ls_cmp cmp, uint32_t threshold_bits, void *ws,
                            size_t ws_bytes, void *stream);

/* The positions i (uint32, ascending) with flags[i] != 0.  n < 2^32. */
ls_status select_indices_flags(const uint8_t *flags, uint32_t *out_indices, int64_t *count,
                               int64_t n, void *ws, size_t ws_bytes, void *stream);

/* Row-wise scan of a rows x cols row-major, contiguous matrix: each row is
 * scanned on its own, with no carry between rows (the uniform-length case of a
 * segmented scan, [Blog2] 7.2).
 *
 *   in, out    rows*cols elements; out == in allowed, other overlap is not.
 *   rows, cols >= 0; either being 0 is a no-op returning LS_OK.
 *   exclusive  nonzero: exclusive scan per row, zero: inclusive.
 * Needs no workspace. */
ls_status batched_row_scan(const void *in, void *out, int64_t rows, int64_t cols, ls_dtype t,
                           ls_op op, int exclusive, void *stream);

/* batched_row_scan with an explicit block-level scan for the one-block-per-row
 * path (see ls_block_scan); with LS_BLOCK_WAVE_DPP it is batched_row_scan.  Other
 * kinds run rows of any length through that path.  An unknown kind is
 * LS_ERR_INVALID_ARG. */
ls_status batched_row_scan_ex(const void *in, void *out, int64_t rows, int64_t cols, ls_dtype t,
                              ls_op op, int exclusive, ls_block_scan block_scan, void *stream);

/* Workspace size for radix_sort (with_values: nonzero when values are sorted
 * along).  Errors: LS_ERR_INVALID_ARG for n < 0, n >= 2^32, bytes == NULL or an
 * unknown dtype. */
ls_status ls_radix_sort_workspace_bytes(int64_t n, ls_dtype t, int with_values, size_t *bytes);

/* Stable ascending radix sort of 32-bit keys, optionally carrying 32-bit values.
 * The pages' scan application ([Scan3] 一: each pass places keys by the scan of
 * a digit predicate, one group offset by the size of the others; [Blog2] 4.2:
 * per-digit histograms, their prefix sums, a reordering).
 *   keys_in, keys_out      n elements of type t.  keys_out == keys_in (in place)
 *                          is allowed; other overlap is LS_ERR_INVALID_ARG.
 *   values_in, values_out  both NULL (keys only) or both non-NULL: n 32-bit
 *                          values moved with their keys; values_out ==
 *                          values_in allowed.  One NULL and one not is
 *                          LS_ERR_INVALID_ARG.
 *   n                      0 <= n < 2^32.
 *   t                      key order: int32 signed, uint32 unsigned, float32
 *                          IEEE total order (-NaN < -inf < ... < -0 < +0 < ...
 *                          < +inf < +NaN, by bit pattern within NaNs).
 *   ws                     >= ls_radix_sort_workspace_bytes(n, t, values != NULL)
 *                          bytes, 16-byte aligned, overlapping no other buffer.
 * Equal keys keep their input order (the sort is stable), so the result,
 * values included, is unique.  Four passes of 8-bit digits; each reads the keys
 * twice and writes them once. */
ls_status radix_sort(const void *keys_in, void *keys_out, const void *values_in, void *values_out,
                     int64_t n, ls_dtype t, void *ws, size_t ws_bytes, void *stream);

/* Workspace size for segmented_scan / segmented_scan_offsets.  Errors as for
 * ls_scan_workspace_bytes. */
ls_status ls_segmented_workspace_bytes(int64_t n, ls_dtype t, ls_op op, size_t *bytes);

/* Segmented scan: the array is cut into consecutive segments and each segment is
 * scanned on its own, no value crossing a boundary ([Blog2] 7.2; the uniform
 * case is batched_row_scan).
 *   in, out    n elements; out == in allowed, other overlap is not.
 *   heads      n bytes; heads[i] != 0 marks the first element of a segment.
 *              Element 0 always starts one.  Any alignment.
 *   exclusive  nonzero: out[i] = identity where a segment starts, else the
 *              operator over the segment's elements before i; zero: inclusive.
 *   total      NULL or 1 element: the inclusive value of element n-1 (the last
 *              segment's reduction); the identity for n == 0.
 *   ws         >= ls_segmented_workspace_bytes(n, t, op) bytes, 16-byte aligned.
 * Operators, identities and float32 behaviour as for scan_inclusive (the same
 * bits on every run for the same input).  Errors: LS_ERR_INVALID_ARG for n <
 * 0, NULL or misaligned buffers with n > 0, overlap (heads or total with out,
 * ws with anything), unknown enums; LS_ERR_UNSUPPORTED and LS_ERR_WORKSPACE as
 * for scan_inclusive. */
ls_status segmented_scan(const void *in, void *out, int64_t n, ls_dtype t, ls_op op, int exclusive,
                         const uint8_t *heads, void *total, void *ws, size_t ws_bytes, void *stream);

/* Segmented scan with segments given as CSR offsets (the row-offset array of a
 * sparse matrix, one of scan's uses in [Scan3] 一): segment k is
 * [offsets[k], offsets[k+1]).
 *   offsets  nseg + 1 int64 (8-byte aligned), offsets[0] == 0, non-decreasing,
 *            offsets[nseg] == n; empty segments are allowed.  The kernel reads
 *            offsets[0 .. nseg-1]; offsets that break these rules give
 *            unspecified results but no access outside the buffers.
 *   nseg     >= 1 when n > 0.
 * Other arguments as for segmented_scan. */
ls_status segmented_scan_offsets(const void *in, void *out, int64_t n, ls_dtype t, ls_op op,
                                 int exclusive, const int64_t *offsets, int64_t nseg, void *total,
                                 void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSCAN_H */
