// ls_internal.hpp -- launchers shared between the kernel files and the C ABI layer.
// Host-side C++ only; the public interface is include/libscan.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace ls {

// Element-type and operator codes (the values of ls_dtype / ls_op / ls_cmp).
enum Dtype : int { DT_INT32 = 0, DT_UINT32 = 1, DT_FLOAT32 = 2 };
enum OpCode : int {
    OP_SUM = 0, OP_MAX = 1, OP_XOR = 2, OP_MIN = 3, OP_AND = 4, OP_OR = 5, OP_PROD = 6, OP_AFFINE = 7
};
// Device-wide schemes (the values of ls_scheme).
enum Scheme : int {
    SCHEME_SINGLE_PASS = 0, SCHEME_REDUCE_THEN_SCAN = 1, SCHEME_SCAN_THEN_PROPAGATE = 2,
    SCHEME_SINGLE_PASS_FIXED = 3
};

// ---- single-pass device-wide scan (ls_scan.hip)
// Zero fill of a workspace of `bytes` bytes (16-byte multiple; the last bytes of
// any other size are left alone), enqueued on `stream`.
hipError_t init_workspace(void* ws, size_t bytes, hipStream_t stream);
int64_t scan_tile_elems();
size_t scan_workspace_bytes(int64_t n, int scheme);
hipError_t launch_scan(const void* in, void* out, int64_t n, int dtype, int op, bool inclusive,
                       void* total, void* ws, int scheme, hipStream_t stream);
// Single-pass exclusive uint32 sum (n >= 1) on a workspace of
// scan_workspace_bytes(n, SCHEME_SINGLE_PASS) bytes whose header and first
// scan_sum_u32_tiles(n) status words are zero (the radix sort zeroes them inside
// its histogram kernel).
int64_t scan_sum_u32_tiles(int64_t n);
hipError_t launch_scan_sum_u32_excl(const uint32_t* in, uint32_t* out, int64_t n, void* ws, hipStream_t stream);

// ---- the scan's fixed per-device workspace (ls_noalloc.hip)
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(8) << 20;
// Device address of the current device's scratch array (NOALLOC_SCRATCH_BYTES);
// the first call on a device enqueues its zero fill on `stream`.
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

// ---- fused compaction (ls_compact.hip)
int64_t compact_tile_elems();
size_t compact_workspace_bytes(int64_t n);
hipError_t launch_compact(const void* in, void* out, int64_t* count, int64_t n, int dtype, int cmp,
                          uint32_t threshold_bits, void* ws, hipStream_t stream);
// src: 0 = predicate (x CMP threshold), 1 = flag bytes; pay: 0 = values, 1 = uint32 indices
hipError_t launch_compact_general(const void* in, const uint8_t* flags, void* out, int64_t* count,
                                  int64_t n, int dtype, int cmp, uint32_t threshold_bits, int src,
                                  int pay, void* ws, hipStream_t stream);

// ---- batched row scan (ls_batched.hip)
// kind: the block-level scan (ls_block_scan values); 0 = wave DPP, the default.
hipError_t launch_batched(const void* in, void* out, int64_t rows, int64_t cols, int dtype, int op,
                          bool exclusive, int kind, hipStream_t stream);

// ---- radix sort (ls_sort.hip)
size_t sort_workspace_bytes(int64_t n, bool with_values);
hipError_t launch_sort(const void* keys_in, void* keys_out, const void* vals_in, void* vals_out,
                       int64_t n, int dtype, void* ws, hipStream_t stream);

// ---- segmented scan (ls_segmented.hip)
size_t segmented_workspace_bytes(int64_t n);
// heads (byte flags) or offsets (nseg + 1 int64, CSR); exactly one is non-null
hipError_t launch_segmented(const void* in, void* out, int64_t n, int dtype, int op, bool excl,
                            const uint8_t* heads, const int64_t* offsets, int64_t nseg, void* total,
                            void* ws, hipStream_t stream);

}  // namespace ls
