// ls_api.cpp -- the extern "C" boundary of libscan: validation, sizing, dispatch.
//
// Every check runs on the host before anything is enqueued, so a rejected call
// has no effect and the checks work without a GPU.  See include/libscan.h for
// the contract of each entry point.
#include "../../include/libscan.h"

#include <hip/hip_runtime_api.h>

#include "ls_internal.hpp"

namespace {

bool valid_dtype(ls_dtype t) { return t == LS_INT32 || t == LS_UINT32 || t == LS_FLOAT32; }
bool valid_op(ls_op op) { return op >= LS_SUM && op <= LS_AFFINE; }
// Valid (dtype, op) pairs the library does not define: bitwise operators and
// affine maps on float32, affine maps on int32.
bool op_unsupported(ls_dtype t, ls_op op)
{
    if (t == LS_FLOAT32)
        return op == LS_XOR || op == LS_AND || op == LS_OR || op == LS_AFFINE;
    return op == LS_AFFINE && t != LS_UINT32;
}
bool valid_cmp(ls_cmp c) { return c >= LS_LT && c <= LS_NE; }
bool valid_scheme(ls_scheme c) { return c >= LS_SCHEME_SINGLE_PASS && c <= LS_SCHEME_SINGLE_PASS_DETERMINISTIC; }
bool valid_block_scan(ls_block_scan c) { return c >= LS_BLOCK_WAVE_DPP && c <= LS_BLOCK_BLELLOCH; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) share a byte
bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (na == 0 || nb == 0)
        return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Element counts the kernels can index: tile ids are 32 bits, compaction counts
// 36 bits.
bool size_ok(int64_t n) { return n >= 0 && n <= LS_MAX_N; }
bool compact_size_ok(int64_t n) { return n >= 0 && n <= LS_COMPACT_MAX_N; }

ls_status from_hip(hipError_t e) { return e == hipSuccess ? LS_OK : LS_ERR_HIP; }

ls_status check_ws(const void* ws, size_t ws_bytes, size_t need)
{
    if (ws == nullptr || ws_bytes < need)
        return LS_ERR_WORKSPACE;
    return LS_OK;
}

// noalloc: ws / ws_bytes are ignored and the library's fixed per-device workspace
// is used (looked up once the arguments have passed their checks).
ls_status scan_common(const void* in, void* out, int64_t n, ls_dtype t, ls_op op, void* total,
                      void* ws, size_t ws_bytes, void* stream, bool inclusive, ls_scheme scheme,
                      bool noalloc = false)
{
    if (!size_ok(n) || !valid_dtype(t) || !valid_op(op) || !valid_scheme(scheme))
        return LS_ERR_INVALID_ARG;
    const size_t bytes = size_t(n) * 4;
    if (n > 0) {
        if (in == nullptr || out == nullptr || !aligned(in, 4) || !aligned(out, 4))
            return LS_ERR_INVALID_ARG;
        if (in != out && overlaps(in, bytes, out, bytes))
            return LS_ERR_INVALID_ARG;
    }
    if (total != nullptr) {
        if (!aligned(total, 4) || overlaps(total, 4, in, bytes) || overlaps(total, 4, out, bytes))
            return LS_ERR_INVALID_ARG;
    }
    if (op_unsupported(t, op))
        return LS_ERR_UNSUPPORTED;
    const size_t need = ls::scan_workspace_bytes(n, int(scheme));
    if (noalloc) {
        if (n > LS_SCAN_NOALLOC_MAX_N || need > ls::NOALLOC_SCRATCH_BYTES)
            return LS_ERR_WORKSPACE;
        if (ls::noalloc_scratch(reinterpret_cast<hipStream_t>(stream), &ws) != hipSuccess)
            return LS_ERR_HIP;
        ws_bytes = ls::NOALLOC_SCRATCH_BYTES;
    }
    ls_status st = check_ws(ws, ws_bytes, need);
    if (st != LS_OK)
        return st;
    if (!aligned(ws, 16) || overlaps(ws, need, in, bytes) || overlaps(ws, need, out, bytes) ||
        (total != nullptr && overlaps(ws, need, total, 4)))
        return LS_ERR_INVALID_ARG;
    return from_hip(ls::launch_scan(in, out, n, int(t), int(op), inclusive, total, ws, int(scheme),
                                    reinterpret_cast<hipStream_t>(stream)));
}

// Shared checks of the compaction family.  in may be NULL when has_in is false;
// flags when has_flags is false.
ls_status compact_common(const void* in, const uint8_t* flags, void* out, int64_t* count,
                                int64_t n, ls_dtype t, ls_cmp cmp, uint32_t thr, int src, int pay,
                                void* ws, size_t ws_bytes, void* stream)
{
    const bool has_in = src == 0 || pay == 0;
    const bool has_flags = src == 1;
    if (!compact_size_ok(n) || !valid_dtype(t) || !valid_cmp(cmp) || count == nullptr || !aligned(count, 8))
        return LS_ERR_INVALID_ARG;
    if (pay == 1 && n > int64_t(UINT32_MAX))
        return LS_ERR_INVALID_ARG;
    const size_t bytes = size_t(n) * 4;
    const size_t fbytes = has_flags ? size_t(n) : 0;
    const size_t ibytes = has_in ? bytes : 0;
    if (n > 0) {
        if (out == nullptr || !aligned(out, 4))
            return LS_ERR_INVALID_ARG;
        if (has_in && (in == nullptr || !aligned(in, 4)))
            return LS_ERR_INVALID_ARG;
        if (has_flags && flags == nullptr)
            return LS_ERR_INVALID_ARG;
        if (overlaps(in, ibytes, out, bytes) || overlaps(flags, fbytes, out, bytes))
            return LS_ERR_INVALID_ARG;
    }
    if (overlaps(count, 8, in, ibytes) || overlaps(count, 8, out, bytes) || overlaps(count, 8, flags, fbytes))
        return LS_ERR_INVALID_ARG;
    const size_t need = ls::compact_workspace_bytes(n);
    ls_status st = check_ws(ws, ws_bytes, need);
    if (st != LS_OK)
        return st;
    if (!aligned(ws, 16) || overlaps(ws, need, in, ibytes) || overlaps(ws, need, out, bytes) ||
        overlaps(ws, need, count, 8) || overlaps(ws, need, flags, fbytes))
        return LS_ERR_INVALID_ARG;
    return from_hip(ls::launch_compact_general(has_in ? in : nullptr, flags, out, count, n, int(t), int(cmp),
                                               thr, src, pay, ws, reinterpret_cast<hipStream_t>(stream)));
}

// Shared checks of the segmented scans: head flags (n bytes) when offsets is NULL
// and by_offsets is false, else CSR offsets (nseg + 1 int64, nseg >= 1 when n > 0).
ls_status segmented_common(const void* in, void* out, int64_t n, ls_dtype t, ls_op op, int exclusive,
                           const uint8_t* heads, const int64_t* offsets, int64_t nseg, bool by_offsets,
                           void* total, void* ws, size_t ws_bytes, void* stream)
{
    if (!size_ok(n) || !valid_dtype(t) || !valid_op(op))
        return LS_ERR_INVALID_ARG;
    const size_t bytes = size_t(n) * 4;
    size_t side_bytes = 0;
    const void* side = nullptr;
    if (by_offsets) {
        if (nseg < 0 || nseg > (INT64_MAX / 8) - 1 || (n > 0 && nseg < 1))
            return LS_ERR_INVALID_ARG;
        side = offsets;
        side_bytes = size_t(nseg + 1) * 8;
        if (n > 0 && (offsets == nullptr || !aligned(offsets, 8)))
            return LS_ERR_INVALID_ARG;
    } else {
        side = heads;
        side_bytes = size_t(n);
        if (n > 0 && heads == nullptr)
            return LS_ERR_INVALID_ARG;
    }
    if (n > 0) {
        if (in == nullptr || out == nullptr || !aligned(in, 4) || !aligned(out, 4))
            return LS_ERR_INVALID_ARG;
        if (in != out && overlaps(in, bytes, out, bytes))
            return LS_ERR_INVALID_ARG;
        if (overlaps(side, side_bytes, out, bytes))
            return LS_ERR_INVALID_ARG;
    }
    if (total != nullptr) {
        if (!aligned(total, 4) || overlaps(total, 4, in, bytes) || overlaps(total, 4, out, bytes) ||
            overlaps(total, 4, side, side_bytes))
            return LS_ERR_INVALID_ARG;
    }
    if (op_unsupported(t, op))
        return LS_ERR_UNSUPPORTED;
    const size_t need = ls::segmented_workspace_bytes(n);
    ls_status st = check_ws(ws, ws_bytes, need);
    if (st != LS_OK)
        return st;
    if (!aligned(ws, 16) || overlaps(ws, need, in, bytes) || overlaps(ws, need, out, bytes) ||
        overlaps(ws, need, side, side_bytes) || (total != nullptr && overlaps(ws, need, total, 4)))
        return LS_ERR_INVALID_ARG;
    return from_hip(ls::launch_segmented(in, out, n, int(t), int(op), exclusive != 0,
                                         by_offsets ? nullptr : heads, by_offsets ? offsets : nullptr,
                                         nseg, total, ws, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int ls_abi_version(void) { return LS_ABI_VERSION; }

const char* ls_status_string(ls_status s)
{
    switch (s) {
    case LS_OK: return "LS_OK: success";
    case LS_ERR_INVALID_ARG: return "LS_ERR_INVALID_ARG: invalid argument (size, pointer, alignment, enum or overlap)";
    case LS_ERR_UNSUPPORTED: return "LS_ERR_UNSUPPORTED: operator not defined for this element type";
    case LS_ERR_WORKSPACE: return "LS_ERR_WORKSPACE: workspace missing or too small";
    case LS_ERR_HIP: return "LS_ERR_HIP: the HIP runtime reported an error";
    case LS_ERR_INCOMPLETE:
        return "LS_ERR_INCOMPLETE: a call on this workspace gave up waiting for another tile; its output is "
               "incomplete (re-initialise the workspace)";
    }
    return "unknown libscan status";
}

ls_status ls_workspace_init(void* ws, size_t ws_bytes, void* stream)
{
    if (ws == nullptr || ws_bytes < 256 || ws_bytes % 16 != 0 || !aligned(ws, 16))
        return LS_ERR_INVALID_ARG;
    return from_hip(ls::init_workspace(ws, ws_bytes, reinterpret_cast<hipStream_t>(stream)));
}

ls_status ls_workspace_check(const void* ws, uint32_t* flags, void* stream)
{
    if (ws == nullptr || !aligned(ws, 16))
        return LS_ERR_INVALID_ARG;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t word = 0;
    const char* p = reinterpret_cast<const char*>(ws) + 8;  // the header's error word
    if (hipMemcpyAsync(&word, p, sizeof word, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return LS_ERR_HIP;
    if (flags != nullptr)
        *flags = word;
    return word == 0 ? LS_OK : LS_ERR_INCOMPLETE;
}

ls_status ls_scan_workspace_bytes(int64_t n, ls_dtype t, ls_op op, size_t* bytes)
{
    if (bytes == nullptr || !size_ok(n) || !valid_dtype(t) || !valid_op(op))
        return LS_ERR_INVALID_ARG;
    if (op_unsupported(t, op))
        return LS_ERR_UNSUPPORTED;
    *bytes = ls::scan_workspace_bytes(n, ls::SCHEME_SINGLE_PASS);
    return LS_OK;
}

ls_status ls_scan_ex_workspace_bytes(int64_t n, ls_dtype t, ls_op op, ls_scheme scheme, size_t* bytes)
{
    if (bytes == nullptr || !size_ok(n) || !valid_dtype(t) || !valid_op(op) || !valid_scheme(scheme))
        return LS_ERR_INVALID_ARG;
    if (op_unsupported(t, op))
        return LS_ERR_UNSUPPORTED;
    *bytes = ls::scan_workspace_bytes(n, int(scheme));
    return LS_OK;
}

ls_status scan_inclusive(const void* in, void* out, int64_t n, ls_dtype t, ls_op op, void* total,
                         void* ws, size_t ws_bytes, void* stream)
{
    return scan_common(in, out, n, t, op, total, ws, ws_bytes, stream, true, LS_SCHEME_SINGLE_PASS);
}

ls_status scan_exclusive(const void* in, void* out, int64_t n, ls_dtype t, ls_op op, void* total,
                         void* ws, size_t ws_bytes, void* stream)
{
    return scan_common(in, out, n, t, op, total, ws, ws_bytes, stream, false, LS_SCHEME_SINGLE_PASS);
}

ls_status scan_ex(const void* in, void* out, int64_t n, ls_dtype t, ls_op op, int exclusive,
                  ls_scheme scheme, void* total, void* ws, size_t ws_bytes, void* stream)
{
    return scan_common(in, out, n, t, op, total, ws, ws_bytes, stream, exclusive == 0, scheme);
}

ls_status scan_noalloc(const void* in, void* out, int64_t n, ls_dtype t, ls_op op, int exclusive,
                       void* total, void* stream)
{
    return scan_common(in, out, n, t, op, total, nullptr, 0, stream, exclusive == 0, LS_SCHEME_SINGLE_PASS,
                       true);
}

ls_status ls_compact_workspace_bytes(int64_t n, ls_dtype t, size_t* bytes)
{
    if (bytes == nullptr || !compact_size_ok(n) || !valid_dtype(t))
        return LS_ERR_INVALID_ARG;
    *bytes = ls::compact_workspace_bytes(n);
    return LS_OK;
}

ls_status compact_if(const void* in, void* out, int64_t* count, int64_t n, ls_dtype t, ls_cmp cmp,
                     uint32_t threshold_bits, void* ws, size_t ws_bytes, void* stream)
{
    return compact_common(in, nullptr, out, count, n, t, cmp, threshold_bits, 0, 0, ws, ws_bytes, stream);
}

ls_status compact_flags(const void* in, const uint8_t* flags, void* out, int64_t* count, int64_t n,
                        void* ws, size_t ws_bytes, void* stream)
{
    return compact_common(in, flags, out, count, n, LS_UINT32, LS_LT, 0, 1, 0, ws, ws_bytes, stream);
}

ls_status select_indices_if(const void* in, uint32_t* out_indices, int64_t* count, int64_t n, ls_dtype t,
                            ls_cmp cmp, uint32_t threshold_bits, void* ws, size_t ws_bytes, void* stream)
{
    return compact_common(in, nullptr, out_indices, count, n, t, cmp, threshold_bits, 0, 1, ws, ws_bytes,
                          stream);
}

ls_status select_indices_flags(const uint8_t* flags, uint32_t* out_indices, int64_t* count, int64_t n,
                               void* ws, size_t ws_bytes, void* stream)
{
    return compact_common(nullptr, flags, out_indices, count, n, LS_UINT32, LS_LT, 0, 1, 1, ws, ws_bytes,
                          stream);
}

static ls_status batched_common(const void* in, void* out, int64_t rows, int64_t cols, ls_dtype t,
                                ls_op op, int exclusive, ls_block_scan kind, void* stream)
{
    if (rows < 0 || cols < 0 || !valid_dtype(t) || !valid_op(op) || !valid_block_scan(kind))
        return LS_ERR_INVALID_ARG;
    if (rows > 0 && cols > INT64_MAX / 8 / rows)
        return LS_ERR_INVALID_ARG;
    const int64_t n = rows * cols;
    const size_t bytes = size_t(n) * 4;
    if (n > 0) {
        if (in == nullptr || out == nullptr || !aligned(in, 4) || !aligned(out, 4))
            return LS_ERR_INVALID_ARG;
        if (in != out && overlaps(in, bytes, out, bytes))
            return LS_ERR_INVALID_ARG;
    }
    if (op_unsupported(t, op))
        return LS_ERR_UNSUPPORTED;
    return from_hip(ls::launch_batched(in, out, rows, cols, int(t), int(op), exclusive != 0, int(kind),
                                       reinterpret_cast<hipStream_t>(stream)));
}

ls_status batched_row_scan(const void* in, void* out, int64_t rows, int64_t cols, ls_dtype t,
                           ls_op op, int exclusive, void* stream)
{
    return batched_common(in, out, rows, cols, t, op, exclusive, LS_BLOCK_WAVE_DPP, stream);
}

ls_status batched_row_scan_ex(const void* in, void* out, int64_t rows, int64_t cols, ls_dtype t,
                              ls_op op, int exclusive, ls_block_scan block_scan, void* stream)
{
    return batched_common(in, out, rows, cols, t, op, exclusive, block_scan, stream);
}

ls_status ls_radix_sort_workspace_bytes(int64_t n, ls_dtype t, int with_values, size_t* bytes)
{
    if (bytes == nullptr || n < 0 || n > int64_t(UINT32_MAX) || !valid_dtype(t))
        return LS_ERR_INVALID_ARG;
    *bytes = ls::sort_workspace_bytes(n, with_values != 0);
    return LS_OK;
}

ls_status radix_sort(const void* keys_in, void* keys_out, const void* values_in, void* values_out,
                     int64_t n, ls_dtype t, void* ws, size_t ws_bytes, void* stream)
{
    if (n < 0 || n > int64_t(UINT32_MAX) || !valid_dtype(t))
        return LS_ERR_INVALID_ARG;
    if ((values_in == nullptr) != (values_out == nullptr))
        return LS_ERR_INVALID_ARG;
    const bool vals = values_in != nullptr;
    const size_t bytes = size_t(n) * 4;
    if (n > 0) {
        if (keys_in == nullptr || keys_out == nullptr || !aligned(keys_in, 4) || !aligned(keys_out, 4))
            return LS_ERR_INVALID_ARG;
        if (keys_in != keys_out && overlaps(keys_in, bytes, keys_out, bytes))
            return LS_ERR_INVALID_ARG;
        if (vals) {
            if (!aligned(values_in, 4) || !aligned(values_out, 4))
                return LS_ERR_INVALID_ARG;
            if (values_in != values_out && overlaps(values_in, bytes, values_out, bytes))
                return LS_ERR_INVALID_ARG;
            const void* ks[2] = {keys_in, keys_out};
            const void* vs[2] = {values_in, values_out};
            for (const void* a : ks)
                for (const void* b : vs)
                    if (overlaps(a, bytes, b, bytes))
                        return LS_ERR_INVALID_ARG;
        }
    }
    const size_t need = ls::sort_workspace_bytes(n, vals);
    ls_status st = check_ws(ws, ws_bytes, need);
    if (st != LS_OK)
        return st;
    if (!aligned(ws, 16) || overlaps(ws, need, keys_in, bytes) || overlaps(ws, need, keys_out, bytes) ||
        (vals && (overlaps(ws, need, values_in, bytes) || overlaps(ws, need, values_out, bytes))))
        return LS_ERR_INVALID_ARG;
    return from_hip(ls::launch_sort(keys_in, keys_out, values_in, values_out, n, int(t), ws,
                                    reinterpret_cast<hipStream_t>(stream)));
}

ls_status ls_segmented_workspace_bytes(int64_t n, ls_dtype t, ls_op op, size_t* bytes)
{
    if (bytes == nullptr || !size_ok(n) || !valid_dtype(t) || !valid_op(op))
        return LS_ERR_INVALID_ARG;
    if (op_unsupported(t, op))
        return LS_ERR_UNSUPPORTED;
    *bytes = ls::segmented_workspace_bytes(n);
    return LS_OK;
}

ls_status segmented_scan(const void* in, void* out, int64_t n, ls_dtype t, ls_op op, int exclusive,
                         const uint8_t* heads, void* total, void* ws, size_t ws_bytes, void* stream)
{
    return segmented_common(in, out, n, t, op, exclusive, heads, nullptr, 0, false, total, ws, ws_bytes,
                            stream);
}

ls_status segmented_scan_offsets(const void* in, void* out, int64_t n, ls_dtype t, ls_op op, int exclusive,
                                 const int64_t* offsets, int64_t nseg, void* total, void* ws,
                                 size_t ws_bytes, void* stream)
{
    return segmented_common(in, out, n, t, op, exclusive, nullptr, offsets, nseg, true, total, ws,
                            ws_bytes, stream);
}

}  // extern "C"
