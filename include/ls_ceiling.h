/*
 * ls_ceiling.h -- measurement kernels (libls_ceiling.so), not part of libscan.
 *
 * Plain streaming kernels that give the practical HBM ceilings on the GPU they
 * run on: what a kernel that only reads, only writes, or copies the same number of
 * bytes reaches.  The benchmark times them beside the scan (whose minimum traffic
 * is a copy: every element read once and written once) and the compaction (a read
 * of the input plus a write of the kept elements).  They compute nothing else.
 *
 * Common rules: pointers are device memory, 16-byte aligned; bytes is a multiple
 * of 16; blocks_per_cu (1..64) sets the grid to that many 256-thread blocks per
 * compute unit; stream is a hipStream_t passed as void* (NULL: the null stream).
 * Calls are asynchronous.  Return value: 0 on success, 1 for an invalid argument
 * (nothing enqueued), 4 when the HIP runtime reports an error.
 */
#ifndef LS_CEILING_H
#define LS_CEILING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of src once.  sink: one device uint32, written only in the
 * (practically impossible) case that the xor of all words equals 0x9e3779b9. */
int ls_ceiling_read(const void *src, size_t bytes, void *sink, int blocks_per_cu, void *stream);

/* Writes `bytes` bytes of dst once. */
int ls_ceiling_write(void *dst, size_t bytes, int blocks_per_cu, void *stream);

/* dst[0 .. bytes) = src[0 .. bytes); the buffers must not overlap. */
int ls_ceiling_copy(const void *src, void *dst, size_t bytes, int blocks_per_cu, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LS_CEILING_H */
