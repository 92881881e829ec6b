// ls_ceiling.hip -- plain streaming kernels that bound what any kernel moving the
// same bytes can reach on this GPU: read-only, write-only and copy, each a
// grid-stride loop of coalesced 128-bit accesses with the library's streaming
// (non-temporal) cache policy.  They compute nothing; the benchmark times them
// beside the scan and the compaction as the practical HBM ceilings.  Built into
// libls_ceiling.so, which only the benchmark loads; see include/ls_ceiling.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ls_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int THREADS = 256;
constexpr int UNROLL = 4;  // independent 16-byte accesses in flight per thread and trip

// Reads every 16-byte word once; the xor of all words goes to *sink only if it
// equals a value no test input produces, so the loads cannot be dropped.
__global__ __launch_bounds__(THREADS) void read_kernel(const u32x4* __restrict__ src, int64_t words,
                                                       uint32_t* __restrict__ sink)
{
    uint32_t x = 0;
    const int64_t step = int64_t(gridDim.x) * THREADS * UNROLL;
    for (int64_t base = int64_t(blockIdx.x) * THREADS * UNROLL + threadIdx.x; base < words; base += step) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
            const int64_t i = base + int64_t(k) * THREADS;
            v[k] = i < words ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < UNROLL; ++k)
            x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    if (x == 0x9e3779b9u)
        sink[0] = x;
}

__global__ __launch_bounds__(THREADS) void write_kernel(u32x4* __restrict__ dst, int64_t words)
{
    const int64_t step = int64_t(gridDim.x) * THREADS;
    for (int64_t i = int64_t(blockIdx.x) * THREADS + threadIdx.x; i < words; i += step)
        __builtin_nontemporal_store(u32x4{uint32_t(i), uint32_t(i >> 32), 0u, 0u}, dst + i);
}

__global__ __launch_bounds__(THREADS) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                       int64_t words)
{
    const int64_t step = int64_t(gridDim.x) * THREADS;
    for (int64_t i = int64_t(blockIdx.x) * THREADS + threadIdx.x; i < words; i += step)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

int grid_for(int blocks_per_cu)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess)
        return 0;
    return cus * blocks_per_cu;
}

bool bad(const void* p, size_t bytes, int blocks_per_cu)
{
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) != 0 || bytes % 16 != 0 || blocks_per_cu < 1 ||
           blocks_per_cu > 64;
}

}  // namespace

extern "C" {

int ls_ceiling_read(const void* src, size_t bytes, void* sink, int blocks_per_cu, void* stream)
{
    if (bad(src, bytes, blocks_per_cu) || sink == nullptr || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
        return 1;
    const int grid = grid_for(blocks_per_cu);
    if (grid == 0)
        return 4;
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(THREADS), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const u32x4*>(src), int64_t(bytes / 16), reinterpret_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int ls_ceiling_write(void* dst, size_t bytes, int blocks_per_cu, void* stream)
{
    if (bad(dst, bytes, blocks_per_cu))
        return 1;
    const int grid = grid_for(blocks_per_cu);
    if (grid == 0)
        return 4;
    hipLaunchKernelGGL(write_kernel, dim3(grid), dim3(THREADS), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<u32x4*>(dst), int64_t(bytes / 16));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int ls_ceiling_copy(const void* src, void* dst, size_t bytes, int blocks_per_cu, void* stream)
{
    if (bad(src, bytes, blocks_per_cu) || bad(dst, bytes, blocks_per_cu))
        return 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (bytes != 0 && a < b + bytes && b < a + bytes)
        return 1;  // overlapping buffers
    const int grid = grid_for(blocks_per_cu);
    if (grid == 0)
        return 4;
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(THREADS), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), int64_t(bytes / 16));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
