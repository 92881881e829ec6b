// ls_noalloc.hip -- workspace of the scan entry point that allocates nothing.
//
// Some callers cannot allocate device memory at the point of the call (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  For
// them scan_noalloc runs the single-pass scan on a fixed array in device memory
// that the library owns, one copy per GPU, held until the process ends.  The
// array's device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept; host code never passes the array's name itself
// to a kernel, since on the host that name is only a stand-in for the symbol.
#include <mutex>

#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
// Status words compare epochs modulo 2^26 at the least: the array is zeroed again
// after this many calls on a device (one fill kernel ahead of the call's scan).
constexpr int64_t NOALLOC_REINIT_CALLS = int64_t(1) << 25;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES];     // device address of `scratch` on each device, once known
int64_t g_scratch_calls[NOALLOC_MAX_DEVICES];  // calls since the last zero fill

}  // namespace

// Zero fill with 128-bit stores (a kernel, not a memset, so a caller may capture it).
__global__ __launch_bounds__(256) void scratch_zero_kernel(u32x4* p, int64_t words)
{
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < words; i += int64_t(gridDim.x) * 256)
        p[i] = z;
}

static hipError_t zero_scratch(void* p, hipStream_t s)
{
    constexpr int64_t words = int64_t(NOALLOC_SCRATCH_BYTES / 16);
    hipLaunchKernelGGL(scratch_zero_kernel, dim3(256), dim3(256), 0, s, reinterpret_cast<u32x4*>(p), words);
    return hipGetLastError();
}

// Device address of this device's scratch array.  The first call on a device
// looks it up and enqueues a zero fill of the whole array on `s`, ahead of the
// caller's work on the same stream; so does every NOALLOC_REINIT_CALLS-th call.
hipError_t noalloc_scratch(hipStream_t s, void** ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        if ((e = zero_scratch(p, s)) != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
        g_scratch_calls[dev] = 0;
    } else if (++g_scratch_calls[dev] >= NOALLOC_REINIT_CALLS) {
        if ((e = zero_scratch(g_scratch_ptr[dev], s)) != hipSuccess)
            return e;
        g_scratch_calls[dev] = 0;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace ls
