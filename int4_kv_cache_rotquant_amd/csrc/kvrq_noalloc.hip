// Static scratch of the allocation-free decode entry point (kv_int4_paged_decode_noalloc):
// the decode's workspace -- split counters, then partials -- in a file-scope device array,
// one per GPU the library runs on, held until the process ends.  Its device address is
// looked up once per device with hipGetSymbolAddress (the array's name in host code is a
// host-side stand-in, not a device address) and kept; everything that hands the array to a
// kernel uses that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvrq_internal.h"

namespace kvrq {
namespace {

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device (null: not yet)

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

}  // namespace

int noalloc_scratch(void **ptr, void *stream)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        // the split counters at the front must be zero before the first decode; every decode
        // leaves them zero again (a fill kernel, not a memset, so that a caller capturing a
        // graph records no memset node)
        const int64_t words = (int64_t)(kCounterBytes / 4);
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), static_cast<uint32_t *>(p), words);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace kvrq
