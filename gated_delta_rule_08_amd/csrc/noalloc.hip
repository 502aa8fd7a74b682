// Fixed device scratch of gdr_chunk_prefill_noalloc, the prefill call that
// allocates nothing (for callers that cannot call hipMalloc: code under graph
// capture, tight serving loops).  The scratch is a file-scope device array;
// each GPU the library runs on holds its own copy from the first use of this
// file's code object there until the process ends.  Its address on a device
// is looked up once, with that device current, and cached per device: in
// host code the array's name is only a stand-in, never a device address.
#include <mutex>

#include "gdr_internal.h"

namespace gdr {
namespace {

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t sd = 0;
        if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess) return e;
        dev = sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [&] {
        hipError_t r = dev == cur ? hipSuccess : hipSetDevice(dev);
        if (r == hipSuccess) r = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (r == hipSuccess) r = back;
        }
        g_err[dev] = r;
    });
    if (g_err[dev] != hipSuccess) return g_err[dev];
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gdr
