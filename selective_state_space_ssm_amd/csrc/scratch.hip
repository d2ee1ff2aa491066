// scratch.hip -- the library's one static device buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  ssm_scan_fwd_static
// (abi.cpp) runs the forward's time split with its chunk summaries here
// instead of in a caller's workspace.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, allocated when this code object is loaded on that
// device, until the process ends.  Its name in host code is only a
// host-side stand-in, never a device address: the device address is looked
// up once per device with hipGetSymbolAddress, with that device current,
// and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "ssm.h"

namespace ssm {
namespace {

static __device__ __align__(256) unsigned char scratch[SSM_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace ssm
