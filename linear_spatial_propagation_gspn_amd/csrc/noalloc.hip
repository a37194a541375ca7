// noalloc.hip -- the static device scratch array behind gspn_forward4_noalloc
// (internal to libgspn).
//
// Callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid allocation) get the forward's workspace from a
// file-scope device array instead of a buffer of their own.  Each GPU the
// library runs on holds one copy of the array, at its own address, from the
// moment the library's code object is loaded on that device until the process
// ends.  In host code the array's name is only a host-side handle: its device
// address is looked up once per device with hipGetSymbolAddress and cached,
// and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace gspn {

namespace {

#ifndef GSPN_CHECK_LAUNCHES
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
#endif

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
#ifdef GSPN_CHECK_LAUNCHES
    // the host-only checking build has no device array: a fixed address
    // range stands for it, which the caller registers as a buffer
    *out = reinterpret_cast<void*>(check::kScratchStandIn);
    return hipSuccess;
#endif
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
#ifndef GSPN_CHECK_LAUNCHES
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with dev current
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
#endif
    *out = scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gspn
