// check.hpp -- the host-side launch checker (internal to libgspn).
//
// The library's sources can be built a second way, host code only, with
// GSPN_CHECK_LAUNCHES defined (libgspn_check.so): the C ABI and every
// launcher run as usual, but a launch queues nothing.  Each launcher first
// replays its kernel on the host, block by block and thread by thread: the
// addresses come from the same index functions (GSPN_HD) that the kernel's
// own code calls, and every access is checked against the registered buffer
// that holds the pointer it goes through.  Then the launch macro records the
// kernel, grid, block and LDS size.  A launch whose kernel has no replay is
// itself reported.  Nothing here is compiled into the GPU library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Index code shared by a kernel and its host-side replay.
#define GSPN_HD __host__ __device__ __forceinline__

#ifdef GSPN_CHECK_LAUNCHES

namespace gspn {
namespace check {

// A registered buffer: [lo, hi) in the caller's address space (the checker
// never dereferences it, so any address range that no other buffer overlaps
// will do).
struct Region {
    uint64_t lo = 0, hi = 0;
    const char* name = nullptr;
};

// The buffer that holds address p; reports a violation (and returns an
// empty region) if none does.
Region region_of(const void* p, const char* kernel, const char* what);

void violation(const char* kernel, const char* what, const char* fmt, ...);
void count_accesses(int64_t n);

// An access of nbytes at base + off (bytes) must lie in r.
inline bool in_region(const Region& r, const void* base, int64_t off, int64_t nbytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base) + static_cast<uint64_t>(off);
    return off >= 0 && a >= r.lo && a + static_cast<uint64_t>(nbytes) <= r.hi;
}

// Marks the kernel about to be launched as replayed (kernel: its name, as
// the launch macro spells it; max_threads: its launch bound; static_lds: its
// static LDS bytes).
void replayed(const char* kernel, int max_threads, int64_t static_lds);
// Called by the launch macro in place of the launch.
void launched(const char* kernel, dim3 grid, dim3 block, size_t dyn_lds);

// The address the checking build gives the allocation-free forward's
// scratch array (kNoallocScratchBytes from here).
constexpr uint64_t kScratchStandIn = uint64_t{0x7e} << 40;

}  // namespace check
}  // namespace gspn

#undef hipLaunchKernelGGL
#define hipLaunchKernelGGL(kernel, grid, block, lds, stream, ...) \
    ::gspn::check::launched(#kernel, dim3(grid), dim3(block), static_cast<size_t>(lds))
#undef hipGetLastError
#define hipGetLastError() hipSuccess
// no kernels in the host-only build: kernel bodies become device functions,
// which the host pass does not compile
#undef __global__
#define __global__ __device__
#undef __launch_bounds__
#define __launch_bounds__(...)
#define GSPN_WAVES_PER_EU(n)

#else

#define GSPN_WAVES_PER_EU(n) __attribute__((amdgpu_waves_per_eu(n)))

#endif
