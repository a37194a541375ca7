// plane4.hip -- the four-direction propagation of small planes in one pass:
// x read once, y written once.
//
// GSPN-2 paper notes, "2D spatial propagation recap": four line scans over
// the same x, merged here by summation; chunks restart h every K steps in
// scan order ("Optimisation 1").  When a plane is at most 64 x 64 (the
// GSPN-T stage maps, e.g. 56 x 56) it fits in LDS, so one workgroup owns one
// (n, c) plane and runs all four directions on it:
//  - x is read from HBM once into an LDS tile (fp32, rows padded by one
//    element so that column accesses of the horizontal directions do not
//    conflict);
//  - wave d runs direction d with one lane per line position (lines are at
//    most 64 long), h in a VGPR and the neighbour values moved with DPP lane
//    shifts, so no step needs a barrier;
//  - the per-step logits and lambda stream from HBM in the directions' scan
//    frames (one contiguous line per step), prefetched D steps ahead;
//  - T2B and B2T add their h into one LDS partial, L2R and R2L into another,
//    with plain LDS reads and writes, no atomics (LDS float atomics made the
//    kernel 1.6x slower): each direction of a pair first writes the lines of
//    the first half of its steps, which the two directions split between
//    them, and after one barrier adds onto the lines the other one wrote.
//    Every element receives exactly two additions onto 0, and
//    fl(a + b) = fl(b + a), so the result does not depend on their order;
//  - y = partial_vertical + partial_horizontal is written to HBM once.
// Compulsory traffic only: x, the four directions' logits and lambdas, y.
#include <utility>

#include "device.hpp"
#include "launch.hpp"
#include "plane_common.hpp"

namespace gspn {
namespace {

using namespace plane;

// y = pv + ph over the plane, 16-byte stores when possible.
template <typename T>
__device__ __forceinline__ void store_plane(T* yg, int64_t hw, int W, int ld, const float* pv, const float* ph) {
    constexpr int VW = 16 / static_cast<int>(sizeof(T));
    const int n = static_cast<int>(hw);
    if (n % VW == 0 && (reinterpret_cast<uintptr_t>(yg) & 15) == 0) {
        for (int v = threadIdx.x; v < n / VW; v += blockDim.x) {
            uint32_t w4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < VW; ++j) {
                const int e = v * VW + j;
                const int a = e + (e / W) * (ld - W);
                const float f = pv[a] + ph[a];
                if constexpr (sizeof(T) == 4) {
                    w4[j] = __float_as_uint(f);
                } else {
                    w4[j >> 1] |= static_cast<uint32_t>(f32_to_bf16(f)) << ((j & 1) * 16);
                }
            }
            reinterpret_cast<uint4*>(yg)[v] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
    } else {
        for (int e = threadIdx.x; e < n; e += blockDim.x) {
            const int a = e + (e / W) * (ld - W);
            Store<T>::st(yg + e, pv[a] + ph[a]);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void plane4_kernel(const Plane4K a) {
    extern __shared__ float lds[];
    const int H = a.H;
    const int W = a.W;
    const int ld = W + 1;  // padded row: column walks hit distinct banks
    float* xs = lds;
    float* pv = xs + H * ld;  // T2B + B2T
    float* ph = pv + H * ld;  // L2R + R2L
    const int64_t p = blockIdx.x;
    const int64_t hw = static_cast<int64_t>(H) * W;
    const T* xp = static_cast<const T*>(a.x) + p * hw;
    for (int e = threadIdx.x; e < H * ld; e += blockDim.x) {
        pv[e] = 0.0f;
        ph[e] = 0.0f;
    }
    switch (threadIdx.x >> 6) {
        case 0: plane_direction<T, false, false, false>(a, 0, p, xs, pv, ld, xp, hw); break;
        case 1: plane_direction<T, false, true, false>(a, 1, p, xs, pv, ld, xp, hw); break;
        case 2: plane_direction<T, true, false, false>(a, 2, p, xs, ph, ld, xp, hw); break;
        default: plane_direction<T, true, true, false>(a, 3, p, xs, ph, ld, xp, hw); break;
    }
    __syncthreads();
    T* yp = static_cast<T*>(a.y) + p * hw;
    store_plane<T>(yp, hw, W, ld, pv, ph);
}

}  // namespace

bool plane4_supported(int64_t h, int64_t w) { return h >= 1 && w >= 1 && h <= kPlaneMax && w <= kPlaneMax; }

hipError_t launch_plane4(const void* x, const void* const logits[4], const void* const lam[4], const float* merge,
                         void* y, int64_t n, int64_t c, int64_t cw, int64_t h, int64_t w, const int64_t chunk[4],
                         int dtype, hipStream_t stream) {
    Plane4K k;
    k.x = x;
    k.y = y;
    k.merge = merge;
    for (int d = 0; d < 4; ++d) {
        k.logits[d] = logits[d];
        k.lam[d] = lam[d];
        k.K[d] = static_cast<int>(chunk[d]);
    }
    k.c = c;
    k.cw = cw;
    k.H = static_cast<int>(h);
    k.W = static_cast<int>(w);
    for (int d = 0; d < 4; ++d) k.states[d] = nullptr;
    const size_t lds = 3 * sizeof(float) * static_cast<size_t>(h) * static_cast<size_t>(w + 1);
    const dim3 grid(static_cast<unsigned>(n * c));
    if (dtype == kF32) {
        hipLaunchKernelGGL((plane4_kernel<float>), grid, dim3(256), lds, stream, k);
    } else {
        hipLaunchKernelGGL((plane4_kernel<bf16_t>), grid, dim3(256), lds, stream, k);
    }
    return hipGetLastError();
}

}  // namespace gspn
