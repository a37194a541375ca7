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

namespace gspn {
namespace {

constexpr int kPlaneMax = 64;
constexpr int kDepth = 8;  // steps of logits / lambda in flight per wave

template <int V>
using IC = std::integral_constant<int, V>;

struct Plane4K {
    const void* x;
    const void* logits[4];
    const void* lam[4];
    void* y;
    int64_t c;
    int64_t cw;
    int H;
    int W;
    int K[4];  // steps per chunk of each direction (S_d for one chunk)
    const float* merge;  // learnable merge weights [4][c], or null for the plain sum
    float* states[4];    // STATES: direction d's fp32 scan h_d in its scan frame [planes][S_d][L_d]
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Default cache policy: the per-step rows are not 128-byte aligned, so
// consecutive steps share cache lines (with the non-temporal hint the
// logits and lambda streams fetched 20% more bytes, and ran no faster).
template <typename E>
__device__ __forceinline__ uint32_t load_raw(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(E) == 4) {
        return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    } else {
        return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
    }
}

template <typename E>
__device__ __forceinline__ float widen(uint32_t raw) {
    if constexpr (sizeof(E) == 4) {
        return __uint_as_float(raw);
    } else {
        return __uint_as_float(raw << 16);
    }
}

// x plane (hw elements, rows of W) into the padded LDS tile, fp32; 16-byte
// loads when the plane is a whole number of aligned vectors.
template <typename T>
__device__ __forceinline__ void load_plane(const T* xg, int64_t hw, int W, int ld, float* xs) {
    constexpr int VW = 16 / static_cast<int>(sizeof(T));
    const int n = static_cast<int>(hw);
    if (n % VW == 0 && (reinterpret_cast<uintptr_t>(xg) & 15) == 0) {
        for (int v = threadIdx.x; v < n / VW; v += blockDim.x) {
            const uint4 q = reinterpret_cast<const uint4*>(xg)[v];
            const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < VW; ++j) {
                const int e = v * VW + j;
                const int r = e / W;
                float f;
                if constexpr (sizeof(T) == 4) {
                    f = __uint_as_float(w4[j]);
                } else {
                    f = __uint_as_float((j & 1) ? (w4[j >> 1] & 0xffff0000u) : (w4[j >> 1] << 16));
                }
                xs[e + r * (ld - W)] = f;
            }
        }
    } else {
        for (int e = threadIdx.x; e < n; e += blockDim.x) xs[e + (e / W) * (ld - W)] = Store<T>::ld(xg + e);
    }
}

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

// Direction d of one plane: S steps over lines of L positions; element
// (step i, position k) of the direction sits at LDS (row, col) = (i, k) for
// the vertical directions and (k, i) for the horizontal ones.  The first
// kDepth steps' logits and lambdas are requested before x reaches LDS, so
// their latency overlaps the plane load.
// STATES: write the direction's unweighted h to a.states[d] (fp32, scan
// frame) instead of adding it into the partial.
template <typename T, bool HORIZ, bool REV, bool STATES>
__device__ __forceinline__ void plane_direction(const Plane4K& a, int d, int64_t p, const float* xs, float* part,
                                                int ld, const T* xg, int64_t hw) {
    const int lane = threadIdx.x & 63;
    const int S = HORIZ ? a.W : a.H;
    const int L = HORIZ ? a.H : a.W;
    const int K = a.K[d];
    const int64_t plane = static_cast<int64_t>(S) * L;
    const int64_t nidx = p / a.c;
    const int64_t ci = p - nidx * a.c;
    const float msc = (!STATES && a.merge) ? a.merge[d * a.c + ci] : 1.0f;
    float* hst = STATES ? a.states[d] + p * plane : nullptr;
    const auto rl = rsrc(static_cast<const T*>(a.lam[d]) + p * plane, plane * sizeof(T));
    const auto rz = rsrc(static_cast<const T*>(a.logits[d]) + (nidx * a.cw + (a.cw == 1 ? 0 : ci)) * 3 * plane,
                         3 * plane * sizeof(T));
    const bool active = lane < L;
    const int k = active ? lane : L - 1;
    const uint32_t vk = static_cast<uint32_t>(k) * sizeof(T);
    const uint32_t row = static_cast<uint32_t>(L) * sizeof(T);
    const uint32_t pz = static_cast<uint32_t>(plane) * sizeof(T);
    const bool has_l = lane > 0;
    const bool has_r = lane + 1 < L;

    auto line_of = [&](int t) { return REV ? S - 1 - t : t; };
    uint32_t rz0[kDepth], rz1[kDepth], rz2[kDepth], rlam[kDepth];
    auto fill = [&](auto slot, int t) {
        constexpr int s = decltype(slot)::value;
        const uint32_t o = static_cast<uint32_t>(line_of(min(t, S - 1))) * row;
        rz0[s] = load_raw<T>(rz, vk, o);
        rz1[s] = load_raw<T>(rz, vk, o + pz);
        rz2[s] = load_raw<T>(rz, vk, o + 2 * pz);
        rlam[s] = load_raw<T>(rl, vk, o);
    };

    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        (fill(IC<Ss>{}, Ss), ...);
    }(std::make_integer_sequence<int, kDepth>{});

    load_plane<T>(xg, hw, a.W, ld, const_cast<float*>(xs));
    __syncthreads();

    float h = 0.0f;
    int cpos = 0;  // step within the current chunk
    // The two directions of a pair share `part` without atomics: up to the
    // barrier each writes the lines of its first half of the steps (disjoint:
    // the forward direction stops after floor(S/2) steps, the reverse one
    // after ceil(S/2)), after it each adds onto lines the other one wrote.
    // Every element takes two additions onto 0, so the order of the pair does
    // not matter.
    const int split = REV ? (S + 1) / 2 : S / 2;
    auto step = [&](auto slot, int t) {
        constexpr int s = decltype(slot)::value;
        if (!STATES && t == split) __syncthreads();
        const int i = line_of(t);
        const int pos = HORIZ ? k * ld + i : i * ld + k;
        const float u = (widen<T>(rlam[s]) * msc) * xs[pos];
        float hn = u;
        const bool first = cpos == 0;  // chunk start: h_prev = 0, logits unused
        cpos = cpos + 1 == K ? 0 : cpos + 1;
        const float hl = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(h), 0x138, 0xf, 0xf, true));
        const float hr = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(h), 0x130, 0xf, 0xf, true));
        if (!first) {
            float w0, w1, w2;
            normalise_row(widen<T>(rz0[s]), widen<T>(rz1[s]), widen<T>(rz2[s]), has_l, has_r, w0, w1, w2);
            hn = __builtin_fmaf(w0, hl, __builtin_fmaf(w1, h, __builtin_fmaf(w2, hr, u)));
        }
        fill(slot, t + kDepth);
        h = active ? hn : 0.0f;
        if constexpr (STATES) {
            if (active) hst[static_cast<int64_t>(i) * L + k] = h;
        } else {
            if (active) part[pos] = part[pos] + h;
        }
    };

    int t = 0;
    for (; t + kDepth <= S; t += kDepth) {
        [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
            (step(IC<Ss>{}, t + Ss), ...);
        }(std::make_integer_sequence<int, kDepth>{});
    }
    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        ((t + Ss < S ? step(IC<Ss>{}, t + Ss) : void()), ...);
    }(std::make_integer_sequence<int, kDepth - 1>{});
    if (!STATES && split >= S) __syncthreads();  // a one-step reverse scan
}

// STATES: the four directions' fp32 scans go to a.states (only the x tile
// in LDS), with no merge and no y.
template <typename T, bool STATES>
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
    if constexpr (!STATES) {
        for (int e = threadIdx.x; e < H * ld; e += blockDim.x) {
            pv[e] = 0.0f;
            ph[e] = 0.0f;
        }
    }
    switch (threadIdx.x >> 6) {
        case 0: plane_direction<T, false, false, STATES>(a, 0, p, xs, pv, ld, xp, hw); break;
        case 1: plane_direction<T, false, true, STATES>(a, 1, p, xs, pv, ld, xp, hw); break;
        case 2: plane_direction<T, true, false, STATES>(a, 2, p, xs, ph, ld, xp, hw); break;
        default: plane_direction<T, true, true, STATES>(a, 3, p, xs, ph, ld, xp, hw); break;
    }
    if constexpr (!STATES) {
        __syncthreads();
        T* yp = static_cast<T*>(a.y) + p * hw;
        store_plane<T>(yp, hw, W, ld, pv, ph);
    }
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
        hipLaunchKernelGGL((plane4_kernel<float, false>), grid, dim3(256), lds, stream, k);
    } else {
        hipLaunchKernelGGL((plane4_kernel<bf16_t, false>), grid, dim3(256), lds, stream, k);
    }
    return hipGetLastError();
}

}  // namespace gspn

namespace gspn {

hipError_t launch_plane4_states(const void* x, const void* const logits[4], const void* const lam[4],
                                float* const states[4], int64_t n, int64_t c, int64_t cw, int64_t h, int64_t w,
                                const int64_t chunk[4], int dtype, hipStream_t stream) {
    Plane4K k;
    k.x = x;
    k.y = nullptr;
    k.merge = nullptr;
    for (int d = 0; d < 4; ++d) {
        k.logits[d] = logits[d];
        k.lam[d] = lam[d];
        k.K[d] = static_cast<int>(chunk[d]);
        k.states[d] = states[d];
    }
    k.c = c;
    k.cw = cw;
    k.H = static_cast<int>(h);
    k.W = static_cast<int>(w);
    const size_t lds = sizeof(float) * static_cast<size_t>(h) * static_cast<size_t>(w + 1);  // the x tile only
    const dim3 grid(static_cast<unsigned>(n * c));
    if (dtype == kF32) {
        hipLaunchKernelGGL((plane4_kernel<float, true>), grid, dim3(256), lds, stream, k);
    } else {
        hipLaunchKernelGGL((plane4_kernel<bf16_t, true>), grid, dim3(256), lds, stream, k);
    }
    return hipGetLastError();
}

}  // namespace gspn
