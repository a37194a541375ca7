// plane_common.hpp -- one direction's forward scan over a plane held in LDS
// (internal to libgspn): the body of the plane-resident four-direction
// kernel (plane4.hip), which the plane-resident adjoint (adjplane.hip) also
// runs to recompute the forward states it differentiates.
//
// GSPN-2 paper notes, "2D spatial propagation recap": the line-scan
// recurrence with sigmoid-and-normalised tridiagonal weights; chunks restart
// h every K steps in scan order ("Optimisation 1").  Planes of at most
// 64 x 64: one lane per line position, h in a VGPR, neighbours by DPP.
#pragma once

#include <utility>

#include "device.hpp"

namespace gspn {
namespace plane {

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

}  // namespace plane
}  // namespace gspn
