// elementwise.hip -- the standalone weight normalisation and the four-way
// merge.  Both are pure streaming kernels (HBM-bound): grid-stride loops over
// contiguous elements so every wavefront access is a coalesced run.
#include "device.hpp"
#include "launch.hpp"

namespace gspn {
namespace {

// Element e of [planes][S][L] positions (per_plane = S * L): the offset of
// its first logit in [planes][3][S][L] and its position k on the line.
// Shared by the kernels and their host replay.
struct NormPos {
    int64_t base;
    int64_t k;
};

GSPN_HD NormPos norm_pos(int64_t e, int64_t per_plane, int64_t L) {
    const int64_t pl = e / per_plane;
    const int64_t r = e - pl * per_plane;
    return {pl * 3 * per_plane + r, r % L};
}

// w = sigmoid row normalisation of the logit triple at every (plane, i, k)
// (GSPN summary page, "Approach"; rows sum to 1, border rows renormalised
// over the neighbours that exist).  Layout [planes][3][S][L].
template <typename T, typename TO>
__global__ __launch_bounds__(256) void normalize_kernel(const T* __restrict__ z, TO* __restrict__ w,
                                                        int64_t planes, int64_t S, int64_t L) {
    const int64_t per_plane = S * L;
    const int64_t total = planes * per_plane;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
         e += stride) {
        const NormPos np = norm_pos(e, per_plane, L);
        const int64_t k = np.k;
        const int64_t base = np.base;
        float w0, w1, w2;
        normalise_row(Store<T>::ld(z + base), Store<T>::ld(z + base + per_plane),
                      Store<T>::ld(z + base + 2 * per_plane), k > 0, k + 1 < L, w0, w1, w2);
        Store<TO>::st(w + base, w0);
        Store<TO>::st(w + base + per_plane, w1);
        Store<TO>::st(w + base + 2 * per_plane, w2);
    }
}

// The four directions' channel-shared logits normalised into packed half
// pairs (w_{k-1}, w_{k+1}) per position, layout [planes][S][L] of 32-bit
// words, in one launch (blockIdx.y = direction).  vec: every line is whole 16-byte vectors
// and every tensor is 16-byte aligned, so a lane normalises one vector of
// positions with three 16-byte loads and writes its pairs with 16-byte
// stores; otherwise one position per lane.
struct Pair4K {
    const void* z[4];
    uint32_t* w[4];
    int64_t planes;
    int64_t S[4];
    int64_t L[4];
    int vec;
};

template <typename T>
__global__ __launch_bounds__(256) void normalize_pair4_kernel(const Pair4K a) {
    constexpr int VW = 16 / static_cast<int>(sizeof(T));
    const int d = blockIdx.y;
    const T* __restrict__ z = static_cast<const T*>(a.z[d]);
    uint32_t* __restrict__ w = a.w[d];
    const int64_t L = a.L[d];
    const int64_t per_plane = a.S[d] * L;
    const int64_t total = a.planes * per_plane;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (a.vec) {
        struct alignas(16) V {
            T e[VW];
        };
        struct alignas(16) W4 {
            uint32_t e[4];
        };
        for (int64_t v = first; v < total / VW; v += stride) {
            const int64_t e = v * VW;
            const NormPos np = norm_pos(e, per_plane, L);
            const int64_t k0 = np.k;
            const T* zb = z + np.base;
            const V z0 = *reinterpret_cast<const V*>(zb);
            const V z1 = *reinterpret_cast<const V*>(zb + per_plane);
            const V z2 = *reinterpret_cast<const V*>(zb + 2 * per_plane);
            uint32_t out[VW];
#pragma unroll
            for (int j = 0; j < VW; ++j) {
                float w0, w1, w2;
                normalise_row(Store<T>::ld(&z0.e[j]), Store<T>::ld(&z1.e[j]), Store<T>::ld(&z2.e[j]), k0 + j > 0,
                              k0 + j + 1 < L, w0, w1, w2);
                out[j] = pack_pair(w0, w2);
            }
#pragma unroll
            for (int q = 0; q < VW / 4; ++q)
                *reinterpret_cast<W4*>(w + e + 4 * q) = W4{{out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]}};
        }
    } else {
        for (int64_t e = first; e < total; e += stride) {
            const NormPos np = norm_pos(e, per_plane, L);
            const int64_t k = np.k;
            const int64_t base = np.base;
            float w0, w1, w2;
            normalise_row(Store<T>::ld(z + base), Store<T>::ld(z + base + per_plane),
                          Store<T>::ld(z + base + 2 * per_plane), k > 0, k + 1 < L, w0, w1, w2);
            w[e] = pack_pair(w0, w2);
        }
    }
}

// y = ((h0 + h1) + h2) + h3
template <typename T>
__global__ __launch_bounds__(256) void merge4_kernel(const T* __restrict__ h0, const T* __restrict__ h1,
                                                     const T* __restrict__ h2, const T* __restrict__ h3,
                                                     T* __restrict__ y, int64_t numel) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < numel;
         e += stride) {
        const float v = ((Store<T>::ld(h0 + e) + Store<T>::ld(h1 + e)) + Store<T>::ld(h2 + e)) +
                        Store<T>::ld(h3 + e);
        Store<T>::st(y + e, v);
    }
}

unsigned grid_for(int64_t total, int threads) {
    int64_t blocks = (total + threads - 1) / threads;
    const int64_t cap = 256 * 64;  // 64 workgroups per CU is plenty for a grid-stride loop
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return static_cast<unsigned>(blocks);
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

#ifdef GSPN_CHECK_LAUNCHES
// Host replay of the normalisation kernels: for every element (or vector of
// VW elements) the grid-stride loops visit, the three logits read and the
// outputs written, at the offsets norm_pos gives.
void replay_normalize(const char* kn, const void* z, const void* w, int64_t planes, int64_t S, int64_t L, int es,
                      int eo, int vw, bool pair, bool vec) {
    const check::Region rz = check::region_of(z, kn, "logits");
    const check::Region rw = check::region_of(w, kn, "weights");
    const int64_t per_plane = S * L;
    const int64_t total = planes * per_plane;
    const int64_t step = vec ? vw : 1;
    int64_t bad = 0;
    for (int64_t e = 0; e + step <= total; e += step) {
        const NormPos np = norm_pos(e, per_plane, L);
        for (int o = 0; o < 3; ++o)
            if (!check::in_region(rz, z, (np.base + o * per_plane) * es, step * es) ||
                (vec && (reinterpret_cast<uint64_t>(z) + (np.base + o * per_plane) * es) % 16 != 0))
                ++bad;
        if (pair) {
            if (!check::in_region(rw, w, e * 4, step * 4)) ++bad;
        } else {
            for (int o = 0; o < 3; ++o)
                if (!check::in_region(rw, w, (np.base + o * per_plane) * eo, eo)) ++bad;
        }
    }
    if (bad) check::violation(kn, "accesses", "%lld bad", static_cast<long long>(bad));
    check::count_accesses(total * 6);
}
#endif

}  // namespace

hipError_t launch_normalize(int dir, int64_t n, int64_t cw, int64_t h, int64_t w,
                            const void* logits, void* w_out, int dtype, hipStream_t stream,
                            int out_dtype) {
    const bool horiz = (dir == 2 || dir == 3);
    const int64_t S = horiz ? w : h;
    const int64_t L = horiz ? h : w;
    const int64_t planes = n * cw;
    const unsigned grid = grid_for(planes * S * L, 256);
    if (out_dtype < 0) out_dtype = dtype;
#ifdef GSPN_CHECK_LAUNCHES
    replay_normalize("normalize_kernel", logits, w_out, planes, S, L, dtype == kF32 ? 4 : 2,
                     out_dtype == kF32 ? 4 : 2, 1, false, false);
    check::replayed("normalize_kernel", 256, 0);
#endif
    if (dtype == kF32) {
        hipLaunchKernelGGL((normalize_kernel<float, float>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const float*>(logits), static_cast<float*>(w_out), planes, S, L);
    } else if (out_dtype == kF32) {
        hipLaunchKernelGGL((normalize_kernel<bf16_t, float>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const bf16_t*>(logits), static_cast<float*>(w_out), planes, S, L);
    } else {
        hipLaunchKernelGGL((normalize_kernel<bf16_t, bf16_t>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const bf16_t*>(logits), static_cast<bf16_t*>(w_out), planes, S,
                           L);
    }
    return hipGetLastError();
}

hipError_t launch_normalize_pair4(int64_t n, int64_t h, int64_t w, const void* const logits[4],
                                  void* const w_out[4], int dtype, hipStream_t stream) {
    Pair4K k;
    const int vw = dtype == kF32 ? 4 : 8;
    k.planes = n;
    k.vec = 1;
    for (int d = 0; d < 4; ++d) {
        const bool horiz = (d == 2 || d == 3);
        k.z[d] = logits[d];
        k.w[d] = static_cast<uint32_t*>(w_out[d]);
        k.S[d] = horiz ? w : h;
        k.L[d] = horiz ? h : w;
        k.vec = k.vec && k.L[d] % vw == 0 && aligned16(logits[d]) && aligned16(w_out[d]);
    }
    const int64_t total = n * h * w;
    const dim3 grid(grid_for(k.vec ? total / vw : total, 256), 4);
#ifdef GSPN_CHECK_LAUNCHES
    for (int d = 0; d < 4; ++d)
        replay_normalize("normalize_pair4_kernel", k.z[d], k.w[d], n, k.S[d], k.L[d], dtype == kF32 ? 4 : 2, 4, vw,
                         true, k.vec != 0);
    check::replayed("normalize_pair4_kernel", 256, 0);
#endif
    if (dtype == kF32) hipLaunchKernelGGL(normalize_pair4_kernel<float>, grid, dim3(256), 0, stream, k);
    else hipLaunchKernelGGL(normalize_pair4_kernel<bf16_t>, grid, dim3(256), 0, stream, k);
    return hipGetLastError();
}

hipError_t launch_merge4(const void* h0, const void* h1, const void* h2, const void* h3, void* y,
                         int64_t numel, int dtype, hipStream_t stream) {
    const unsigned grid = grid_for(numel, 256);
    if (dtype == kF32) {
        hipLaunchKernelGGL(merge4_kernel<float>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const float*>(h0), static_cast<const float*>(h1),
                           static_cast<const float*>(h2), static_cast<const float*>(h3),
                           static_cast<float*>(y), numel);
    } else {
        hipLaunchKernelGGL(merge4_kernel<bf16_t>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const bf16_t*>(h0), static_cast<const bf16_t*>(h1),
                           static_cast<const bf16_t*>(h2), static_cast<const bf16_t*>(h3),
                           static_cast<bf16_t*>(y), numel);
    }
    return hipGetLastError();
}

}  // namespace gspn
