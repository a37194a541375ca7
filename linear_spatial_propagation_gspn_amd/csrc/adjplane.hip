// adjplane.hip -- the adjoint of the four-direction propagation for planes of
// at most 64 x 64: one workgroup per (n, c) plane runs all four directions'
// adjoint scans on it, with x, dL/dy and the dx partials resident in LDS.
//
// The gradient is the exact derivative of the forward that the GSPN-2 paper
// notes define ("2D spatial propagation recap"; chunks from "Optimisation
// 1"), the same recurrence as the long-line adjoint (backward.hip): in a
// direction's scan frame, with g_t = dL/dy at line t,
//   a_t          = g_t + M_{t+1}^T a_{t+1}         (backwards in t, per chunk)
//   dlambda_t[k] = m a_t[k] x_t[k],   dx_t[k] += m a_t[k] lambda_t[k]
//   dz_t[k,q]    = w_q (1 - s_q) (dw_q - sum_o dw_o w_o),  dw_o = m a_t[k] h_{t-1}[k+o]
// (m: the learnable merge weight, 1 without).  Here:
//  - x and dL/dy are read from HBM once, into padded LDS tiles, in the array
//    frame; every direction reads them there (the horizontal ones by
//    columns), so neither is transposed in HBM;
//  - wave d runs direction d with one lane per line position (lines of at
//    most 64), a_t in a VGPR, the neighbour products moved by DPP lane
//    shifts, so no step needs a barrier;
//  - the forward states h_{t-1} are recomputed in the same launch: each wave
//    first runs its direction's forward scan (plane_common.hpp) on the x
//    tile, writing its fp32 states to a workspace; after one barrier it
//    reads them back, newest first, while they are still in the cache (the
//    same lanes wrote them, so no other wave's writes are involved);
//  - the logits, lambda and those states stream in, D steps ahead;
//  - dx is summed in two LDS partials, T2B + B2T and L2R + R2L, with plain
//    reads and writes: each direction of a pair first writes the lines of the
//    first half of its steps, the two halves disjoint, and after one barrier
//    adds onto the lines the other one wrote (two additions onto 0 per
//    element, so the order does not matter); dx = partial + partial is
//    written once.
#include <utility>

#include "device.hpp"
#include "launch.hpp"
#include "plane_common.hpp"

namespace gspn {
namespace {

using plane::kPlaneMax;
using plane::load_raw;
using plane::rsrc;
using plane::widen;

constexpr int kDepth = 8;  // steps of logits, lambda and states in flight per wave

template <int V>
using IC = std::integral_constant<int, V>;

struct AdjPlaneK {
    const void* x;       // [planes][H][W]
    const void* g;       // dL/dy, [planes][H][W]
    const void* z[4];    // logits of direction d, [n][cw][3][S_d][L_d]
    const void* lam[4];  // [planes][S_d][L_d]
    float* hs[4];        // forward states, fp32 [planes][S_d][L_d], written by the kernel's forward phase
    void* dlam[4];       // [planes][S_d][L_d]
    void* dz[4];         // [n][cw][3][S_d][L_d], or for shared logits fp32 sums of dw differences [n][3][S_d][L_d] (added into)
    void* dx;            // [planes][H][W]
    const float* merge;  // [4][c] or null
    float* dmerge;       // [4][c] fp32, added into, or null
    int64_t c;
    int64_t cw;
    int H;
    int W;
    int K[4];  // steps per chunk (S_d for one chunk)
    int shared;
};

__device__ __forceinline__ float from_lower_lane(float v) {  // lane i gets lane i-1 (0 for lane 0)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, true));
}
__device__ __forceinline__ float from_upper_lane(float v) {  // lane i gets lane i+1 (0 for lane 63)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xf, 0xf, true));
}

// dL/dy (n elements, rows of W) into its padded fp32 LDS tile (x is there
// already, loaded by the forward phase): every thread's 16-byte loads are
// issued before its first LDS write (256 threads, at most 64 x 64 elements:
// at most four vectors).
template <typename T>
__device__ __forceinline__ void load_g_tile(const T* gg, int n, int W, int ld, float* gs) {
    constexpr int VW = 16 / static_cast<int>(sizeof(T));
    constexpr int NV = kPlaneMax * kPlaneMax / VW / 256;
    if (n % VW != 0 || (reinterpret_cast<uintptr_t>(gg) & 15) != 0) {
        for (int e = threadIdx.x; e < n; e += blockDim.x) gs[e + (e / W) * (ld - W)] = Store<T>::ld(gg + e);
        return;
    }
    const int nv = n / VW;
    uint4 qg[NV];
#pragma unroll
    for (int b = 0; b < NV; ++b) {
        const int v = min(static_cast<int>(threadIdx.x) + 256 * b, nv - 1);
        qg[b] = reinterpret_cast<const uint4*>(gg)[v];
    }
#pragma unroll
    for (int b = 0; b < NV; ++b) {
        const int v = static_cast<int>(threadIdx.x) + 256 * b;
        if (v >= nv) continue;
        const uint32_t wg[4] = {qg[b].x, qg[b].y, qg[b].z, qg[b].w};
#pragma unroll
        for (int j = 0; j < VW; ++j) {
            const int e = v * VW + j;
            const int a = e + (e / W) * (ld - W);
            if constexpr (sizeof(T) == 4) {
                gs[a] = __uint_as_float(wg[j]);
            } else {
                gs[a] = __uint_as_float((j & 1) ? (wg[j >> 1] & 0xffff0000u) : (wg[j >> 1] << 16));
            }
        }
    }
}

// The adjoint of direction d of plane p.  Processing step u = 0 .. S-1 is
// scan step t = S-1-u (line i = line_of(t)); element (line i, position k)
// sits at LDS (row, col) = (i, k) for the vertical directions, (k, i) for
// the horizontal ones.
template <typename T, bool HORIZ, bool REV, bool MERGE>
__device__ __forceinline__ void adj_direction(const AdjPlaneK& a, int d, int64_t p, float* xs, float* gs,
                                              float* part, int ld) {
    const int lane = threadIdx.x & 63;
    const int S = HORIZ ? a.W : a.H;
    const int L = HORIZ ? a.H : a.W;
    const int K = a.K[d];
    const int64_t plane = static_cast<int64_t>(S) * L;
    const int64_t nidx = p / a.c;
    const int64_t ci = p - nidx * a.c;
    const float msc = (MERGE && a.merge) ? a.merge[d * a.c + ci] : 1.0f;
    const auto rl = rsrc(static_cast<const T*>(a.lam[d]) + p * plane, plane * sizeof(T));
    const auto rz = rsrc(static_cast<const T*>(a.z[d]) + (nidx * a.cw + (a.cw == 1 ? 0 : ci)) * 3 * plane,
                         3 * plane * sizeof(T));
    const auto rh = rsrc(a.hs[d] + p * plane, plane * 4);
    const bool active = lane < L;
    const int k = active ? lane : L - 1;
    const uint32_t vk = static_cast<uint32_t>(k) * sizeof(T);
    const uint32_t vh = static_cast<uint32_t>(k) * 4;
    const uint32_t row = static_cast<uint32_t>(L) * sizeof(T);
    const uint32_t rowh = static_cast<uint32_t>(L) * 4;
    const uint32_t pz = static_cast<uint32_t>(plane) * sizeof(T);
    const bool has_l = lane > 0;
    const bool has_r = lane + 1 < L;
    T* dlp = static_cast<T*>(a.dlam[d]) + p * plane;
    T* dzp = a.shared ? nullptr : static_cast<T*>(a.dz[d]) + (nidx * a.cw + ci) * 3 * plane;
    float* dzs = a.shared ? static_cast<float*>(a.dz[d]) + nidx * 3 * plane : nullptr;

    auto line_of = [&](int t) { return REV ? S - 1 - t : t; };
    uint32_t rz0[kDepth], rz1[kDepth], rz2[kDepth], rlam[kDepth];
    float rhp[kDepth];
    auto fill = [&](auto slot, int u) {
        constexpr int s = decltype(slot)::value;
        const int t = S - 1 - min(u, S - 1);
        const uint32_t o = static_cast<uint32_t>(line_of(t)) * row;
        rz0[s] = load_raw<T>(rz, vk, o);
        rz1[s] = load_raw<T>(rz, vk, o + pz);
        rz2[s] = load_raw<T>(rz, vk, o + 2 * pz);
        rlam[s] = load_raw<T>(rl, vk, o);
        // h_{t-1}: the state one scan step earlier (clamped at the scan's
        // first step, where it is not used)
        rhp[s] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(
            rh, vh, static_cast<uint32_t>(line_of(max(t - 1, 0))) * rowh, 0)));
    };

    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        (fill(IC<Ss>{}, Ss), ...);
    }(std::make_integer_sequence<int, kDepth>{});

    // dL/dy into LDS (all four waves)
    const int64_t hw = static_cast<int64_t>(a.H) * a.W;
    load_g_tile<T>(static_cast<const T*>(a.g) + p * hw, static_cast<int>(hw), a.W, ld, gs);
    __syncthreads();

    float qn0 = 0.0f, qn1 = 0.0f, qn2 = 0.0f;  // w_{t+1}[k, o] a_{t+1}[k] for o = -1, 0, +1
    float dm = 0.0f;
    // the pair's partial, without atomics: lines of the first half of the
    // steps before the barrier (disjoint between the two directions), the
    // other direction's lines after it
    const int split = REV ? (S + 1) / 2 : S / 2;
    auto step = [&](auto slot, int u) {
        constexpr int s = decltype(slot)::value;
        if (u == split) __syncthreads();
        const int t = S - 1 - u;
        const int i = line_of(t);
        const int tk = t % K;
        const bool first = tk == 0;                   // the chunk's first line: no h_{t-1}, logits unused
        const bool last = tk == K - 1 || t == S - 1;  // the chunk's last line: no a_{t+1}
        float s0, s1, s2, w0, w1, w2;
        normalise_row_s(widen<T>(rz0[s]), widen<T>(rz1[s]), widen<T>(rz2[s]), has_l, has_r, s0, s1, s2, w0, w1, w2);
        const int pos = HORIZ ? k * ld + i : i * ld + k;
        const float from_r = from_upper_lane(qn0);  // w_{t+1}[k+1, -1] a_{t+1}[k+1]
        const float from_l = from_lower_lane(qn2);  // w_{t+1}[k-1, +1] a_{t+1}[k-1]
        float v = gs[pos];
        if (!last) v += (qn1 + from_r) + from_l;
        const float at = active ? v : 0.0f;
        const float am = MERGE ? at * msc : at;  // the adjoint of the merged output
        const float xk = xs[pos];
        const float lk = widen<T>(rlam[s]);
        if constexpr (MERGE) dm = __builtin_fmaf(at, lk * xk, dm);
        // dw_o = m a_t[k] h_{t-1}[k+o]
        const float hp = rhp[s];
        const float hl = from_lower_lane(hp);
        const float hr = from_upper_lane(hp);
        float dz[3] = {0.0f, 0.0f, 0.0f};
        const float dw0 = am * hl, dw1 = am * hp, dw2 = am * hr;
        if (!first && !a.shared) {
            const float dot = (dw0 * w0 + dw1 * w1) + dw2 * w2;
            dz[0] = w0 * (1.0f - s0) * (dw0 - dot);
            dz[1] = w1 * (1.0f - s1) * (dw1 - dot);
            dz[2] = w2 * (1.0f - s2) * (dw2 - dot);
            if (k == 0) dz[0] = 0.0f;
            if (k + 1 >= L) dz[2] = 0.0f;
            if (L == 1) dz[1] = 0.0f;  // a single neighbour: w = [1] whatever its logit
        }
        if (active) {
            const int64_t e = static_cast<int64_t>(i) * L + k;
            Store<T>::st(dlp + e, am * xk);
            part[pos] = part[pos] + am * lk;
            if (a.shared) {
                // channel sums of the weight-gradient differences; the
                // shared Jacobian is applied once to them afterwards
                if (!first) {
                    atomicAdd(dzs + e, dw0 - dw1);
                    atomicAdd(dzs + plane + e, dw2 - dw1);
                }
            } else {
#pragma unroll
                for (int o = 0; o < 3; ++o) Store<T>::st(dzp + o * plane + e, dz[o]);
            }
        }
        qn0 = first ? 0.0f : w0 * at;
        qn1 = first ? 0.0f : w1 * at;
        qn2 = first ? 0.0f : w2 * at;
        fill(slot, u + kDepth);
    };

    int u = 0;
    for (; u + kDepth <= S; u += kDepth) {
        [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
            (step(IC<Ss>{}, u + Ss), ...);
        }(std::make_integer_sequence<int, kDepth>{});
    }
    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        ((u + Ss < S ? step(IC<Ss>{}, u + Ss) : void()), ...);
    }(std::make_integer_sequence<int, kDepth - 1>{});
    if (split >= S) __syncthreads();  // a one-step reverse scan

    if (MERGE && a.dmerge) {
        float sum = dm;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        if (lane == 0) atomicAdd(a.dmerge + d * a.c + ci, sum);
    }
}

// Each wave first runs its direction's forward scan, writing the states to
// a.hs[d] (f describes that forward: the same x, logits, lambdas and chunks,
// states at a.hs), then, after a barrier, its adjoint reading them back.
template <typename T, bool MERGE>
__global__ __launch_bounds__(256) void adjplane_kernel(const AdjPlaneK a, const plane::Plane4K f) {
    extern __shared__ float lds[];
    const int H = a.H;
    const int W = a.W;
    const int ld = W + 1;  // padded rows: column walks hit distinct banks
    float* xs = lds;
    float* gs = xs + H * ld;
    float* pv = gs + H * ld;  // dx of T2B + B2T
    float* ph = pv + H * ld;  // dx of L2R + R2L
    const int64_t p = blockIdx.x;
    for (int e = threadIdx.x; e < H * ld; e += blockDim.x) {
        pv[e] = 0.0f;
        ph[e] = 0.0f;
    }
    // the forward: x into its tile (all waves), then direction d's states
    const int64_t hw0 = static_cast<int64_t>(H) * W;
    const T* xp = static_cast<const T*>(a.x) + p * hw0;
    switch (threadIdx.x >> 6) {
        case 0: plane::plane_direction<T, false, false, true>(f, 0, p, xs, nullptr, ld, xp, hw0); break;
        case 1: plane::plane_direction<T, false, true, true>(f, 1, p, xs, nullptr, ld, xp, hw0); break;
        case 2: plane::plane_direction<T, true, false, true>(f, 2, p, xs, nullptr, ld, xp, hw0); break;
        default: plane::plane_direction<T, true, true, true>(f, 3, p, xs, nullptr, ld, xp, hw0); break;
    }
    // the lanes that wrote the states read them back; the barrier orders
    // those writes before the reads, as for any access of the workgroup
    __syncthreads();
    switch (threadIdx.x >> 6) {
        case 0: adj_direction<T, false, false, MERGE>(a, 0, p, xs, gs, pv, ld); break;
        case 1: adj_direction<T, false, true, MERGE>(a, 1, p, xs, gs, pv, ld); break;
        case 2: adj_direction<T, true, false, MERGE>(a, 2, p, xs, gs, ph, ld); break;
        default: adj_direction<T, true, true, MERGE>(a, 3, p, xs, gs, ph, ld); break;
    }
    __syncthreads();
    const int64_t hw = static_cast<int64_t>(H) * W;
    T* dxp = static_cast<T*>(a.dx) + p * hw;
    for (int e = threadIdx.x; e < H * W; e += blockDim.x) {
        const int r = e / W;
        const int q = r * ld + (e - r * W);
        Store<T>::st(dxp + e, pv[q] + ph[q]);
    }
}

}  // namespace

hipError_t launch_adjplane(const AdjPlaneParams& p, hipStream_t stream) {
    AdjPlaneK k;
    k.x = p.x;
    k.g = p.g;
    for (int d = 0; d < 4; ++d) {
        k.z[d] = p.z[d];
        k.lam[d] = p.lam[d];
        k.hs[d] = p.hs[d];
        k.dlam[d] = p.dlam[d];
        k.dz[d] = p.dz[d];
        k.K[d] = static_cast<int>(p.chunk[d]);
    }
    k.dx = p.dx;
    k.merge = p.merge;
    k.dmerge = p.dmerge;
    k.c = p.c;
    k.cw = p.cw;
    k.H = static_cast<int>(p.h);
    k.W = static_cast<int>(p.w);
    k.shared = p.shared;
    // the forward the kernel recomputes: unweighted states into hs
    plane::Plane4K f;
    f.x = p.x;
    f.y = nullptr;
    f.merge = nullptr;
    for (int d = 0; d < 4; ++d) {
        f.logits[d] = p.z[d];
        f.lam[d] = p.lam[d];
        f.K[d] = static_cast<int>(p.chunk[d]);
        f.states[d] = p.hs[d];
    }
    f.c = p.c;
    f.cw = p.cw;
    f.H = k.H;
    f.W = k.W;
    const size_t lds = 4 * sizeof(float) * static_cast<size_t>(p.h) * static_cast<size_t>(p.w + 1);
    const dim3 grid(static_cast<unsigned>(p.n * p.c));
    const bool merge = p.merge || p.dmerge;
    if (p.dtype == kF32) {
        if (merge) hipLaunchKernelGGL((adjplane_kernel<float, true>), grid, dim3(256), lds, stream, k, f);
        else hipLaunchKernelGGL((adjplane_kernel<float, false>), grid, dim3(256), lds, stream, k, f);
    } else {
        if (merge) hipLaunchKernelGGL((adjplane_kernel<bf16_t, true>), grid, dim3(256), lds, stream, k, f);
        else hipLaunchKernelGGL((adjplane_kernel<bf16_t, false>), grid, dim3(256), lds, stream, k, f);
    }
    return hipGetLastError();
}

}  // namespace gspn
