// scan_kernel.hpp -- the line-scan kernel template and its launch families
// (internal to libgspn; instantiated per storage type and direction family in
// scan_{f32,bf16}_{vert,horiz}.hip).
//
// What it computes (GSPN-2 paper notes, "2D spatial propagation recap"):
//   h_i[k] = sum_{o in {-1,0,+1}, 0 <= k+o < L} w_i[k,o] h_{i-1}[k+o]
//            + lambda_i[k] x_i[k]
// for the lines i of one direction in scan order, with h = 0 before the
// first line of the scan and of every chunk ("Optimisation 1": independent
// (chunk, n, c) blocks).  w_i is the sigmoid row normalisation of the three
// logits at (i, k) (GSPN summary page, "Approach").
//
// Mapping on gfx950:
//  - A workgroup owns one line of L positions; each lane owns P contiguous
//    positions.  h stays in VGPRs for the whole scan.  The two values a lane
//    needs from its neighbours (h[k0-1], h[k0+P]) go through a
//    double-buffered LDS edge array: one barrier per step.
//  - The scan-frame tensors (logits, lambda) are line-contiguous, so every
//    step reads P contiguous values per lane: one coalesced row per stream.
//    Their next D steps sit in a register ring, so HBM latency overlaps the
//    serial chain of steps.
//  - Vertical directions (T2B, B2T): x and y rows are lines too and go
//    through the same ring.
//  - Horizontal directions (L2R, R2L): a line is an array column, so x and y
//    are read and written as per-lane row tiles: for a block of U steps each
//    lane loads the U consecutive columns of each of its rows (16-byte vector
//    loads), keeps the y tile in registers while the block runs, and writes
//    it back in one piece.  The next block's tiles are loaded while the
//    current block runs.
#pragma once

#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace gspn {

struct ScanK {
    const void* x;
    const void* wts;
    const void* lam;
    void* out;
    int64_t c;
    int64_t cw;
    int S;          // scan steps
    int L;          // line length
    int K;          // steps per chunk
    int nchunks;
    int reverse;    // scan runs from line S-1 down to 0
    int logits;     // wts holds logits (1) or normalised weights (0)
    int accumulate;
    int vec_frame;  // wts / lam allow P-wide vector access
    int vec_arr;    // vertical: x / out allow P-wide vector access
    int vec_tile;   // horizontal: x / out rows allow 16-byte access at 16-byte columns
};

template <typename T, int N>
struct alignas(sizeof(T) * N) VecT {
    T e[N];
};

// Streaming access: the scan reads each logit, lambda and (vertical) x value
// once and writes each output once.  With GSPN_STREAM_NT=1 those accesses
// carry the nontemporal hint; measured on MI355X it slows the scan by about
// half (profile workload, scan4 3.35 -> 4.97 ms), so it is off by default.
#ifndef GSPN_STREAM_NT
#define GSPN_STREAM_NT 0
#endif

template <typename T, int N>
struct Ext {
    typedef T type __attribute__((ext_vector_type(N)));
};
template <typename T>
struct Ext<T, 1> {
    typedef T type;
};

template <typename T, int N, bool NT>
__device__ __forceinline__ VecT<T, N> vload(const T* p) {
    if constexpr (NT && GSPN_STREAM_NT) {
        using V = typename Ext<T, N>::type;
        const V v = __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
        VecT<T, N> r;
        if constexpr (N == 1) {
            r.e[0] = v;
        } else {
#pragma unroll
            for (int j = 0; j < N; ++j) r.e[j] = v[j];
        }
        return r;
    } else {
        return *reinterpret_cast<const VecT<T, N>*>(p);
    }
}

template <typename T, int N, bool NT>
__device__ __forceinline__ void vstore(T* p, const VecT<T, N>& r) {
    if constexpr (NT && GSPN_STREAM_NT) {
        using V = typename Ext<T, N>::type;
        V v;
        if constexpr (N == 1) {
            v = r.e[0];
        } else {
#pragma unroll
            for (int j = 0; j < N; ++j) v[j] = r.e[j];
        }
        __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
    } else {
        *reinterpret_cast<VecT<T, N>*>(p) = r;
    }
}

template <typename T, bool NT>
__device__ __forceinline__ float sload(const T* p) {
    const VecT<T, 1> r = vload<T, 1, NT>(p);
    return Store<T>::ld(&r.e[0]);
}

template <typename T, bool NT>
__device__ __forceinline__ void sstore(T* p, float v) {
    VecT<T, 1> r;
    Store<T>::st(&r.e[0], v);
    vstore<T, 1, NT>(p, r);
}

// P values of a line starting at position k0; positions >= L read as 0.
template <typename T, int P, bool NT>
__device__ __forceinline__ void load_run(const T* __restrict__ base, int k0, int L, bool vec,
                                         float (&dst)[P]) {
    if (vec) {
        const VecT<T, P> v = vload<T, P, NT>(base + k0);
#pragma unroll
        for (int j = 0; j < P; ++j) dst[j] = Store<T>::ld(&v.e[j]);
    } else {
#pragma unroll
        for (int j = 0; j < P; ++j) dst[j] = (k0 + j < L) ? sload<T, NT>(base + k0 + j) : 0.0f;
    }
}

template <typename T, int P, bool NT>
__device__ __forceinline__ void store_run(T* __restrict__ base, int k0, int L, bool vec,
                                          const float (&src)[P]) {
    if (vec) {
        VecT<T, P> v;
#pragma unroll
        for (int j = 0; j < P; ++j) Store<T>::st(&v.e[j], src[j]);
        vstore<T, P, NT>(base + k0, v);
    } else {
#pragma unroll
        for (int j = 0; j < P; ++j)
            if (k0 + j < L) sstore<T, NT>(base + k0 + j, src[j]);
    }
}

// One line scan: plane p, chunk q of the direction described by a.
// T: storage type.  P: positions per lane.  D: prefetch ring depth.
// U: steps per block (a multiple of D; the horizontal tile width).
// HORIZ / REV: direction.  Every lane of the workgroup takes part (lanes past
// the end of the line hold no positions but join every barrier).
// edge_raw: 4 * blockDim.x floats of LDS for the neighbour exchange.
template <typename T, int P, int D, int U, bool HORIZ, bool REV>
__device__ __forceinline__ void scan_line(const ScanK& a, int64_t p, int q, float* edge_raw) {
    static_assert(U % D == 0, "a block must hold whole ring turns");
    constexpr int VW = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte vector
    static_assert(!HORIZ || U % VW == 0, "tile width must be whole vectors");

    // Edge exchange, [buffer][0 = first position, 1 = last position][lane].
    auto edge = [&](int b, int which, int lane) -> float& {
        return edge_raw[(b * 2 + which) * blockDim.x + lane];
    };

    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int64_t nidx = p / a.c;
    const int64_t ci = p - nidx * a.c;
    const int S = a.S;
    const int L = a.L;
    const int64_t plane = static_cast<int64_t>(S) * L;

    const T* __restrict__ xp = static_cast<const T*>(a.x) + p * plane;
    const T* __restrict__ lp = static_cast<const T*>(a.lam) + p * plane;
    const T* __restrict__ zp =
        static_cast<const T*>(a.wts) + (nidx * a.cw + (a.cw == 1 ? 0 : ci)) * 3 * plane;
    T* __restrict__ op = static_cast<T*>(a.out) + p * plane;

    const int k0 = tid * P;
    const int t0 = q * a.K;
    const int t1 = min(t0 + a.K, S);
    const bool rev = HORIZ ? REV : (a.reverse != 0);
    const bool vf = a.vec_frame && (k0 + P <= L);
    const bool va = !HORIZ && a.vec_arr && (k0 + P <= L);
    const bool acc = a.accumulate != 0;

    // Register ring: per-step inputs of the next D steps.
    float rz[D][3][P];
    float rl[D][P];
    float rx[HORIZ ? 1 : D][P];
    float ry[HORIZ ? 1 : D][P];
    // Horizontal tiles (two blocks: current and next).
    float xt[HORIZ ? 2 : 1][P][HORIZ ? U : 1];
    float yt[HORIZ ? 2 : 1][P][HORIZ ? U : 1];

    auto fetch = [&](int slot, int t) {
        if (t >= t1) return;
        const int i = rev ? S - 1 - t : t;
        const int64_t lo = static_cast<int64_t>(i) * L;
#pragma unroll
        for (int o = 0; o < 3; ++o) load_run<T, P, true>(zp + o * plane + lo, k0, L, vf, rz[slot][o]);
        load_run<T, P, true>(lp + lo, k0, L, vf, rl[slot]);
        if constexpr (!HORIZ) {
            load_run<T, P, true>(xp + lo, k0, L, va, rx[slot]);
            if (acc) load_run<T, P, true>(op + lo, k0, L, va, ry[slot]);
        }
    };

    // Horizontal tile of the block starting at step tb: array columns
    // [c_lo, c_lo + U); step tb + s sits at column offset (REV ? U-1-s : s).
    auto tile_lo = [&](int tb) { return REV ? S - tb - U : tb; };

    auto load_tile = [&](float (&xd)[P][HORIZ ? U : 1], float (&yd)[P][HORIZ ? U : 1], int tb) {
        if constexpr (HORIZ) {
            const int clo = tile_lo(tb);
            const bool full = tb + U <= t1;
            const bool vec = full && a.vec_tile && (clo % VW == 0);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const int k = k0 + j;
                const bool row = k < L;
                const T* xr = xp + static_cast<int64_t>(k) * S;
                const T* yr = op + static_cast<int64_t>(k) * S;
                if (vec && row) {
#pragma unroll
                    for (int v = 0; v < U / VW; ++v) {
                        const VecT<T, VW> xv = *reinterpret_cast<const VecT<T, VW>*>(xr + clo + v * VW);
#pragma unroll
                        for (int e = 0; e < VW; ++e) xd[j][v * VW + e] = Store<T>::ld(&xv.e[e]);
                        if (acc) {
                            const VecT<T, VW> yv = vload<T, VW, true>(yr + clo + v * VW);
#pragma unroll
                            for (int e = 0; e < VW; ++e) yd[j][v * VW + e] = Store<T>::ld(&yv.e[e]);
                        }
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int s = REV ? U - 1 - u : u;
                        const bool on = row && (tb + s < t1);
                        xd[j][u] = on ? Store<T>::ld(xr + clo + u) : 0.0f;
                        yd[j][u] = (on && acc) ? sload<T, true>(yr + clo + u) : 0.0f;
                    }
                }
            }
        }
    };

    auto store_tile = [&](const float (&yd)[P][HORIZ ? U : 1], int tb) {
        if constexpr (HORIZ) {
            const int clo = tile_lo(tb);
            const bool full = tb + U <= t1;
            const bool vec = full && a.vec_tile && (clo % VW == 0);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const int k = k0 + j;
                if (k >= L) continue;
                T* yr = op + static_cast<int64_t>(k) * S;
                if (vec) {
#pragma unroll
                    for (int v = 0; v < U / VW; ++v) {
                        VecT<T, VW> yv;
#pragma unroll
                        for (int e = 0; e < VW; ++e) Store<T>::st(&yv.e[e], yd[j][v * VW + e]);
                        vstore<T, VW, true>(yr + clo + v * VW, yv);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int s = REV ? U - 1 - u : u;
                        if (tb + s < t1) sstore<T, true>(yr + clo + u, yd[j][u]);
                    }
                }
            }
        }
    };

    float h[P];
#pragma unroll
    for (int j = 0; j < P; ++j) h[j] = 0.0f;

#pragma unroll
    for (int s = 0; s < D; ++s) fetch(s, t0 + s);
    if constexpr (HORIZ) load_tile(xt[0], yt[0], t0);

    int buf = 0;

    // One block of U steps; CUR selects the tile buffers statically.
    auto run_block = [&](auto cur_c, int tb) {
        constexpr int CUR = decltype(cur_c)::value;
        constexpr int NXT = HORIZ ? 1 - CUR : 0;
        constexpr int CB = HORIZ ? CUR : 0;
        if constexpr (HORIZ) {
            if (tb + U < t1) load_tile(xt[NXT], yt[NXT], tb + U);
        }
#pragma unroll
        for (int s = 0; s < U; ++s) {
            const int t = tb + s;
            if (t < t1) {
                const int slot = s % D;
                const int off = HORIZ ? (REV ? U - 1 - s : s) : 0;
                const int i = rev ? S - 1 - t : t;
                const bool first = (t == t0);
                float left = 0.0f, right = 0.0f;
                if (!first) {
                    left = tid > 0 ? edge(buf, 1, tid - 1) : 0.0f;
                    right = tid + 1 < nt ? edge(buf, 0, tid + 1) : 0.0f;
                }
                float hn[P];
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const int k = k0 + j;
                    const float xv = HORIZ ? xt[CB][j][off] : rx[HORIZ ? 0 : slot][j];
                    float u = rl[slot][j] * xv;
                    if (!first) {
                        float w0, w1, w2;
                        const bool has_l = k > 0;
                        const bool has_r = k + 1 < L;
                        if (a.logits) {
                            normalise_row(rz[slot][0][j], rz[slot][1][j], rz[slot][2][j], has_l, has_r,
                                          w0, w1, w2);
                        } else {
                            w0 = has_l ? rz[slot][0][j] : 0.0f;
                            w1 = rz[slot][1][j];
                            w2 = has_r ? rz[slot][2][j] : 0.0f;
                        }
                        const float hl = (j == 0) ? left : h[j - 1];
                        const float hr = (j == P - 1) ? right : h[j + 1];
                        u = __builtin_fmaf(w0, hl, __builtin_fmaf(w1, h[j], __builtin_fmaf(w2, hr, u)));
                    }
                    hn[j] = (k < L) ? u : 0.0f;
                }
                if constexpr (HORIZ) {
#pragma unroll
                    for (int j = 0; j < P; ++j)
                        yt[CB][j][off] = acc ? yt[CB][j][off] + hn[j] : hn[j];
                } else {
                    float ov[P];
#pragma unroll
                    for (int j = 0; j < P; ++j) ov[j] = acc ? ry[slot][j] + hn[j] : hn[j];
                    store_run<T, P, true>(op + static_cast<int64_t>(i) * L, k0, L, va, ov);
                }
#pragma unroll
                for (int j = 0; j < P; ++j) h[j] = hn[j];

                fetch(slot, t + D);

                buf ^= 1;
                edge(buf, 0, tid) = h[0];
                edge(buf, 1, tid) = h[P - 1];
                __syncthreads();
            }
        }
        if constexpr (HORIZ) store_tile(yt[CB], tb);
    };

    for (int tb = t0; tb < t1; tb += 2 * U) {
        run_block(std::integral_constant<int, 0>{}, tb);
        if (tb + U < t1) run_block(std::integral_constant<int, 1>{}, tb + U);
    }
}


// Single-direction launch: one workgroup per (plane, chunk).
template <typename T, int P, int D, int U, bool HORIZ, bool REV, int MAXT>
__global__ __launch_bounds__(MAXT) void scan_kernel(const ScanK a) {
    extern __shared__ float s_edge_raw[];
    const int64_t blk = blockIdx.x;
    const int64_t p = blk / a.nchunks;  // plane n * c + ci
    const int q = static_cast<int>(blk - p * a.nchunks);
    scan_line<T, P, D, U, HORIZ, REV>(a, p, q, s_edge_raw);
}

// ---------------------------------------------------------------------------
// Launch families
// ---------------------------------------------------------------------------

// Positions per lane and most lanes per workgroup.
struct ScanConfig {
    int P;
    int maxt;
};

// Horizontal tile width: 16 steps for one position per lane, fewer for more
// positions so the two tiles of x and y stay in registers; at least one
// 16-byte vector per row and one turn of the prefetch ring.
template <typename T, int P, int D>
constexpr int tile_width() {
    constexpr int vw = 16 / static_cast<int>(sizeof(T));
    constexpr int u = (16 / P) > vw ? (16 / P) : vw;
    return u > D ? u : D;
}

template <typename T, int P, int D, int MAXT, bool HORIZ, bool REV>
hipError_t launch_one(const ScanK& k, int64_t nblocks, int nthreads, hipStream_t stream) {
    constexpr int U = HORIZ ? tile_width<T, P, D>() : D;
    const size_t lds = 4 * sizeof(float) * static_cast<size_t>(nthreads);
    hipLaunchKernelGGL((scan_kernel<T, P, D, U, HORIZ, REV, MAXT>), dim3(static_cast<unsigned>(nblocks)),
                       dim3(nthreads), lds, stream, k);
    return hipGetLastError();
}

#ifndef GSPN_RING_D
#define GSPN_RING_D 4
#endif

template <typename T, int P, int D, int MAXT, bool HORIZ>
hipError_t launch_rev(bool rev, const ScanK& k, int64_t nblocks, int nthreads, hipStream_t stream) {
    if constexpr (HORIZ) {
        return rev ? launch_one<T, P, D, MAXT, true, true>(k, nblocks, nthreads, stream)
                   : launch_one<T, P, D, MAXT, true, false>(k, nblocks, nthreads, stream);
    } else {
        return launch_one<T, P, D, MAXT, false, false>(k, nblocks, nthreads, stream);
    }
}

// Instantiated families.  Up to 256 lanes: one position per lane.  Up to
// 1024 lanes: P in {1, 2, 4} with a GSPN_RING_D-deep ring; P = 8 (lines over
// 4096 positions) with a 2-deep ring.  Builds with GSPN_TUNING also
// instantiate P in {2, 4, 8} on 256 lanes.
template <typename T, bool HORIZ>
hipError_t launch_family(const ScanConfig& c, bool rev, const ScanK& k, int64_t nblocks, int nthreads,
                         hipStream_t stream) {
    constexpr int D = GSPN_RING_D;
    if (c.maxt == 256) {
#ifdef GSPN_TUNING
        switch (c.P) {
            case 2: return launch_rev<T, 2, D, 256, HORIZ>(rev, k, nblocks, nthreads, stream);
            case 4: return launch_rev<T, 4, D, 256, HORIZ>(rev, k, nblocks, nthreads, stream);
            case 8: return launch_rev<T, 8, D, 256, HORIZ>(rev, k, nblocks, nthreads, stream);
            default: break;
        }
#endif
        return launch_rev<T, 1, D, 256, HORIZ>(rev, k, nblocks, nthreads, stream);
    }
    switch (c.P) {
        case 1: return launch_rev<T, 1, D, 1024, HORIZ>(rev, k, nblocks, nthreads, stream);
        case 2: return launch_rev<T, 2, D, 1024, HORIZ>(rev, k, nblocks, nthreads, stream);
        case 4: return launch_rev<T, 4, D, 1024, HORIZ>(rev, k, nblocks, nthreads, stream);
        default: return launch_rev<T, 8, 2, 1024, HORIZ>(rev, k, nblocks, nthreads, stream);
    }
}

// ---------------------------------------------------------------------------
// Four directions in one launch
// ---------------------------------------------------------------------------

// The four directions' scans of one forward, each writing its own output
// buffer, so that all of them run concurrently and a small plane count still
// fills the chip.  Block b belongs to direction b % 4 when every direction has
// the same number of blocks (interleave = 1), else to consecutive ranges.
struct Scan4K {
    ScanK d[4];
    int64_t blocks[4];
    int interleave;
};

template <typename T, int PV, int PH>
__global__ __launch_bounds__(1024) void scan4_kernel(const Scan4K a) {
    extern __shared__ float s_edge_raw[];
    constexpr int D = GSPN_RING_D;
    constexpr int UH = tile_width<T, PH, D>();
    const int64_t b = blockIdx.x;
    int dir = 0;
    int64_t idx = b;
    if (a.interleave) {
        dir = static_cast<int>(b & 3);
        idx = b >> 2;
    } else {
        while (dir < 3 && idx >= a.blocks[dir]) {
            idx -= a.blocks[dir];
            ++dir;
        }
    }
    const ScanK& k = a.d[dir];
    const int64_t p = idx / k.nchunks;
    const int q = static_cast<int>(idx - p * k.nchunks);
    switch (dir) {
        case 0:
        case 1: scan_line<T, PV, D, D, false, false>(k, p, q, s_edge_raw); break;
        case 2: scan_line<T, PH, D, UH, true, false>(k, p, q, s_edge_raw); break;
        default: scan_line<T, PH, D, UH, true, true>(k, p, q, s_edge_raw); break;
    }
}

template <typename T>
hipError_t launch_fused4(const Scan4K& k, int pv, int ph, int nthreads, hipStream_t stream) {
    const int64_t nblocks = k.blocks[0] + k.blocks[1] + k.blocks[2] + k.blocks[3];
    const size_t lds = 4 * sizeof(float) * static_cast<size_t>(nthreads);
    const dim3 grid(static_cast<unsigned>(nblocks));
    if (pv == 1 && ph == 1) {
        hipLaunchKernelGGL((scan4_kernel<T, 1, 1>), grid, dim3(nthreads), lds, stream, k);
    } else if (pv == 1) {
        hipLaunchKernelGGL((scan4_kernel<T, 1, 2>), grid, dim3(nthreads), lds, stream, k);
    } else if (ph == 1) {
        hipLaunchKernelGGL((scan4_kernel<T, 2, 1>), grid, dim3(nthreads), lds, stream, k);
    } else {
        hipLaunchKernelGGL((scan4_kernel<T, 2, 2>), grid, dim3(nthreads), lds, stream, k);
    }
    return hipGetLastError();
}

}  // namespace gspn
