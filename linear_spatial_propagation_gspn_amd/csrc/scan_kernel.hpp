// scan_kernel.hpp -- the line-scan kernel template and its launch families
// (internal to libgspn; instantiated per storage type and direction family in
// scan_*_{vert,horiz}.hip and scan4_*.hip).
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
//  - The scan-frame tensors (logits, lambda) are line-contiguous, so a step
//    reads one coalesced row per stream.  Vertical directions (T2B, B2T) read
//    and write x and y rows the same way.
//  - Horizontal directions (L2R, R2L): a line is an array column, so x and y
//    move as per-lane row tiles: for a tile of UT steps each lane loads the UT
//    consecutive columns of each of its rows with 16-byte loads, keeps the y
//    tile in registers while the tile runs and writes it back in one piece.
//  - Latency hiding: per-step inputs are fetched a sub-block of U steps ahead
//    and tiles a tile ahead, into double buffers selected at compile time.
//    In the main loop every load address is clamped into the tensors instead
//    of being guarded by a branch, so the loads form one straight sequence and
//    the compiler waits only for the sub-block it needs (a guarded or
//    branching load sequence makes it wait for every load in flight at every
//    step).  A guarded tail loop finishes the last partial blocks.
#pragma once

#include <type_traits>
#include <utility>

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
    int S;         // scan steps
    int L;         // line length
    int K;         // steps per chunk
    int nchunks;
    int reverse;   // scan runs from line S-1 down to 0
    int logits;    // wts holds logits (1) or normalised weights (0)
    int vec_tile;  // horizontal: every full tile of every chunk allows 16-byte row access
    const float* mscale;  // merge weight of each channel for this direction ([c]), or null for 1
    int xtile;     // long-line kernel: x is the array-frame plane [L][S], read through LDS column tiles
};

// Index code of scan_line and the long-line kernel, shared with the host
// replay: a position clamped into the line (addresses of lanes past its end),
// the row of scan step t, the step whose row a prefetch for step t reads
// (steps past the chunk read its last row), and the offset of plane p's
// weight rows from a.wts in weight elements (packed pairs: one a position).
GSPN_HD int scan_pos(int k, int L) { return k < L - 1 ? k : L - 1; }
GSPN_HD int scan_row(int t, int S, bool rev) { return rev ? S - 1 - t : t; }
GSPN_HD int scan_fetch_step(int t, int t1) { return t < t1 - 1 ? t : t1 - 1; }
GSPN_HD int64_t scan_weight_offset(const ScanK& a, int64_t p, int64_t plane, bool pair) {
    const int64_t nidx = p / a.c;
    const int64_t ci = p - nidx * a.c;
    return pair ? nidx * plane : (nidx * a.cw + (a.cw == 1 ? 0 : ci)) * 3 * plane;
}
// LDS edge value `which` (0: the lane's first position, 1: its last) of lane
// `lane` in buffer b, for nt lanes.
GSPN_HD int scan_edge(int b, int which, int nt, int lane) { return (b * 2 + which) * nt + lane; }

template <typename T, int N>
struct alignas(sizeof(T) * N) VecT {
    T e[N];
};

template <int V>
using IC = std::integral_constant<int, V>;

// One line scan: plane p, chunk q of the direction described by a.
// T: storage type of x, lambda and the output; TW: storage type of the
// logits / weights (the same as T, fp32 weights normalised beforehand, or
// WPair: channel-shared weights normalised beforehand as packed half pairs).
// P: positions per lane.  U: steps per prefetch sub-block.  UT: steps per
// tile (a multiple of U; the horizontal tile width).  HORIZ / REV: direction.
// ACC: add into the output instead of overwriting it.
// Every lane of the workgroup takes part: lanes past the end of the line hold
// no positions but join every barrier.  edge_raw: 4 * blockDim.x floats of LDS.
// TO: element type of the output (T, or fp32 for vertical-form scans that
// keep their states at full precision).
template <typename T, typename TW, int P, int U, int UT, bool HORIZ, bool REV, bool ACC, typename TO = T>
__device__ __forceinline__ void scan_line(const ScanK& a, int64_t p, int q, float* edge_raw) {
    static_assert(std::is_same_v<TO, T> || (!HORIZ && !ACC), "a wider output only for plain vertical scans");
    static_assert(UT % U == 0, "a tile holds whole sub-blocks");
    constexpr int NS = UT / U;                             // sub-blocks per tile
    constexpr int VW = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte vector
    static_assert(!HORIZ || UT % VW == 0, "tile width must be whole vectors");

    auto edge = [&](int b, int which, int lane) -> float& {
        return edge_raw[scan_edge(b, which, blockDim.x, lane)];
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
    const float msc = a.mscale ? a.mscale[ci] : 1.0f;  // learnable merge: this direction's weight
    constexpr bool PAIR = std::is_same_v<TW, WPair>;
    using ZT = std::conditional_t<PAIR, uint32_t, TW>;
    const ZT* __restrict__ zp = static_cast<const ZT*>(a.wts) + scan_weight_offset(a, p, plane, PAIR);
    T* __restrict__ op = static_cast<T*>(a.out) + p * plane;
    TO* __restrict__ oq = static_cast<TO*>(a.out) + p * plane;

    const int k0 = tid * P;
    const int t0 = q * a.K;
    const int t1 = min(t0 + a.K, S);
    const bool rev = HORIZ ? REV : (a.reverse != 0);
    const bool logits = !PAIR && a.logits != 0;

    // Positions of this lane, clamped into the line for addressing.
    int kk[P];
    bool kin[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        kk[j] = scan_pos(k0 + j, L);
        kin[j] = k0 + j < L;
    }

    // Double-buffered per-step inputs: [buffer][step of the sub-block].
    float rz[2][U][PAIR ? 1 : 3][P];
    float rl[2][U][P];
    float rx[HORIZ ? 1 : 2][U][P];
    float ry[(!HORIZ && ACC) ? 2 : 1][U][P];
    // Horizontal tiles: [buffer][position][step of the tile].
    float xt[HORIZ ? 2 : 1][P][HORIZ ? UT : 1];
    float yt[HORIZ ? 2 : 1][P][HORIZ ? UT : 1];

    auto line_of = [&](int t) { return scan_row(t, S, rev); };

    // Inputs of the U steps from tb into ring buffer R; steps past the chunk
    // read the chunk's last line (loaded, never used).
    auto load_ring = [&](auto rc, int tb) {
        constexpr int R = decltype(rc)::value;
#pragma unroll
        for (int s = 0; s < U; ++s) {
            const int64_t lo = static_cast<int64_t>(line_of(scan_fetch_step(tb + s, t1))) * L;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                if constexpr (PAIR) {
                    rz[R][s][0][j] = __uint_as_float(zp[lo + kk[j]]);
                } else {
#pragma unroll
                    for (int o = 0; o < 3; ++o) rz[R][s][o][j] = Store<TW>::ld(zp + o * plane + lo + kk[j]);
                }
                rl[R][s][j] = Store<T>::ld(lp + lo + kk[j]);
                if constexpr (!HORIZ) {
                    rx[R][s][j] = Store<T>::ld(xp + lo + kk[j]);
                    if constexpr (ACC) ry[R][s][j] = Store<T>::ld(op + lo + kk[j]);
                }
            }
        }
    };

    // Horizontal tile of the UT steps from tb: array columns [c_lo, c_lo+UT);
    // step tb + s sits at column offset (REV ? UT-1-s : s).
    auto tile_lo = [&](int tb) { return REV ? S - tb - UT : tb; };

    // Full tile with 16-byte loads; the column range is clamped into the row
    // (a tile past the chunk end is loaded but never used).
    auto load_tile_vec = [&](auto tc, int tb) {
        if constexpr (HORIZ) {
            constexpr int C = decltype(tc)::value;
            const int clo = min(max(tile_lo(tb), 0), S - UT);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const T* xr = xp + static_cast<int64_t>(kk[j]) * S + clo;
                const T* yr = op + static_cast<int64_t>(kk[j]) * S + clo;
#pragma unroll
                for (int v = 0; v < UT / VW; ++v) {
                    const VecT<T, VW> xv = *reinterpret_cast<const VecT<T, VW>*>(xr + v * VW);
#pragma unroll
                    for (int e = 0; e < VW; ++e) xt[C][j][v * VW + e] = Store<T>::ld(&xv.e[e]);
                    if constexpr (ACC) {
                        const VecT<T, VW> yv = *reinterpret_cast<const VecT<T, VW>*>(yr + v * VW);
#pragma unroll
                        for (int e = 0; e < VW; ++e) yt[C][j][v * VW + e] = Store<T>::ld(&yv.e[e]);
                    }
                }
            }
        }
    };

    // Any tile with element loads, columns clamped into the row.
    auto load_tile_elem = [&](auto tc, int tb) {
        if constexpr (HORIZ) {
            constexpr int C = decltype(tc)::value;
            const int clo = tile_lo(tb);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const T* xr = xp + static_cast<int64_t>(kk[j]) * S;
                const T* yr = op + static_cast<int64_t>(kk[j]) * S;
#pragma unroll
                for (int u = 0; u < UT; ++u) {
                    const int col = min(max(clo + u, 0), S - 1);
                    xt[C][j][u] = Store<T>::ld(xr + col);
                    if constexpr (ACC) yt[C][j][u] = Store<T>::ld(yr + col);
                }
            }
        }
    };

    // Full tile with 16-byte stores (its columns lie inside the chunk).
    auto store_tile_vec = [&](auto tc, int tb) {
        if constexpr (HORIZ) {
            constexpr int C = decltype(tc)::value;
            const int clo = tile_lo(tb);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                if (kin[j]) {
                    T* yr = op + static_cast<int64_t>(k0 + j) * S + clo;
#pragma unroll
                    for (int v = 0; v < UT / VW; ++v) {
                        VecT<T, VW> yv;
#pragma unroll
                        for (int e = 0; e < VW; ++e) Store<T>::st(&yv.e[e], yt[C][j][v * VW + e]);
                        *reinterpret_cast<VecT<T, VW>*>(yr + v * VW) = yv;
                    }
                }
            }
        }
    };

    // Partial tile: element stores for the steps inside the chunk only.
    auto store_tile_elem = [&](auto tc, int tb) {
        if constexpr (HORIZ) {
            constexpr int C = decltype(tc)::value;
            const int clo = tile_lo(tb);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                if (kin[j]) {
                    T* yr = op + static_cast<int64_t>(k0 + j) * S;
#pragma unroll
                    for (int u = 0; u < UT; ++u) {
                        const int s = REV ? UT - 1 - u : u;
                        if (tb + s < t1) Store<T>::st(yr + clo + u, yt[C][j][u]);
                    }
                }
            }
        }
    };

    float h[P];
#pragma unroll
    for (int j = 0; j < P; ++j) h[j] = 0.0f;
    int buf = 0;

    // U steps from tb, inputs in ring buffer R, inside the tile of buffer C
    // whose first step is tb - M * U.  GUARD: steps at or past t1 are skipped.
    auto sub_block = [&](auto rc, auto tc, auto mc, auto gc, int tb) {
        constexpr int R = decltype(rc)::value;
        constexpr int C = HORIZ ? decltype(tc)::value : 0;
        constexpr int M = decltype(mc)::value;
        constexpr bool GUARD = decltype(gc)::value != 0;
#pragma unroll
        for (int s = 0; s < U; ++s) {
            const int t = tb + s;
            if (!GUARD || t < t1) {
                const int off = HORIZ ? (REV ? UT - 1 - (M * U + s) : (M * U + s)) : 0;
                const bool first = (t == t0);
                float left = 0.0f, right = 0.0f;
                if (!first) {
                    left = tid > 0 ? edge(buf, 1, tid - 1) : 0.0f;
                    right = tid + 1 < nt ? edge(buf, 0, tid + 1) : 0.0f;
                }
                float hn[P];
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const float xv = HORIZ ? xt[C][j][off] : rx[HORIZ ? 0 : R][s][j];
                    float u = (rl[R][s][j] * msc) * xv;
                    if (!first) {
                        const bool has_l = k0 + j > 0;
                        const bool has_r = k0 + j + 1 < L;
                        float w0, w1, w2;
                        if constexpr (PAIR) {
                            const uint32_t b = __float_as_uint(rz[R][s][0][j]);
                            w0 = has_l ? pair_lo(b) : 0.0f;
                            w2 = has_r ? pair_hi(b) : 0.0f;
                            w1 = (1.0f - w0) - w2;
                        } else if (logits) {
                            normalise_row(rz[R][s][0][j], rz[R][s][1][j], rz[R][s][2][j], has_l, has_r, w0,
                                          w1, w2);
                        } else {
                            w0 = has_l ? rz[R][s][0][j] : 0.0f;
                            w1 = rz[R][s][1][j];
                            w2 = has_r ? rz[R][s][2][j] : 0.0f;
                        }
                        const float hl = (j == 0) ? left : h[j - 1];
                        const float hr = (j == P - 1) ? right : h[j + 1];
                        u = __builtin_fmaf(w0, hl, __builtin_fmaf(w1, h[j], __builtin_fmaf(w2, hr, u)));
                    }
                    hn[j] = kin[j] ? u : 0.0f;
                }
                if constexpr (HORIZ) {
#pragma unroll
                    for (int j = 0; j < P; ++j) yt[C][j][off] = ACC ? yt[C][j][off] + hn[j] : hn[j];
                } else {
                    TO* orow = oq + static_cast<int64_t>(line_of(t)) * L;
#pragma unroll
                    for (int j = 0; j < P; ++j) {
                        const float v = ACC ? ry[(HORIZ || !ACC) ? 0 : R][s][j] + hn[j] : hn[j];
                        if (kin[j]) Store<TO>::st(orow + k0 + j, v);
                    }
                }
#pragma unroll
                for (int j = 0; j < P; ++j) h[j] = hn[j];
                buf ^= 1;
                edge(buf, 0, tid) = h[0];
                edge(buf, 1, tid) = h[P - 1];
                __syncthreads();
            }
        }
    };

    // One tile of UT steps from tb with tile buffer C; the ring parity of its
    // first sub-block is R0.  Loads for the next tile / sub-block are issued
    // before the steps that precede their use.
    auto run_tile = [&](auto tc, auto r0c, auto gc, int tb) {
        constexpr int C = decltype(tc)::value;
        constexpr int R0 = decltype(r0c)::value;
        constexpr bool GUARD = decltype(gc)::value != 0;
        if constexpr (HORIZ) {
            if constexpr (GUARD) {
                if (tb + UT < t1) load_tile_elem(IC<1 - C>{}, tb + UT);
            } else {
                load_tile_vec(IC<1 - C>{}, tb + UT);
            }
        }
        auto one = [&](auto mc) {
            constexpr int M = decltype(mc)::value;
            constexpr int R = (R0 + M) & 1;
            load_ring(IC<1 - R>{}, tb + (M + 1) * U);
            sub_block(IC<R>{}, IC<C>{}, IC<M>{}, gc, tb + M * U);
        };
        [&]<int... Ms>(std::integer_sequence<int, Ms...>) {
            (one(IC<Ms>{}), ...);
        }(std::make_integer_sequence<int, NS>{});
        if constexpr (HORIZ) {
            if constexpr (GUARD) {
                store_tile_elem(IC<C>{}, tb);
            } else {
                store_tile_vec(IC<C>{}, tb);
            }
        }
    };

    constexpr int RT1 = NS & 1;  // ring parity at the start of the second tile
    int tb = t0;
    const bool fast = !HORIZ || a.vec_tile;
    if (fast) {
        load_ring(IC<0>{}, t0);
        load_tile_vec(IC<0>{}, t0);
        for (; tb + 2 * UT <= t1; tb += 2 * UT) {
            run_tile(IC<0>{}, IC<0>{}, IC<0>{}, tb);
            run_tile(IC<1>{}, IC<RT1>{}, IC<0>{}, tb + UT);
        }
    }
    if (tb < t1) {
        load_ring(IC<0>{}, tb);
        load_tile_elem(IC<0>{}, tb);
        for (; tb < t1; tb += 2 * UT) {
            run_tile(IC<0>{}, IC<0>{}, IC<1>{}, tb);
            if (tb + UT < t1) run_tile(IC<1>{}, IC<RT1>{}, IC<1>{}, tb + UT);
        }
    }
}

#ifndef GSPN_VERT_WAVES
#define GSPN_VERT_WAVES 8
#endif

// Waves per SIMD to budget registers for: vertical-form scans with one
// position per lane fit in 64 VGPRs, so two 1024-lane workgroups share a CU.
template <bool HORIZ, int P>
constexpr int waves_per_eu() {
    return (!HORIZ && P == 1) ? GSPN_VERT_WAVES : 4;
}

// Single-direction launch: one workgroup per (plane, chunk).
template <typename T, typename TW, int P, int U, int UT, bool HORIZ, bool REV, bool ACC>
__global__ __launch_bounds__(1024) GSPN_WAVES_PER_EU((waves_per_eu<HORIZ, P>()))
void scan_kernel(const ScanK a) {
    extern __shared__ float s_edge_raw[];
    const int64_t blk = blockIdx.x;
    const int64_t p = blk / a.nchunks;  // plane n * c + ci
    const int q = static_cast<int>(blk - p * a.nchunks);
    scan_line<T, TW, P, U, UT, HORIZ, REV, ACC>(a, p, q, s_edge_raw);
}

// ---------------------------------------------------------------------------
// Launch families
// ---------------------------------------------------------------------------

// Positions per lane (P in {1, 2, 4}: up to 1024 lanes per workgroup).
struct ScanConfig {
    int P;
};

#ifndef GSPN_SUB_U
#define GSPN_SUB_U 2
#endif

// Steps per prefetch sub-block and per tile.  One position per lane (lines
// up to 1024) keeps the sub-block short so that two 1024-lane workgroups fit a
// CU; two positions per lane serve lines up to 2048, which come in small
// numbers (few workgroups, each on the critical path), so their sub-block is
// deeper.  Horizontal tiles hold 16 steps (64 bytes of fp32 or 32 of bf16 per
// row) for one position per lane, fewer for more positions, so that the
// double buffers stay in registers.
#ifndef GSPN_SUB_U2
#define GSPN_SUB_U2 4
#endif

template <int P>
constexpr int sub_block_steps() {
    return P == 1 ? GSPN_SUB_U : (P == 2 ? GSPN_SUB_U2 : 2);
}

template <typename T, int P, bool HORIZ>
struct Blocking {
    static constexpr int U = sub_block_steps<P>();
    static constexpr int VW = 16 / static_cast<int>(sizeof(T));
    static constexpr int T0 = (16 / P) > VW ? (16 / P) : VW;
    static constexpr int UT = HORIZ ? (T0 > U ? T0 : U) : 2 * U;
};

template <typename T, typename TW, int P, bool HORIZ, bool REV, bool ACC>
hipError_t launch_one(const ScanK& k, int64_t nblocks, int nthreads, hipStream_t stream) {
    using B = Blocking<T, P, HORIZ>;
    const size_t lds = 4 * sizeof(float) * static_cast<size_t>(nthreads);
    hipLaunchKernelGGL((scan_kernel<T, TW, P, B::U, B::UT, HORIZ, REV, ACC>),
                       dim3(static_cast<unsigned>(nblocks)), dim3(nthreads), lds, stream, k);
    return hipGetLastError();
}

template <typename T, typename TW, int P, bool HORIZ>
hipError_t launch_p(bool rev, bool acc, const ScanK& k, int64_t nblocks, int nthreads, hipStream_t stream) {
    if constexpr (HORIZ) {
        if (rev) {
            return acc ? launch_one<T, TW, P, true, true, true>(k, nblocks, nthreads, stream)
                       : launch_one<T, TW, P, true, true, false>(k, nblocks, nthreads, stream);
        }
        return acc ? launch_one<T, TW, P, true, false, true>(k, nblocks, nthreads, stream)
                   : launch_one<T, TW, P, true, false, false>(k, nblocks, nthreads, stream);
    } else {
        return acc ? launch_one<T, TW, P, false, false, true>(k, nblocks, nthreads, stream)
                   : launch_one<T, TW, P, false, false, false>(k, nblocks, nthreads, stream);
    }
}

template <typename T, typename TW, bool HORIZ>
hipError_t launch_family(const ScanConfig& c, bool rev, bool acc, const ScanK& k, int64_t nblocks,
                         int nthreads, hipStream_t stream) {
    switch (c.P) {
        case 1: return launch_p<T, TW, 1, HORIZ>(rev, acc, k, nblocks, nthreads, stream);
        case 2: return launch_p<T, TW, 2, HORIZ>(rev, acc, k, nblocks, nthreads, stream);
        default: return launch_p<T, TW, 4, HORIZ>(rev, acc, k, nblocks, nthreads, stream);
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
    int group;       // long-line kernel: planes per workgroup
    int64_t planes;  // long-line kernel: planes per direction (n * c)
};

// Direction and index within it of block b of a four-direction launch:
// direction b % 4 when interleaved, else consecutive ranges.
GSPN_HD void scan4_block(const Scan4K& a, int64_t b, int& dir, int64_t& idx) {
    dir = 0;
    idx = b;
    if (a.interleave) {
        dir = static_cast<int>(b & 3);
        idx = b >> 2;
    } else {
        while (dir < 3 && idx >= a.blocks[dir]) {
            idx -= a.blocks[dir];
            ++dir;
        }
    }
}

template <typename T, typename TW, int PV, int PH>
__global__ __launch_bounds__(1024) void scan4_kernel(const Scan4K a) {
    extern __shared__ float s_edge_raw[];
    using BV = Blocking<T, PV, false>;
    using BH = Blocking<T, PH, true>;
    int dir;
    int64_t idx;
    scan4_block(a, blockIdx.x, dir, idx);
    const ScanK& k = a.d[dir];
    const int64_t p = idx / k.nchunks;
    const int q = static_cast<int>(idx - p * k.nchunks);
    switch (dir) {
        case 0:
        case 1: scan_line<T, TW, PV, BV::U, BV::UT, false, false, false>(k, p, q, s_edge_raw); break;
        case 2: scan_line<T, TW, PH, BH::U, BH::UT, true, false, false>(k, p, q, s_edge_raw); break;
        default: scan_line<T, TW, PH, BH::U, BH::UT, true, true, false>(k, p, q, s_edge_raw); break;
    }
}

// Four scans in one launch, all in the vertical form: the horizontal
// directions are described as vertical scans of the transposed input (their
// scan frame), so every access is a coalesced row.  PV / PH: positions per
// lane of the first two / last two scans.
template <typename T, typename TW, int PV, int PH, typename TO = T>
__global__ __launch_bounds__(1024)
GSPN_WAVES_PER_EU((waves_per_eu<false, (PV > PH ? PV : PH)>()))
void scan4v_kernel(const Scan4K a) {
    extern __shared__ float s_edge_raw[];
    using BV = Blocking<T, PV, false>;
    using BH = Blocking<T, PH, false>;
    int dir;
    int64_t idx;
    scan4_block(a, blockIdx.x, dir, idx);
    const ScanK& k = a.d[dir];
    const int64_t p = idx / k.nchunks;
    const int q = static_cast<int>(idx - p * k.nchunks);
    if (dir < 2) {
        scan_line<T, TW, PV, BV::U, BV::UT, false, false, false, TO>(k, p, q, s_edge_raw);
    } else {
        scan_line<T, TW, PH, BH::U, BH::UT, false, false, false, TO>(k, p, q, s_edge_raw);
    }
}

#ifdef GSPN_CHECK_LAUNCHES
// Host replay of scan4v_kernel (vertical-form scan_line, no accumulate): for
// every block and thread, each element access of every step at the offsets
// scan_line computes with the functions above (prefetches for steps t0 ..
// t1, clamped to the chunk's last row; stores by lanes on the line), and
// every LDS edge index against the launch's dynamic LDS.
template <typename T, typename TW, typename TO>
void replay_fused4v(const Scan4K& k, int pv, int ph, int nthreads, size_t lds) {
    const char* kn = "scan4v_kernel";
    constexpr bool PAIR = std::is_same_v<TW, WPair>;
    constexpr int ZE = PAIR ? 4 : static_cast<int>(sizeof(TW));
    constexpr int NZ = PAIR ? 1 : 3;
    constexpr int ES = static_cast<int>(sizeof(T));
    constexpr int EO = static_cast<int>(sizeof(TO));
    const int64_t nblocks = k.blocks[0] + k.blocks[1] + k.blocks[2] + k.blocks[3];
    int64_t bad = 0, n = 0;
    auto fail = [&](const char* what, int64_t b, int tid, int t) {
        if (bad++ < 4) check::violation(kn, what, "block %lld thread %d step %d", static_cast<long long>(b), tid, t);
    };
    for (int lane = 0; lane < nthreads; ++lane)
        if (static_cast<size_t>(scan_edge(1, 1, nthreads, lane) + 1) * 4 > lds) fail("edge LDS", -1, lane, -1);
    check::Region rx[4], rl[4], ro[4], rz[4];
    for (int d = 0; d < 4; ++d) {
        rx[d] = check::region_of(k.d[d].x, kn, "x");
        rl[d] = check::region_of(k.d[d].lam, kn, "lambda");
        ro[d] = check::region_of(k.d[d].out, kn, "out");
        rz[d] = check::region_of(k.d[d].wts, kn, "weights");
    }
    for (int64_t b = 0; b < nblocks; ++b) {
        int dir;
        int64_t idx;
        scan4_block(k, b, dir, idx);
        const ScanK& a = k.d[dir];
        const int P = dir < 2 ? pv : ph;
        const int64_t p = idx / a.nchunks;
        const int q = static_cast<int>(idx - p * a.nchunks);
        const int S = a.S, L = a.L;
        const int64_t plane = static_cast<int64_t>(S) * L;
        const int t0 = q * a.K;
        const int t1 = (t0 + a.K < S) ? t0 + a.K : S;
        const bool rev = a.reverse != 0;
        const char* xb = static_cast<const char*>(a.x) + p * plane * ES;
        const char* lb = static_cast<const char*>(a.lam) + p * plane * ES;
        const char* ob = static_cast<const char*>(a.out) + p * plane * EO;
        const char* zb = static_cast<const char*>(a.wts) + scan_weight_offset(a, p, plane, PAIR) * ZE;
        for (int tid = 0; tid < nthreads; ++tid) {
            const int k0 = tid * P;
            for (int t = t0; t <= t1; ++t) {
                const int64_t lo = static_cast<int64_t>(scan_row(scan_fetch_step(t, t1), S, rev)) * L;
                for (int j = 0; j < P; ++j) {
                    const int64_t e = lo + scan_pos(k0 + j, L);
                    for (int o = 0; o < NZ; ++o)
                        if (!check::in_region(rz[dir], zb, (o * plane + e) * ZE, ZE)) fail("weight load", b, tid, t);
                    if (!check::in_region(rl[dir], lb, e * ES, ES)) fail("lambda load", b, tid, t);
                    if (!check::in_region(rx[dir], xb, e * ES, ES)) fail("x load", b, tid, t);
                    n += NZ + 2;
                    if (t < t1 && k0 + j < L) {
                        const int64_t so = static_cast<int64_t>(scan_row(t, S, rev)) * L + k0 + j;
                        if (!check::in_region(ro[dir], ob, so * EO, EO)) fail("store", b, tid, t);
                        ++n;
                    }
                }
            }
        }
    }
    if (bad) check::violation(kn, "accesses", "%lld bad", static_cast<long long>(bad));
    check::count_accesses(n);
    check::replayed(kn, 1024, 0);
}
#endif

template <typename T, typename TW, typename TO = T>
hipError_t launch_fused4v(const Scan4K& k, int pv, int ph, int nthreads, hipStream_t stream) {
    const int64_t nblocks = k.blocks[0] + k.blocks[1] + k.blocks[2] + k.blocks[3];
    const size_t lds = 4 * sizeof(float) * static_cast<size_t>(nthreads);
    const dim3 grid(static_cast<unsigned>(nblocks));
#ifdef GSPN_CHECK_LAUNCHES
    replay_fused4v<T, TW, TO>(k, pv, ph, nthreads, lds);
#endif
    if (pv == 1 && ph == 1) {
        hipLaunchKernelGGL((scan4v_kernel<T, TW, 1, 1, TO>), grid, dim3(nthreads), lds, stream, k);
    } else if (pv == 1) {
        hipLaunchKernelGGL((scan4v_kernel<T, TW, 1, 2, TO>), grid, dim3(nthreads), lds, stream, k);
    } else if (ph == 1) {
        hipLaunchKernelGGL((scan4v_kernel<T, TW, 2, 1, TO>), grid, dim3(nthreads), lds, stream, k);
    } else {
        hipLaunchKernelGGL((scan4v_kernel<T, TW, 2, 2, TO>), grid, dim3(nthreads), lds, stream, k);
    }
    return hipGetLastError();
}

template <typename T, typename TW>
hipError_t launch_fused4(const Scan4K& k, int pv, int ph, int nthreads, hipStream_t stream) {
    const int64_t nblocks = k.blocks[0] + k.blocks[1] + k.blocks[2] + k.blocks[3];
    const size_t lds = 4 * sizeof(float) * static_cast<size_t>(nthreads);
    const dim3 grid(static_cast<unsigned>(nblocks));
    if (pv == 1 && ph == 1) {
        hipLaunchKernelGGL((scan4_kernel<T, TW, 1, 1>), grid, dim3(nthreads), lds, stream, k);
    } else if (pv == 1) {
        hipLaunchKernelGGL((scan4_kernel<T, TW, 1, 2>), grid, dim3(nthreads), lds, stream, k);
    } else if (ph == 1) {
        hipLaunchKernelGGL((scan4_kernel<T, TW, 2, 1>), grid, dim3(nthreads), lds, stream, k);
    } else {
        hipLaunchKernelGGL((scan4_kernel<T, TW, 2, 2>), grid, dim3(nthreads), lds, stream, k);
    }
    return hipGetLastError();
}

}  // namespace gspn
