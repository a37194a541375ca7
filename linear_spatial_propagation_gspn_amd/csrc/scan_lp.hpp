// scan_lp.hpp -- the four-direction line scan for few, long lines (internal
// to libgspn; instantiated in scan4_*.hip).
//
// Same recurrence as scan_kernel.hpp (GSPN-2 paper notes, "2D spatial
// propagation recap"; chunks from "Optimisation 1"), for the case where the
// (plane, chunk) lines of a forward are too few to fill the GPU, e.g. the
// eight proxy-space planes of 2048 positions in the compressive-proxy
// pipeline ("Optimisation 2").  There each workgroup owns a CU by itself and
// the time per scan step is the latency of one step, not bandwidth, so the
// kernel minimises the work on the step's critical path:
//  - each lane owns P contiguous positions (16 bytes of the storage type), so
//    every stream moves one 16-byte vector per lane and step, and the line
//    needs few waves (256 lanes for 2048 bf16 positions);
//  - loads and stores go through buffer resources: the lane's byte offset is
//    fixed for the whole scan and the step's row offset is a scalar, so no
//    vector address arithmetic runs per step;
//  - the neighbour values inside a wave move with DPP lane shifts; only the
//    two wave-edge values of each wave go through LDS, with one barrier per
//    step;
//  - the inputs of the next D steps are in flight at all times: D ring slots,
//    each refilled as soon as its step has read it (the loop is unrolled by
//    D so the slot indices are compile-time constants).
// All four directions are described in vertical form (the horizontal ones on
// x transposed into their scan frame), as for scan4v_kernel.  The outputs are
// the unweighted scans: learnable merge weights are applied where the
// separate outputs are merged.
#pragma once

#include <utility>

#include "coltile.hpp"
#include "scan_kernel.hpp"

namespace gspn {

namespace lp {

constexpr int kMaxLanes = 256;
constexpr int kMaxWaves = kMaxLanes / 64;

#ifndef GSPN_LP_DEPTH
#define GSPN_LP_DEPTH 6
#endif

// Raw buffer resource over `bytes` bytes from `base` (untyped dword accesses).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

typedef int int4v __attribute__((ext_vector_type(4)));

// Cache policy: streams that are touched once (lambda, per-channel logits,
// the outputs) go with the non-temporal hint (buffer instruction bit 1),
// which measured 7% faster on the 1024^2, B=16, C=8 fp32 scan; weights shared
// by many channels keep the default policy, since every channel re-reads
// them (with the hint they ran 40% slower).
#ifndef GSPN_LP_STREAM_AUX
#define GSPN_LP_STREAM_AUX 2
#endif
#ifndef GSPN_LP_X_AUX
#define GSPN_LP_X_AUX 0
#endif

// W 32-bit words from the buffer at voff + soff (W a multiple of 4).
template <int W, int AUX = 0>
__device__ __forceinline__ void load_words(uint32_t (&d)[W], __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff) {
#pragma unroll
    for (int v = 0; v < W / 4; ++v) {
        const int4v q = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * v, soff, AUX);
#pragma unroll
        for (int e = 0; e < 4; ++e) d[4 * v + e] = static_cast<uint32_t>(q[e]);
    }
}

// Element j of P values of type E packed in 32-bit words, widened to fp32.
template <typename E, int W>
__device__ __forceinline__ float elem(const uint32_t (&w)[W], int j) {
    if constexpr (sizeof(E) == 4) {
        return __uint_as_float(w[j]);
    } else {
        const uint32_t word = w[j >> 1];
        return __uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16));
    }
}

__device__ __forceinline__ float shift_from_lower_lane(float v) {  // lane i gets lane i-1 (0 for lane 0)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, true));
}

__device__ __forceinline__ float shift_from_upper_lane(float v) {  // lane i gets lane i+1 (0 for lane 63)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xf, 0xf, true));
}

}  // namespace lp

// Index code of lp_line and scan4lp_kernel, shared with the host replay.

// Byte offsets of a lane's vector in a row of x and lambda (vt), of one
// weight row (vw) and of the output (vo): the lane's first position, or for
// a lane past the line (or of an invalid plane) the line's last vector.
struct LpLane {
    uint32_t vt, vw, vo;
    bool active;  // the lane holds positions of a line
};

GSPN_HD LpLane lp_lane(int tid, bool valid, int L, int P, int es, int zb, int eo) {
    const int k0 = tid * P;
    const bool active = valid && k0 < L;
    const uint32_t k0c = static_cast<uint32_t>(active ? k0 : L - P);
    return {k0c * static_cast<uint32_t>(es), k0c * static_cast<uint32_t>(zb), k0c * static_cast<uint32_t>(eo),
            active};
}

// Bytes from a.wts to the weight rows of plane p (zb bytes a position and row).
GSPN_HD int64_t lp_weight_offset(const ScanK& a, int64_t p, int64_t plane, bool pair, int zb) {
    return scan_weight_offset(a, p, plane, pair) * zb;
}

// Row of scan step t; the step whose row a fill for step t reads (steps past
// the chunk read its last row).
GSPN_HD uint32_t lp_row(int t, int S, bool rev) { return static_cast<uint32_t>(scan_row(t, S, rev)); }
GSPN_HD int lp_fill_step(int t, int t1) { return scan_fetch_step(t, t1); }

// The plane and waves of member g of a long-line workgroup: a.group planes
// share it, per threads each.
struct LpMember {
    int64_t p;    // plane (clamped to an existing one when invalid)
    bool valid;
    int tid;      // thread index within the member
    int wave0;    // the member's first wave
    int nwaves;
};

GSPN_HD LpMember lp_member(const Scan4K& a, int64_t pg, int g, int per, int tid) {
    const int64_t p = pg * a.group + g;
    const bool valid = p < a.planes;
    return {valid ? p : a.planes - 1, valid, tid - g * per, g * (per >> 6), per >> 6};
}

// Column tiles for the horizontal directions' x (XT): whole 128-byte runs of
// every row of the array-frame plane, 128 KB of LDS for lines of 1024
// positions, the next tile in flight in registers (fp32 only: one 256-lane
// workgroup a line).
using LpXTile = coltile::Tile<float, lp::kMaxLanes, 128>;
// steps in flight (a divisor of the tile's 32 steps): 4 and 8 measured the
// same, 2 and 16 slower (profile step 3.08 and 4.35 ms against 2.70)
#ifndef GSPN_LP_XT_DEPTH
#define GSPN_LP_XT_DEPTH 4
#endif
// cache policy of the column tiles' loads: non-temporal (the opposite
// direction reads x again only a whole scan later); with the default policy
// the profile scan took 2.44 ms against 2.26
#ifndef GSPN_LP_XTILE_AUX
#define GSPN_LP_XTILE_AUX 2
#endif

// One (plane, chunk) line of a vertical-form scan, run by `nwaves` waves of
// the workgroup starting at wave `wave0`; tid is the thread's index among
// them.  valid = false: the waves only keep step with the workgroup's
// barriers (p is then any existing plane).  T: storage of x, lambda and the
// output; TW: storage of the weights (WPair: packed half pairs of
// channel-shared weights); LOGITS: the weights are logits normalised here
// (else normalised weights, zero outside the line).  XT: a horizontal
// direction whose x is the array-frame plane [L][S] (a.xtile), its column
// i read from an LDS column tile instead of row i of x transposed; one
// unchunked line a workgroup of lp::kMaxLanes threads (tid = threadIdx.x),
// S a multiple of the tile's 32 steps.
template <typename T, typename TW, bool LOGITS, typename TO = T, bool XT = false>
__device__ __forceinline__ void lp_line(const ScanK& a, int64_t p, int q, bool valid, int tid, int wave0,
                                        int nwaves) {
    constexpr int P = 16 / static_cast<int>(sizeof(T));              // positions per lane
    constexpr int WT = P * static_cast<int>(sizeof(T)) / 4;          // words per lane: x, lambda, out
    constexpr bool PAIR = std::is_same_v<TW, WPair>;
    constexpr int ZB = PAIR ? 4 : static_cast<int>(sizeof(TW));      // weight bytes per position and row
    constexpr int NZ = PAIR ? 1 : 3;                                  // weight rows
    constexpr int WW = P * ZB / 4;                                    // words per lane: one weight row
    constexpr int D = XT ? GSPN_LP_XT_DEPTH : GSPN_LP_DEPTH;          // steps in flight
    static_assert(!XT || sizeof(T) == 4, "column tiles of fp32 x only");
    __shared__ float edges[2][lp::kMaxWaves][2];
    __shared__ uint32_t xtl[XT ? coltile::tile_dwords<128>() : 1];

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int S = a.S;
    const int L = a.L;
    const int64_t plane = static_cast<int64_t>(S) * L;

    const auto rx = lp::rsrc(static_cast<const T*>(a.x) + p * plane, plane * sizeof(T));
    const auto rl = lp::rsrc(static_cast<const T*>(a.lam) + p * plane, plane * sizeof(T));
    const auto ro = lp::rsrc(static_cast<TO*>(a.out) + p * plane, plane * sizeof(TO));
    const auto rz = lp::rsrc(static_cast<const char*>(a.wts) + lp_weight_offset(a, p, plane, PAIR, ZB),
                             NZ * plane * ZB);

    const int k0 = tid * P;
    // lanes past the line read its last vector (unused)
    const LpLane ln = lp_lane(tid, valid, L, P, sizeof(T), ZB, sizeof(TO));
    const bool active = ln.active;
    const uint32_t vt = ln.vt;
    const uint32_t vw = ln.vw;
    const uint32_t rowT = static_cast<uint32_t>(L) * sizeof(T);
    const uint32_t vo = ln.vo;
    const uint32_t rowO = static_cast<uint32_t>(L) * sizeof(TO);
    const uint32_t rowW = static_cast<uint32_t>(L) * ZB;
    const uint32_t planeW = static_cast<uint32_t>(plane) * ZB;
    const bool has_l0 = k0 > 0;       // the lane's first position has a left neighbour
    const bool has_rP = k0 + P < L;   // the lane's last position has a right neighbour

    const int t0 = q * a.K;
    const int t1 = min(t0 + a.K, S);
    const bool rev = a.reverse != 0;
    auto line_of = [&](int t) { return lp_row(t, S, rev); };

    uint32_t sx[XT ? 1 : D][WT], sl[D][WT], sz[D][NZ][WW];
    auto fill = [&](auto slot, int t) {
        constexpr int s = decltype(slot)::value;
        const uint32_t i = line_of(lp_fill_step(t, t1));
        if constexpr (!XT) lp::load_words<WT, GSPN_LP_X_AUX>(sx[s], rx, vt, i * rowT);
        lp::load_words<WT, GSPN_LP_STREAM_AUX>(sl[s], rl, vt, i * rowT);
        // logits are per channel here unless a single channel shares them;
        // normalised weights are always shared
        constexpr int ZAUX = LOGITS ? GSPN_LP_STREAM_AUX : 0;
#pragma unroll
        for (int o = 0; o < NZ; ++o) lp::load_words<WW, ZAUX>(sz[s][o], rz, vw, o * planeW + i * rowW);
    };

    float h[P];
#pragma unroll
    for (int j = 0; j < P; ++j) h[j] = 0.0f;
    int buf = 0;

    // Step t from slot s; FIRST: the first line of the chunk (h_prev = 0 and
    // its weights unused).  The slot is refilled with step t + D.
    // the x words of step t: the ring slot, or (XT) the lane's positions of
    // the tile row of x's column line_of(t)
    const int k0c = active ? k0 : L - P;
    auto x_words = [&](auto slot, int t, uint32_t (&xw)[WT]) {
        constexpr int s = decltype(slot)::value;
        if constexpr (XT) {
            const int tt = static_cast<int>(line_of(t)) % LpXTile::TS;
            const lp::int4v v = *reinterpret_cast<const lp::int4v*>(xtl + tt * LpXTile::row_stride(L) + k0c);
#pragma unroll
            for (int e = 0; e < 4; ++e) xw[e] = static_cast<uint32_t>(v[e]);
        } else {
#pragma unroll
            for (int e = 0; e < WT; ++e) xw[e] = sx[s][e];
        }
    };

    auto step = [&](auto slot, auto firstc, int t) {
        constexpr int s = decltype(slot)::value;
        constexpr bool FIRST = decltype(firstc)::value != 0;
        uint32_t xw[WT];
        x_words(slot, t, xw);
        float hn[P];
        if constexpr (FIRST) {
#pragma unroll
            for (int j = 0; j < P; ++j) hn[j] = lp::elem<T, WT>(sl[s], j) * lp::elem<T, WT>(xw, j);
        } else if constexpr (PAIR) {
            // h + w_{k-1} (h_{k-1} - h) + w_{k+1} (h_{k+1} - h) + lambda x: the
            // same row-stochastic combination with the centre weight
            // (1 - w_{k-1} - w_{k+1}) eliminated, so the half-precision side
            // weights enter the fused multiply-adds as they are stored, and two
            // neighbouring positions share one difference.
            const float eleft = wave > 0 ? edges[buf][wave0 + wave - 1][1] : 0.0f;
            const float eright = wave + 1 < nwaves ? edges[buf][wave0 + wave + 1][0] : 0.0f;
            const float dl = lp::shift_from_lower_lane(h[P - 1]);
            const float dr = lp::shift_from_upper_lane(h[0]);
            const float left = lane == 0 ? eleft : dl;
            const float right = lane == 63 ? eright : dr;
            float dd[P + 1];  // dd[j] = h[j] - h[j - 1], with h[-1] = left and h[P] = right
            dd[0] = h[0] - left;
#pragma unroll
            for (int j = 1; j < P; ++j) dd[j] = h[j] - h[j - 1];
            dd[P] = right - h[P - 1];
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const float base = __builtin_fmaf(lp::elem<T, WT>(sl[s], j), lp::elem<T, WT>(xw, j), h[j]);
                hn[j] = __builtin_fmaf(pair_hi(sz[s][0][j]), dd[j + 1], __builtin_fmaf(pair_lo(sz[s][0][j]), -dd[j], base));
            }
        } else {
            float u[P];
#pragma unroll
            for (int j = 0; j < P; ++j) u[j] = lp::elem<T, WT>(sl[s], j) * lp::elem<T, WT>(xw, j);
            float w[3][P];
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const float z0 = lp::elem<TW, WW>(sz[s][0], j);
                const float z1 = lp::elem<TW, WW>(sz[s][NZ > 1 ? 1 : 0], j);
                const float z2 = lp::elem<TW, WW>(sz[s][NZ > 2 ? 2 : 0], j);
                if constexpr (LOGITS) {
                    const bool hl = j > 0 || has_l0;
                    const bool hr = j < P - 1 || has_rP;
                    normalise_row(z0, z1, z2, hl, hr, w[0][j], w[1][j], w[2][j]);
                } else {
                    w[0][j] = z0;
                    w[1][j] = z1;
                    w[2][j] = z2;
                }
            }
            // neighbours from the previous step: inside the wave by DPP, across
            // wave edges from LDS (0 beyond the line)
            const float eleft = wave > 0 ? edges[buf][wave0 + wave - 1][1] : 0.0f;
            const float eright = wave + 1 < nwaves ? edges[buf][wave0 + wave + 1][0] : 0.0f;
            const float dl = lp::shift_from_lower_lane(h[P - 1]);
            const float dr = lp::shift_from_upper_lane(h[0]);
            const float left = lane == 0 ? eleft : dl;
            const float right = lane == 63 ? eright : dr;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const float hl = j == 0 ? left : h[j - 1];
                const float hr = j == P - 1 ? right : h[j + 1];
                hn[j] = __builtin_fmaf(w[0][j], hl, __builtin_fmaf(w[1][j], h[j], __builtin_fmaf(w[2][j], hr, u[j])));
            }
        }
        fill(slot, t + D);
        // only h[0] of a lane past the line reaches a position on it (as the
        // right neighbour of the line's last position, whose weight to it is
        // 0), so only h[0] is cleared there
        h[0] = active ? hn[0] : 0.0f;
#pragma unroll
        for (int j = 1; j < P; ++j) h[j] = hn[j];
        if (active) {
            constexpr int WO = P * static_cast<int>(sizeof(TO)) / 4;  // output words per lane
            uint32_t ow[WO];
            if constexpr (sizeof(TO) == 4) {
#pragma unroll
                for (int e = 0; e < WO; ++e) ow[e] = __float_as_uint(h[e]);
            } else {
#pragma unroll
                for (int e = 0; e < WO; ++e) ow[e] = pack_bf16x2(h[2 * e], h[2 * e + 1]);
            }
#pragma unroll
            for (int v = 0; v < WO / 4; ++v) {
                const lp::int4v o = {static_cast<int>(ow[4 * v]), static_cast<int>(ow[4 * v + 1]),
                                     static_cast<int>(ow[4 * v + 2]), static_cast<int>(ow[4 * v + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(o, ro, vo + 16 * v, line_of(t) * rowO, GSPN_LP_STREAM_AUX);
            }
        }
        buf ^= 1;
        if (lane == 0) edges[buf][wave0 + wave][0] = h[0];
        if (lane == 63) edges[buf][wave0 + wave][1] = h[P - 1];
        __syncthreads();
    };

    if constexpr (XT) {
        // One loop iteration per column tile of TS steps, its steps unrolled
        // (TS a multiple of D, so the ring slots are compile-time): the next
        // tile's loads are issued at the top, a whole tile ahead, and the
        // first tile's first step is peeled (h_prev = 0).  Lanes past the
        // line read the line's last positions (k0c) and store nothing.
        constexpr int TS = LpXTile::TS;
        static_assert(TS % D == 0, "ring slots align with tiles");
        LpXTile tl;
        const int R = L, C = S;  // x [L][S]: the line's positions are its rows, the steps its columns
        auto block_of = [&](int t) { return static_cast<int>(line_of(t)) / TS * TS; };
        tl.template load<GSPN_LP_XTILE_AUX>(rx, R, C, block_of(0), tid);
        [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
            (fill(IC<Ss>{}, Ss), ...);
        }(std::make_integer_sequence<int, D>{});
        // every lane is past the previous tile (the last step's barrier)
        tl.store(xtl, R, tid);
        __syncthreads();
        tl.template load<GSPN_LP_XTILE_AUX>(rx, R, C, block_of(TS < S ? TS : S - 1), tid);
        step(IC<0>{}, IC<1>{}, 0);
        [&]<int... Js>(std::integer_sequence<int, Js...>) {
            (step(IC<(Js + 1) % D>{}, IC<0>{}, Js + 1), ...);
        }(std::make_integer_sequence<int, TS - 1>{});
        for (int tb = TS; tb < S; tb += TS) {
            tl.store(xtl, R, tid);
            __syncthreads();
            tl.template load<GSPN_LP_XTILE_AUX>(rx, R, C, block_of(tb + TS < S ? tb + TS : S - 1), tid);
            [&]<int... Js>(std::integer_sequence<int, Js...>) {
                (step(IC<Js % D>{}, IC<0>{}, tb + Js), ...);
            }(std::make_integer_sequence<int, TS>{});
        }
        return;
    }

    // prologue: D steps in flight, then the chunk's first line
    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        (fill(IC<Ss>{}, t0 + Ss), ...);
    }(std::make_integer_sequence<int, D>{});
    step(IC<0>{}, IC<1>{}, t0);

    // main loop: D steps per iteration, slots 1, 2, .., D-1, 0
    int t = t0 + 1;
    for (; t + D <= t1; t += D) {
        [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
            (step(IC<(Ss + 1) % D>{}, IC<0>{}, t + Ss), ...);
        }(std::make_integer_sequence<int, D>{});
    }
    // tail: fewer than D steps, uniform guards around whole steps
    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        ((t + Ss < t1 ? step(IC<(Ss + 1) % D>{}, IC<0>{}, t + Ss) : void()), ...);
    }(std::make_integer_sequence<int, D - 1>{});
}

// Four vertical-form scans in one launch; block b is direction b % 4 when the
// directions have equal block counts (Scan4K::interleave), else consecutive
// ranges, as in scan4v_kernel.
template <typename T, typename TW, bool LOGITS, typename TO = T, bool XT = false>
__global__ __launch_bounds__(lp::kMaxLanes) void scan4lp_kernel(const Scan4K a) {
    int dir;
    int64_t idx;
    scan4_block(a, blockIdx.x, dir, idx);
    const ScanK& k = a.d[dir];
    const int64_t pg = idx / k.nchunks;
    const int q = static_cast<int>(idx - pg * k.nchunks);
    // a.group consecutive planes share the workgroup, each on its own waves;
    // with channel-shared weights their weight loads coincide in time, so all
    // but the first are served by the cache
    const int per = static_cast<int>(blockDim.x) / a.group;
    // per is a whole number of waves, so g is uniform in the wave: say so, to
    // keep the plane's buffer resources in scalar registers
    const int g = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / per);
    const LpMember m = lp_member(a, pg, g, per, static_cast<int>(threadIdx.x));
    if constexpr (XT) {
        // the horizontal directions through column tiles, the vertical ones as usual
        if (k.xtile) lp_line<T, TW, LOGITS, TO, true>(k, m.p, q, m.valid, m.tid, m.wave0, m.nwaves);
        else lp_line<T, TW, LOGITS, TO, false>(k, m.p, q, m.valid, m.tid, m.wave0, m.nwaves);
    } else {
        lp_line<T, TW, LOGITS, TO>(k, m.p, q, m.valid, m.tid, m.wave0, m.nwaves);
    }
}

#ifdef GSPN_CHECK_LAUNCHES
// Host replay of scan4lp_kernel: for every block, member and thread, the
// buffer resources of its plane and each 16-byte access of every step, at
// the offsets lp_line computes with the functions above (fills for steps t0
// .. t1 + D - 1, the last D of them clamped to the chunk's last row; stores
// for the chunk's steps by active lanes).  An access must lie in its
// tensor's buffer and inside its resource (the hardware would drop it
// silently otherwise).
template <typename T, typename TW, bool LOGITS, typename TO, bool XT>
void replay_fused4lp(const Scan4K& k, int nthreads) {
    const char* kn = "scan4lp_kernel";
    constexpr int P = 16 / static_cast<int>(sizeof(T));
    constexpr int WT = P * static_cast<int>(sizeof(T)) / 4;
    constexpr bool PAIR = std::is_same_v<TW, WPair>;
    constexpr int ZB = PAIR ? 4 : static_cast<int>(sizeof(TW));
    constexpr int NZ = PAIR ? 1 : 3;
    constexpr int WW = P * ZB / 4;
    constexpr int WO = P * static_cast<int>(sizeof(TO)) / 4;
    constexpr int D = XT ? GSPN_LP_XT_DEPTH : GSPN_LP_DEPTH;
    const int64_t nblocks = k.blocks[0] + k.blocks[1] + k.blocks[2] + k.blocks[3];
    if (k.group < 1 || nthreads % k.group != 0 || (nthreads / k.group) % 64 != 0)
        check::violation(kn, "block", "%d threads do not split into %d whole-wave members", nthreads, k.group);
    const int per = nthreads / k.group;
    check::Region rx[4], rl[4], ro[4], rz[4];
    for (int d = 0; d < 4; ++d) {
        rx[d] = check::region_of(k.d[d].x, kn, "x");
        rl[d] = check::region_of(k.d[d].lam, kn, "lambda");
        ro[d] = check::region_of(k.d[d].out, kn, "out");
        rz[d] = check::region_of(k.d[d].wts, kn, "weights");
    }
    int64_t bad = 0, n = 0;
    auto fail = [&](const char* what, int64_t b, int tid, int t) {
        if (bad++ < 4) check::violation(kn, what, "block %lld thread %d step %d", static_cast<long long>(b), tid, t);
    };
    for (int64_t b = 0; b < nblocks; ++b) {
        int dir;
        int64_t idx;
        scan4_block(k, b, dir, idx);
        const ScanK& a = k.d[dir];
        const int64_t pg = idx / a.nchunks;
        const int q = static_cast<int>(idx - pg * a.nchunks);
        const int S = a.S, L = a.L;
        const int64_t plane = static_cast<int64_t>(S) * L;
        const int t0 = q * a.K;
        const int t1 = (t0 + a.K < S) ? t0 + a.K : S;
        const bool rev = a.reverse != 0;
        if (L % P != 0 || L < P) fail("line not whole vectors", b, -1, -1);
        for (int g = 0; g < k.group; ++g) {
            const LpMember m = lp_member(k, pg, g, per, g * per);
            if (m.wave0 + m.nwaves > lp::kMaxWaves) fail("edge LDS", b, g * per, -1);
            // the resources: the plane of x, lambda and out, the weight rows
            const char* xb = static_cast<const char*>(a.x) + m.p * plane * static_cast<int64_t>(sizeof(T));
            const char* lb = static_cast<const char*>(a.lam) + m.p * plane * static_cast<int64_t>(sizeof(T));
            const char* ob = static_cast<const char*>(a.out) + m.p * plane * static_cast<int64_t>(sizeof(TO));
            const char* zb = static_cast<const char*>(a.wts) + lp_weight_offset(a, m.p, plane, PAIR, ZB);
            const int64_t nt = plane * static_cast<int64_t>(sizeof(T));
            const int64_t no = plane * static_cast<int64_t>(sizeof(TO));
            const int64_t nz = NZ * plane * ZB;
            if (nt > 0x7fffffff || no > 0x7fffffff || nz > 0x7fffffff) fail("resource past 2^31 bytes", b, -1, -1);
            if (!check::in_region(rx[dir], xb, 0, nt)) fail("x resource", b, -1, -1);
            if (!check::in_region(rl[dir], lb, 0, nt)) fail("lambda resource", b, -1, -1);
            if (!check::in_region(ro[dir], ob, 0, no)) fail("out resource", b, -1, -1);
            if (!check::in_region(rz[dir], zb, 0, nz)) fail("weight resource", b, -1, -1);
            const uint32_t rowT = static_cast<uint32_t>(L) * sizeof(T);
            const uint32_t rowO = static_cast<uint32_t>(L) * sizeof(TO);
            const uint32_t rowW = static_cast<uint32_t>(L) * ZB;
            const uint32_t planeW = static_cast<uint32_t>(plane) * ZB;
            for (int tid = g * per; tid < (g + 1) * per; ++tid) {
                const LpMember mt = lp_member(k, pg, g, per, tid);
                const LpLane ln = lp_lane(mt.tid, mt.valid, L, P, sizeof(T), ZB, sizeof(TO));
                const bool xt = XT && a.xtile;
                if (xt) {
                    // column tiles of x [L][S]: every tile's loads (the next
                    // tile's at the top of each, the last reloading its own)
                    // and the lane's tile-row reads
                    constexpr int TS = LpXTile::TS;
                    if (S % TS != 0 || k.group != 1 || nthreads != lp::kMaxLanes || a.nchunks != 1)
                        fail("column tiles", b, tid, -1);
                    for (int tb = 0; tb <= S; tb += TS) {
                        const int c0 = lp_row(tb < S ? tb : S - 1, S, rev) / TS * TS;
                        for (int qd = 0; qd < LpXTile::NQ; ++qd) {
                            const int64_t off = coltile::chunk_offset(qd * lp::kMaxLanes + tid, L, S, c0, 4,
                                                                      LpXTile::CPR);
                            if (off + 16 > nt || !check::in_region(rx[dir], xb, off, 16)) fail("x tile load", b, tid, tb);
                        }
                        n += LpXTile::NQ;
                    }
                    const int k0c = ln.active ? mt.tid * P : L - P;
                    if ((TS - 1) * LpXTile::row_stride(L) + k0c + 4 > coltile::tile_dwords<128>())
                        fail("x tile LDS read", b, tid, -1);
                }
                for (int t = t0; t < t1 + D; ++t) {
                    const uint32_t i = lp_row(lp_fill_step(t, t1), S, rev);
                    for (int v = 0; v < WT / 4; ++v) {
                        const int64_t off = static_cast<int64_t>(ln.vt) + 16 * v + static_cast<int64_t>(i) * rowT;
                        if (!xt && (off + 16 > nt || !check::in_region(rx[dir], xb, off, 16))) fail("x load", b, tid, t);
                        if (off + 16 > nt || !check::in_region(rl[dir], lb, off, 16)) fail("lambda load", b, tid, t);
                    }
                    for (int o = 0; o < NZ; ++o)
                        for (int v = 0; v < WW / 4; ++v) {
                            const int64_t off = static_cast<int64_t>(ln.vw) + 16 * v +
                                                static_cast<int64_t>(o) * planeW + static_cast<int64_t>(i) * rowW;
                            if (off + 16 > nz || !check::in_region(rz[dir], zb, off, 16)) fail("weight load", b, tid, t);
                        }
                    n += 2 * (WT / 4) + NZ * (WW / 4);
                    if (ln.active && t < t1) {
                        const uint32_t io = lp_row(t, S, rev);
                        for (int v = 0; v < WO / 4; ++v) {
                            const int64_t off = static_cast<int64_t>(ln.vo) + 16 * v + static_cast<int64_t>(io) * rowO;
                            if (off + 16 > no || !check::in_region(ro[dir], ob, off, 16)) fail("store", b, tid, t);
                        }
                        n += WO / 4;
                    }
                }
            }
        }
    }
    if (bad) check::violation(kn, "accesses", "%lld bad", static_cast<long long>(bad));
    check::count_accesses(n);
    check::replayed(kn, lp::kMaxLanes,
                    sizeof(float) * 2 * lp::kMaxWaves * 2 + (XT ? 4 * coltile::tile_dwords<128>() : 0));
}
#endif

// Waves of the long-line scan resident on one CU (a build parameter; 0: as
// many as registers allow).  Each step of a line streams a whole row of
// every input, so the CU's share of bandwidth, not its wave count, bounds the
// step; fewer resident lines each step faster.  On the 1024^2, B=16, C=8 fp32
// forward (512 workgroups of four waves) one workgroup per CU ran the scan in
// 2.33 ms, two rounds, against 2.47 ms with two workgroups per CU in one
// round; the wide backward's recompute (2304 workgroups) gained 1.8 ms.  The
// launch reserves LDS it does not use so that no more workgroups fit, and
// only when the grid is whole rounds of them (or many rounds), since a last
// round that is mostly empty would cost more than the gain.
#ifndef GSPN_LP_WAVES_PER_CU
#define GSPN_LP_WAVES_PER_CU 4
#endif
// Only workgroups of at least this many waves (lines of at least 1024
// positions at four waves): short lines are bound by the latency of their
// steps, which more resident workgroups hide.
#ifndef GSPN_LP_RESERVE_MIN_WAVES
#define GSPN_LP_RESERVE_MIN_WAVES 4
#endif
constexpr int64_t kCuLdsBytes = 160 * 1024;

// Dynamic LDS to reserve for nblocks workgroups of nthreads on cus CUs.
GSPN_HD size_t lp_lds_reserve(int64_t nblocks, int nthreads, int64_t cus) {
    const int waves = (nthreads + 63) / 64;
    if (GSPN_LP_WAVES_PER_CU <= 0 || cus <= 0 || waves < GSPN_LP_RESERVE_MIN_WAVES || waves <= 0) return 0;
    const int64_t per_cu = GSPN_LP_WAVES_PER_CU / waves > 1 ? GSPN_LP_WAVES_PER_CU / waves : 1;
    const int64_t round = per_cu * cus;
    if (nblocks < round || (nblocks % round != 0 && nblocks < 4 * round)) return 0;
    // per_cu workgroups fit, one more does not (the edge buffers' few static
    // bytes aside)
    return static_cast<size_t>(kCuLdsBytes / (per_cu + 1) + 1024);
}

// XT: the horizontal directions marked xtile read x through column tiles;
// their 128 KB of static LDS already leave one workgroup a CU, so no LDS is
// reserved.
template <typename T, typename TW, bool LOGITS, typename TO = T, bool XT = false>
hipError_t launch_fused4lp(const Scan4K& k, int nthreads, hipStream_t stream) {
    const int64_t nblocks = k.blocks[0] + k.blocks[1] + k.blocks[2] + k.blocks[3];
#ifdef GSPN_CHECK_LAUNCHES
    replay_fused4lp<T, TW, LOGITS, TO, XT>(k, nthreads);
#endif
    const size_t reserve = XT ? 0 : lp_lds_reserve(nblocks, nthreads, device_compute_units());
    hipLaunchKernelGGL((scan4lp_kernel<T, TW, LOGITS, TO, XT>), dim3(static_cast<unsigned>(nblocks)), dim3(nthreads),
                       reserve, stream, k);
    return hipGetLastError();
}

}  // namespace gspn
