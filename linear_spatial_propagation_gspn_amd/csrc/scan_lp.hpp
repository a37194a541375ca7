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

// One (plane, chunk) line of a vertical-form scan, run by `nwaves` waves of
// the workgroup starting at wave `wave0`; tid is the thread's index among
// them.  valid = false: the waves only keep step with the workgroup's
// barriers (p is then any existing plane).  T: storage of x, lambda and the
// output; TW: storage of the weights (WPair: packed half pairs of
// channel-shared weights); LOGITS: the weights are logits normalised here
// (else normalised weights, zero outside the line).
template <typename T, typename TW, bool LOGITS, typename TO = T>
__device__ __forceinline__ void lp_line(const ScanK& a, int64_t p, int q, bool valid, int tid, int wave0,
                                        int nwaves) {
    constexpr int P = 16 / static_cast<int>(sizeof(T));              // positions per lane
    constexpr int WT = P * static_cast<int>(sizeof(T)) / 4;          // words per lane: x, lambda, out
    constexpr bool PAIR = std::is_same_v<TW, WPair>;
    constexpr int ZB = PAIR ? 4 : static_cast<int>(sizeof(TW));      // weight bytes per position and row
    constexpr int NZ = PAIR ? 1 : 3;                                  // weight rows
    constexpr int WW = P * ZB / 4;                                    // words per lane: one weight row
    constexpr int D = GSPN_LP_DEPTH;                                  // steps in flight
    __shared__ float edges[2][lp::kMaxWaves][2];

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int S = a.S;
    const int L = a.L;
    const int64_t plane = static_cast<int64_t>(S) * L;
    const int64_t nidx = p / a.c;
    const int64_t ci = p - nidx * a.c;

    const auto rx = lp::rsrc(static_cast<const T*>(a.x) + p * plane, plane * sizeof(T));
    const auto rl = lp::rsrc(static_cast<const T*>(a.lam) + p * plane, plane * sizeof(T));
    const auto ro = lp::rsrc(static_cast<TO*>(a.out) + p * plane, plane * sizeof(TO));
    const auto rz = lp::rsrc(static_cast<const char*>(a.wts) +
                                 (PAIR ? nidx * plane : (nidx * a.cw + (a.cw == 1 ? 0 : ci)) * 3 * plane) * ZB,
                             NZ * plane * ZB);

    const int k0 = tid * P;
    const bool active = valid && k0 < L;
    const int k0c = active ? k0 : L - P;  // lanes past the line read its last vector (unused)
    const uint32_t vt = static_cast<uint32_t>(k0c) * sizeof(T);
    const uint32_t vw = static_cast<uint32_t>(k0c) * ZB;
    const uint32_t rowT = static_cast<uint32_t>(L) * sizeof(T);
    const uint32_t vo = static_cast<uint32_t>(k0c) * sizeof(TO);
    const uint32_t rowO = static_cast<uint32_t>(L) * sizeof(TO);
    const uint32_t rowW = static_cast<uint32_t>(L) * ZB;
    const uint32_t planeW = static_cast<uint32_t>(plane) * ZB;
    const bool has_l0 = k0 > 0;       // the lane's first position has a left neighbour
    const bool has_rP = k0 + P < L;   // the lane's last position has a right neighbour

    const int t0 = q * a.K;
    const int t1 = min(t0 + a.K, S);
    const bool rev = a.reverse != 0;
    auto line_of = [&](int t) { return static_cast<uint32_t>(rev ? S - 1 - t : t); };

    uint32_t sx[D][WT], sl[D][WT], sz[D][NZ][WW];
    auto fill = [&](auto slot, int t) {
        constexpr int s = decltype(slot)::value;
        const uint32_t i = line_of(min(t, t1 - 1));
        lp::load_words<WT, GSPN_LP_X_AUX>(sx[s], rx, vt, i * rowT);
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
    auto step = [&](auto slot, auto firstc, int t) {
        constexpr int s = decltype(slot)::value;
        constexpr bool FIRST = decltype(firstc)::value != 0;
        float hn[P];
        if constexpr (FIRST) {
#pragma unroll
            for (int j = 0; j < P; ++j) hn[j] = lp::elem<T, WT>(sl[s], j) * lp::elem<T, WT>(sx[s], j);
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
                const float base = __builtin_fmaf(lp::elem<T, WT>(sl[s], j), lp::elem<T, WT>(sx[s], j), h[j]);
                hn[j] = __builtin_fmaf(pair_hi(sz[s][0][j]), dd[j + 1], __builtin_fmaf(pair_lo(sz[s][0][j]), -dd[j], base));
            }
        } else {
            float u[P];
#pragma unroll
            for (int j = 0; j < P; ++j) u[j] = lp::elem<T, WT>(sl[s], j) * lp::elem<T, WT>(sx[s], j);
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
template <typename T, typename TW, bool LOGITS, typename TO = T>
__global__ __launch_bounds__(lp::kMaxLanes) void scan4lp_kernel(const Scan4K a) {
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
    const int64_t pg = idx / k.nchunks;
    const int q = static_cast<int>(idx - pg * k.nchunks);
    // a.group consecutive planes share the workgroup, each on its own waves;
    // with channel-shared weights their weight loads coincide in time, so all
    // but the first are served by the cache
    const int per = static_cast<int>(blockDim.x) / a.group;
    // per is a whole number of waves, so g is uniform in the wave: say so, to
    // keep the plane's buffer resources in scalar registers
    const int g = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / per);
    const int64_t p = pg * a.group + g;
    const bool valid = p < a.planes;
    lp_line<T, TW, LOGITS, TO>(k, valid ? p : a.planes - 1, q, valid, static_cast<int>(threadIdx.x) - g * per,
                               g * (per >> 6), per >> 6);
}

template <typename T, typename TW, bool LOGITS, typename TO = T>
hipError_t launch_fused4lp(const Scan4K& k, int nthreads, hipStream_t stream) {
    const int64_t nblocks = k.blocks[0] + k.blocks[1] + k.blocks[2] + k.blocks[3];
    hipLaunchKernelGGL((scan4lp_kernel<T, TW, LOGITS, TO>), dim3(static_cast<unsigned>(nblocks)), dim3(nthreads), 0,
                       stream, k);
    return hipGetLastError();
}

}  // namespace gspn
