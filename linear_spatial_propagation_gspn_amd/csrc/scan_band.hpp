// scan_band.hpp -- the four-direction line scan for very few, long lines,
// split across workgroups (internal to libgspn; instantiated in scan4_*.hip).
//
// Same recurrence as scan_lp.hpp (GSPN-2 paper notes, "2D spatial
// propagation recap"; chunks from "Optimisation 1"), for launches whose
// lines are so few that one workgroup per line leaves most of the GPU idle:
// the eight proxy-space planes of the compressive proxy ("Optimisation 2")
// make 32 lines of 2048 positions, and a workgroup moves only about 60 GB/s,
// so each step of such a scan costs the time one CU needs to pull the line's
// inputs.  Here a line is cut into segments of `seg` positions, one
// single-wave workgroup per segment, and the scan advances in bands of
// `halo` steps, one launch per band:
//  - a workgroup is one wave of GSPN_BAND_BYTES-byte vectors (8 bf16 or 4
//    fp32 positions per lane at 16 bytes): its segment of half those
//    positions plus `halo`, a quarter, on each side (the line borders clip
//    this), starting from the exact states at the band's first step, which
//    the previous band stored;
//  - the tridiagonal coupling moves information one position per step, so
//    the values that the halo's outer edge gets wrong (its outer neighbours
//    are taken as 0) reach at most `halo` positions inwards by the band's
//    end: the segment itself stays exact, and only it is stored;
//  - at the band's end the segment's states go to a state buffer (fp32) from
//    which the next band's workgroups, including the neighbours' halos,
//    start.  Bands are separate launches, so no workgroup waits for another.
// The halos double the arithmetic and the rows each workgroup reads.  Those
// rows are the neighbouring segments' own rows at the same steps, but the
// counters find most of them fetched again from beyond the L2.
#pragma once

#include "scan_lp.hpp"

namespace gspn {

#ifndef GSPN_BAND_DEPTH
#define GSPN_BAND_DEPTH 12
#endif
// bytes of each row a lane loads per step (its positions: this over the
// element size), and waves a workgroup: a workgroup spans 64 waves bytes
// lanes' worth of positions
#ifndef GSPN_BAND_BYTES
#define GSPN_BAND_BYTES 16
#endif
#ifndef GSPN_BAND_WAVES
#define GSPN_BAND_WAVES 1
#endif

namespace band {

// W 32-bit words from the buffer at voff + soff, in the widest loads W allows.
template <int W, int AUX = 0>
__device__ __forceinline__ void load_words(uint32_t (&d)[W], __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff) {
    if constexpr (W % 4 == 0) {
        lp::load_words<W, AUX>(d, r, voff, soff);
    } else if constexpr (W == 2) {
        typedef int int2v __attribute__((ext_vector_type(2)));
        const int2v q = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
        d[0] = static_cast<uint32_t>(q[0]);
        d[1] = static_cast<uint32_t>(q[1]);
    } else {
        static_assert(W == 1, "1, 2 or a multiple of 4 words");
        d[0] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
    }
}

// W 32-bit words to the buffer at voff + soff.
template <int W, int AUX = 0>
__device__ __forceinline__ void store_words(const uint32_t (&w)[W], __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                            uint32_t soff) {
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int v = 0; v < W / 4; ++v) {
            const lp::int4v o = {static_cast<int>(w[4 * v]), static_cast<int>(w[4 * v + 1]),
                                 static_cast<int>(w[4 * v + 2]), static_cast<int>(w[4 * v + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(o, r, voff + 16 * v, soff, AUX);
        }
    } else if constexpr (W == 2) {
        typedef int int2v __attribute__((ext_vector_type(2)));
        const int2v o = {static_cast<int>(w[0]), static_cast<int>(w[1])};
        __builtin_amdgcn_raw_buffer_store_b64(o, r, voff, soff, AUX);
    } else {
        static_assert(W == 1, "1, 2 or a multiple of 4 words");
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(w[0]), r, voff, soff, AUX);
    }
}

}  // namespace band

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct BandK {
    ScanK d[4];
    int64_t blocks[4];  // workgroups of each direction in this band (0: its scan has ended)
    int nseg[4];        // segments per line of each direction
    const float* hin;   // states at the band's first step: direction d, plane p at hin + d * sstride + p * L_d
    float* hout;        // states at the band's last step, same layout
    int64_t sstride;    // floats per direction in the state buffers
    int t0;             // first scan step of the band
    int seg;            // positions per segment (a multiple of the lane width P)
    int halo;           // steps per band = positions of halo on each side (a multiple of P)
    int64_t planes;     // planes per direction
    int xcd_lines;      // 1: the segments of a line share an XCD (see scan4band_kernel)
};

// CH: chunks restart inside the band (chunk_len below the scan length), so
// every step checks for a chunk's first line; otherwise only step 0 of the
// scan can be one.
// TO: the stored states' type (T, or fp32 for the fp32 states a backward
// pass reads).
template <typename T, typename TW, bool LOGITS, bool CH, typename TO = T>
__device__ __forceinline__ void band_segment(const BandK& b, int dir, int64_t p, int g) {
    const ScanK& a = b.d[dir];
    constexpr int P = GSPN_BAND_BYTES / static_cast<int>(sizeof(T));  // positions per lane
    constexpr int WT = P * static_cast<int>(sizeof(T)) / 4;
    constexpr bool PAIR = std::is_same_v<TW, WPair>;
    constexpr int ZB = PAIR ? 4 : static_cast<int>(sizeof(TW));
    constexpr int NZ = PAIR ? 1 : 3;
    constexpr int WW = P * ZB / 4;
    constexpr int D = GSPN_BAND_DEPTH;

    constexpr int BW = GSPN_BAND_WAVES;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // several waves: the outer neighbours of a wave's edge lanes cross
    // through LDS (double-buffered, one barrier a step)
    __shared__ float edges[2][BW][2];
    int ebuf = 0;
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

    const int s0 = g * b.seg;
    const int s1 = min(s0 + b.seg, L);
    const int k0 = s0 - b.halo + (wave * 64 + lane) * P;   // the lane's first position (may lie outside the line)
    const bool active = k0 >= 0 && k0 < L && k0 < s1 + b.halo;
    const bool owned = k0 >= s0 && k0 < s1;  // positions this workgroup stores
    const int k0c = min(max(k0, 0), L - P);  // addresses of lanes outside the line stay inside it
    const uint32_t vt = static_cast<uint32_t>(k0c) * sizeof(T);
    const uint32_t vw = static_cast<uint32_t>(k0c) * ZB;
    const uint32_t rowT = static_cast<uint32_t>(L) * sizeof(T);
    const uint32_t vo = static_cast<uint32_t>(k0c) * sizeof(TO);
    const uint32_t rowO = static_cast<uint32_t>(L) * sizeof(TO);
    const uint32_t rowW = static_cast<uint32_t>(L) * ZB;
    const uint32_t planeW = static_cast<uint32_t>(plane) * ZB;
    const bool has_l0 = k0 > 0;
    const bool has_rP = k0 + P < L;

    const int t0 = b.t0;
    const int t1 = min(t0 + b.halo, S);
    const int K = a.K;
    int cpos = t0 % K;  // step within the current chunk
    const bool rev = a.reverse != 0;
    auto line_of = [&](int t) { return static_cast<uint32_t>(rev ? S - 1 - t : t); };

    uint32_t sx[D][WT], sl[D][WT], sz[D][NZ][WW];
    // Row offsets advance by one line per step (downwards for a reverse scan;
    // unsigned wrap-around does the subtraction).  Fills run in step order,
    // so the next fill's offsets are kept as running sums (fT, fW) wherever
    // no clamping is needed, and the store's offset (sT) likewise.
    const uint32_t dT = rev ? 0u - rowT : rowT;
    const uint32_t dW = rev ? 0u - rowW : rowW;
    const uint32_t dO = rev ? 0u - rowO : rowO;
    uint32_t fT = 0, fW = 0;
    auto load_slot = [&](auto slot, uint32_t oT, uint32_t oW) {
        constexpr int s = decltype(slot)::value;
        band::load_words<WT, GSPN_LP_X_AUX>(sx[s], rx, vt, oT);
        band::load_words<WT, GSPN_LP_STREAM_AUX>(sl[s], rl, vt, oT);
        constexpr int ZAUX = LOGITS ? GSPN_LP_STREAM_AUX : 0;
#pragma unroll
        for (int o = 0; o < NZ; ++o) band::load_words<WW, ZAUX>(sz[s][o], rz, vw, o * planeW + oW);
    };
    // step t's inputs, the row clamped to the band (rows past it are never used)
    auto fill = [&](auto slot, int t) {
        const uint32_t i = line_of(min(t, t1 - 1));
        load_slot(slot, i * rowT, i * rowW);
    };
    // the next step's inputs where that row lies inside the band
    auto fill_next = [&](auto slot) {
        load_slot(slot, fT, fW);
        fT += dT;
        fW += dW;
    };

    // states at the band's start (a chunk's first step ignores them)
    float h[P];
    const float* hin = b.hin + dir * b.sstride + p * L;
#pragma unroll
    for (int j = 0; j < P; ++j) h[j] = (t0 > 0 && active) ? hin[k0c + j] : 0.0f;
    if constexpr (BW > 1) {
        // lanes outside the line publish exact zeros (see the step's end)
        if (lane == 0) edges[0][wave][0] = active ? h[0] : 0.0f;
        if (lane == 63) edges[0][wave][1] = active ? h[P - 1] : 0.0f;
        __syncthreads();
    }

    uint32_t sO = line_of(t0) * rowO;
    // lambda_j x_j + c for the bf16 pair (j, j + 1) in word e: one bf16 dot
    // product with the other half of x masked to 0.  Its fp32 result can
    // differ from fmaf's by one unit in the last place (measured on gfx950:
    // in 2-18% of random operands), far below the bf16 rounding of the
    // stored h.
    auto lamx = [&](auto slot, int j, float c) {
        constexpr int s = decltype(slot)::value;
        const uint32_t xw = sx[s][j >> 1] & ((j & 1) ? 0xffff0000u : 0x0000ffffu);
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, sl[s][j >> 1]),
                                               __builtin_bit_cast(bf16x2_t, xw), c, false);
    };

    // CLAMP: fill with the row clamped to the band (the last D steps);
    // PEEL: the band's first step, the only one that can start the scan
    // when chunks do not restart (CH false)
    auto step = [&](auto slot, auto clampc, auto peelc, int t) {
        constexpr int s = decltype(slot)::value;
        float hn[P];
        bool first;
        if constexpr (CH) {
            first = cpos == 0;
            cpos = cpos + 1 == K ? 0 : cpos + 1;
        } else {
            first = decltype(peelc)::value != 0 && t == 0;
        }
        if (first) {  // a chunk's first line: h_prev = 0, its weights unused
#pragma unroll
            for (int j = 0; j < P; ++j) {
                if constexpr (PAIR) {
                    hn[j] = lamx(slot, j, 0.0f);
                } else {
                    hn[j] = lp::elem<T, WT>(sl[s], j) * lp::elem<T, WT>(sx[s], j);
                }
            }
        } else {
            float left = lp::shift_from_lower_lane(h[P - 1]);   // 0 beyond the wave
            float right = lp::shift_from_upper_lane(h[0]);
            if constexpr (BW > 1) {
                if (lane == 0) left = wave > 0 ? edges[ebuf][wave - 1][1] : 0.0f;
                if (lane == 63) right = wave + 1 < BW ? edges[ebuf][wave + 1][0] : 0.0f;
            }
            if constexpr (PAIR) {
                // centre weight eliminated, as in the long-line kernel
                float dd[P + 1];
                dd[0] = h[0] - left;
#pragma unroll
                for (int j = 1; j < P; ++j) dd[j] = h[j] - h[j - 1];
                dd[P] = right - h[P - 1];
                // all dot products first: their results are not read back
                // at once (a dot product's result needs extra cycles before
                // the next instruction may read it)
                float base[P];
#pragma unroll
                for (int j = 0; j < P; ++j) base[j] = lamx(slot, j, h[j]);
#pragma unroll
                for (int j = 0; j < P; ++j)
                    hn[j] = __builtin_fmaf(pair_hi(sz[s][0][j]), dd[j + 1],
                                           __builtin_fmaf(pair_lo(sz[s][0][j]), -dd[j], base[j]));
            } else {
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const float z0 = lp::elem<TW, WW>(sz[s][0], j);
                    const float z1 = lp::elem<TW, WW>(sz[s][NZ > 1 ? 1 : 0], j);
                    const float z2 = lp::elem<TW, WW>(sz[s][NZ > 2 ? 2 : 0], j);
                    float w0, w1, w2;
                    if constexpr (LOGITS) {
                        normalise_row(z0, z1, z2, j > 0 || has_l0, j < P - 1 || has_rP, w0, w1, w2);
                    } else {
                        w0 = z0;
                        w1 = z1;
                        w2 = z2;
                    }
                    const float u = lp::elem<T, WT>(sl[s], j) * lp::elem<T, WT>(sx[s], j);
                    const float hl = j == 0 ? left : h[j - 1];
                    const float hr = j == P - 1 ? right : h[j + 1];
                    hn[j] = __builtin_fmaf(w0, hl, __builtin_fmaf(w1, h[j], __builtin_fmaf(w2, hr, u)));
                }
            }
        }
        if constexpr (decltype(clampc)::value != 0) {
            fill(slot, t + D);
        } else {
            fill_next(slot);
        }
        // lanes outside the line: only their edge values leave the lane, and
        // those are held at exact zeros, whose weights at the line's border
        // positions are 0 anyway
#pragma unroll
        for (int j = 0; j < P; ++j) h[j] = (j == 0 || j == P - 1) && !active ? 0.0f : hn[j];
        if constexpr (BW > 1) {
            ebuf ^= 1;
            if (lane == 0) edges[ebuf][wave][0] = h[0];
            if (lane == 63) edges[ebuf][wave][1] = h[P - 1];
            __syncthreads();
        }
        const uint32_t oO = sO;
        sO += dO;
        if (owned) {
            constexpr int WO = P * static_cast<int>(sizeof(TO)) / 4;  // output words per lane
            uint32_t ow[WO];
            if constexpr (sizeof(TO) == 4) {
#pragma unroll
                for (int e = 0; e < WO; ++e) ow[e] = __float_as_uint(h[e]);
            } else {
#pragma unroll
                for (int e = 0; e < WO; ++e) ow[e] = pack_bf16x2(h[2 * e], h[2 * e + 1]);
            }
            band::store_words<WO, GSPN_LP_STREAM_AUX>(ow, ro, vo, oO);
        }
    };

    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        (fill(IC<Ss>{}, t0 + Ss), ...);
    }(std::make_integer_sequence<int, D>{});
    step(IC<0>{}, IC<1>{}, IC<1>{}, t0);
    // then slots 1, 2, .., D-1, 0; while every fill of an iteration (rows
    // t + D .. t + 2D - 1) lies inside the band, from running offsets
    int t = t0 + 1;
    fT = line_of(t0 + D + 1) * rowT;
    fW = line_of(t0 + D + 1) * rowW;
    for (; t + 2 * D <= t1; t += D) {
        [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
            (step(IC<(Ss + 1) % D>{}, IC<0>{}, IC<0>{}, t + Ss), ...);
        }(std::make_integer_sequence<int, D>{});
    }
    for (; t + D <= t1; t += D) {
        [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
            (step(IC<(Ss + 1) % D>{}, IC<1>{}, IC<0>{}, t + Ss), ...);
        }(std::make_integer_sequence<int, D>{});
    }
    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        ((t + Ss < t1 ? step(IC<(Ss + 1) % D>{}, IC<1>{}, IC<0>{}, t + Ss) : void()), ...);
    }(std::make_integer_sequence<int, D - 1>{});

    if (owned) {
        float* ho = b.hout + dir * b.sstride + p * L + k0;
#pragma unroll
        for (int j = 0; j < P; ++j) ho[j] = h[j];
    }
}

// Block b runs on XCD b % 8 (round-robin dispatch).  With xcd_lines, the
// segments of one line all go to the same XCD, so a segment's halo rows,
// which its neighbours read in the same steps, come from that XCD's L2
// (every direction active, equal segment counts, lines a multiple of 8).
template <typename T, typename TW, bool LOGITS, bool CH, typename TO = T>
__global__ __launch_bounds__(64 * GSPN_BAND_WAVES) void scan4band_kernel(const BandK b) {
    int dir = 0;
    int64_t p;
    int g;
    if (b.xcd_lines) {
        const int64_t x = blockIdx.x % 8;
        const int64_t k = blockIdx.x / 8;
        const int nseg = b.nseg[0];
        const int64_t line = x + 8 * (k / nseg);  // dir * planes + plane
        g = static_cast<int>(k % nseg);
        dir = static_cast<int>(line / b.planes);
        p = line - dir * b.planes;
    } else {
        int64_t idx = blockIdx.x;
        while (dir < 3 && idx >= b.blocks[dir]) {
            idx -= b.blocks[dir];
            ++dir;
        }
        p = idx / b.nseg[dir];
        g = static_cast<int>(idx - p * b.nseg[dir]);
    }
    band_segment<T, TW, LOGITS, CH, TO>(b, dir, p, g);
}

// One band: every direction whose scan has not ended by step b.t0.
template <typename T, typename TW, bool LOGITS, typename TO = T>
hipError_t launch_band4(const BandK& b, hipStream_t stream) {
    const int64_t nblocks = b.blocks[0] + b.blocks[1] + b.blocks[2] + b.blocks[3];
    if (nblocks == 0) return hipSuccess;
    bool chunked = false;
    for (int d = 0; d < 4; ++d) chunked = chunked || (b.blocks[d] > 0 && b.d[d].K < b.d[d].S);
    if (chunked) {
        hipLaunchKernelGGL((scan4band_kernel<T, TW, LOGITS, true, TO>), dim3(static_cast<unsigned>(nblocks)),
                           dim3(64 * GSPN_BAND_WAVES), 0, stream, b);
    } else {
        hipLaunchKernelGGL((scan4band_kernel<T, TW, LOGITS, false, TO>), dim3(static_cast<unsigned>(nblocks)),
                           dim3(64 * GSPN_BAND_WAVES), 0, stream, b);
    }
    return hipGetLastError();
}

}  // namespace gspn
