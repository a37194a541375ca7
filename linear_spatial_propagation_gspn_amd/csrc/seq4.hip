// seq4.hip -- the four-direction propagation of many big planes, y built in
// place by one workgroup per plane (internal to libgspn).
//
// What it computes: y = sum over T2B, B2T, L2R, R2L of the line scans
//   h_i[k] = sum_{o in {-1,0,+1}, 0 <= k+o < L} w_i[k,o] h_{i-1}[k+o] + lambda_i[k] x_i[k]
// (GSPN-2 paper notes, "2D spatial propagation recap"; h = 0 before the
// first line and before every chunk, "Optimisation 1"), optionally weighted
// per direction and channel (the learnable merge).
//
// When: lines of at most 1024 positions and enough (n, c) planes to give
// every CU its own (the wide-channel workload: 1152 planes of 1024 x 1024).
// One workgroup of four waves, four positions per lane, owns a plane and runs
// the directions one after another; h stays in VGPRs, neighbours move by DPP
// inside a wave and through LDS across waves (one barrier per step):
//   1. L2R: the lines are array columns.  x is read through LDS column tiles:
//      the next 128 bytes of every row, loaded coalesced (eight lanes per
//      row) into registers while the current tile is read, then written into
//      LDS step-major so that a step reads one contiguous line.  h of column
//      i is stored as row i of a transposed scratch map z ([W][H], workspace).
//   2. R2L: the same, adding onto z's rows: z = h_L2R + h_R2L.
//   3. T2B: x rows; z is read back through LDS column tiles (column i of z
//      holds row i of the plane); y row i = h_T2B + (row i of z^T).
//   4. B2T: x rows; y row i += h_B2T.
// A plane's bytes: x four times, every lambda and weight stream once, z
// written, read + written, read (4U), y written, read + written (3U): 15U
// for channel-shared weights.  No map goes through a separate transpose or
// merge pass, and every tile is read-only.  A column tile needs whole
// 128-byte runs of each row to stream at speed (a tile of 64 bytes a row
// reads at about two thirds of the rate): 128 KB of LDS for a 1024-row line,
// so one workgroup per CU.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include <atomic>

#include "device.hpp"
#include "coltile.hpp"
#include "launch.hpp"

namespace gspn {

namespace {

constexpr int kLanes = 256;
constexpr int kWaves = kLanes / 64;
constexpr int kP = 4;                      // positions per lane
// bytes of every source row a column tile holds: a whole 128-byte cache line
// of each row, so every line is fetched once (a 64-byte tile leaves the
// other half of each line to a later tile, which fetches it again: 1U more
// per tile phase on the counters).  128 KB of LDS for a 1024-row line, so one
// workgroup per CU (measured faster than two with 64-byte tiles: 7.6 against
// 8.6 ms on 1152 planes of 1024^2 bf16).
#ifndef GSPN_SEQ4_TILE_ROW_BYTES
#define GSPN_SEQ4_TILE_ROW_BYTES 128
#endif
constexpr int kTileRowBytes = GSPN_SEQ4_TILE_ROW_BYTES;
constexpr int kTileDwords = coltile::tile_dwords<kTileRowBytes>();  // LDS tile: TS rows of RS dwords
// planes per workgroup, each on its own four waves: with channel-shared
// weights the planes' weight loads then coincide in time and all but the
// first are served by the cache
#ifndef GSPN_SEQ4_PLANES_PER_BLOCK
#define GSPN_SEQ4_PLANES_PER_BLOCK 1
#endif
constexpr int kGroups = GSPN_SEQ4_PLANES_PER_BLOCK;
constexpr int kBlocksPerCU = (kTileRowBytes <= 64 ? 2 : 1) / kGroups > 0 ? (kTileRowBytes <= 64 ? 2 : 1) / kGroups : 1;
// cache policy of the z / y row accesses (read back only a phase later)
#ifndef GSPN_SEQ4_RMW_AUX
#define GSPN_SEQ4_RMW_AUX 2
#endif

typedef int int2v __attribute__((ext_vector_type(2)));
typedef int int4v __attribute__((ext_vector_type(4)));

template <int V>
using IC = std::integral_constant<int, V>;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// NW 32-bit words (2 or 4) from the buffer at voff + soff.
template <int NW, int AUX>
__device__ __forceinline__ void ldw(uint32_t (&d)[NW], __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (NW == 4) {
        const int4v q = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = static_cast<uint32_t>(q[e]);
    } else {
        static_assert(NW == 2, "two or four words");
        const int2v q = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
        d[0] = static_cast<uint32_t>(q[0]);
        d[1] = static_cast<uint32_t>(q[1]);
    }
}

template <int NW, int AUX>
__device__ __forceinline__ void stw(const uint32_t (&d)[NW], __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                    uint32_t soff) {
    if constexpr (NW == 4) {
        const int4v q = {static_cast<int>(d[0]), static_cast<int>(d[1]), static_cast<int>(d[2]),
                         static_cast<int>(d[3])};
        __builtin_amdgcn_raw_buffer_store_b128(q, r, voff, soff, AUX);
    } else {
        const int2v q = {static_cast<int>(d[0]), static_cast<int>(d[1])};
        __builtin_amdgcn_raw_buffer_store_b64(q, r, voff, soff, AUX);
    }
}

// Element j of kP values of type E packed in words, widened to fp32.
template <typename E, int NW>
__device__ __forceinline__ float elem(const uint32_t (&w)[NW], int j) {
    if constexpr (sizeof(E) == 4) {
        return __uint_as_float(w[j]);
    } else {
        const uint32_t word = w[j >> 1];
        return __uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16));
    }
}

// kP fp32 values into words of type E (bf16: rounded to nearest even).
template <typename E, int NW>
__device__ __forceinline__ void pack(uint32_t (&w)[NW], const float (&v)[kP]) {
    if constexpr (sizeof(E) == 4) {
#pragma unroll
        for (int j = 0; j < kP; ++j) w[j] = __float_as_uint(v[j]);
    } else {
#pragma unroll
        for (int e = 0; e < NW; ++e) w[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    }
}

__device__ __forceinline__ float from_lower_lane(float v) {  // lane i gets lane i-1 (0 for lane 0)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, true));
}

__device__ __forceinline__ float from_upper_lane(float v) {  // lane i gets lane i+1 (0 for lane 63)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xf, 0xf, true));
}

// Non-temporal hint (buffer instruction bit 1) for streams touched once.
constexpr int kNT = 2;

}  // namespace

struct Seq4K {
    int64_t planes;        // n * c
    const void* x;         // [planes][H][W]
    const void* wts[4];    // direction d: logits [n][cw][3][S][L] (LOGITS) or half pairs [n][S][L]
    const void* lam[4];    // direction d: [planes][S][L], its scan frame
    void* y;               // [planes][H][W]
    void* z;               // workspace [planes][W][H]: the horizontal directions' sum, transposed
    const float* merge;    // [4][c] learnable merge weights, or null
    float* st;             // fp32 state maps (map d: st + d * st_ld, its scan frame), or null
    int64_t st_ld;         // floats between the state maps
    int64_t c;
    int64_t cw;
    int H, W;
    int K[4];              // steps per chunk of each direction, in [1, S]
};

namespace {

// Column tiles of x (and of z): 128-byte runs of every row (coltile.hpp).
template <typename T>
using Tile = coltile::Tile<T, kLanes, kTileRowBytes>;

// One direction's scan over a whole plane.  MODE: 0 L2R (x tiles, z = h),
// 1 R2L (x tiles, z += h), 2 T2B (x rows, y = h + z^T tiles), 3 B2T (x rows,
// y += h).  T: storage type; TW: WPair (channel-shared weights normalised
// beforehand) or T (logits, normalised here); D: steps of per-step inputs in
// flight; LOGITS: TW holds logits (else fp32 weights normalised beforehand);
// STATES: h of every line is also stored, in fp32, as a row of the
// direction's state map (the rows of z and y are already in the maps' frames);
// the scan then runs unweighted and a merge weight scales h where it enters
// z or y (else the weight scales lambda x, the scan being linear in it).
// tid: the thread's index among the plane's kLanes; valid = false: the
// waves only keep step with the workgroup's barriers (p is then any plane).
template <typename T, typename TW, bool LOGITS, int MODE, int D, bool MERGE, bool STATES>
__device__ __forceinline__ void seq_phase(const Seq4K& a, int64_t p, bool valid, int tid, uint32_t* tile,
                                          float (*edges)[kWaves][2], Tile<T>& tl) {
    constexpr bool PAIR = std::is_same_v<TW, WPair>;
    constexpr bool HORIZ = MODE < 2;
    constexpr bool REV = MODE == 1 || MODE == 3;
    constexpr int DIR = MODE == 0 ? 2 : MODE == 1 ? 3 : MODE == 2 ? 0 : 1;
    constexpr int ES = static_cast<int>(sizeof(T));
    constexpr int NW = kP * ES / 4;                  // words of kP values: x, lambda, z / y
    constexpr int NZW = PAIR ? 4 : kP * static_cast<int>(sizeof(TW)) / 4;  // words of one weight row
    constexpr int NZ = PAIR ? 1 : 3;                 // weight rows
    constexpr int TS = Tile<T>::TS;
    constexpr bool TILE = MODE <= 2;                 // a column tile feeds this phase
    constexpr bool EXTRA_ROW = MODE == 1 || MODE == 3;  // a row of z / y is added
    static_assert(64 % D == 0 && TS % D == 0, "ring groups align with tiles and lines");

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H;
    const int W = a.W;
    const int S = HORIZ ? W : H;
    const int L = HORIZ ? H : W;
    const int K = a.K[DIR];
    const int64_t plane = static_cast<int64_t>(H) * W;
    const int64_t nidx = p / a.c;
    const int64_t ci = p - nidx * a.c;
    const float msc = MERGE ? a.merge[DIR * a.c + ci] : 1.0f;

    const auto rl = rsrc(static_cast<const T*>(a.lam[DIR]) + p * plane, plane * ES);
    const int zb = PAIR ? 4 : static_cast<int>(sizeof(TW));  // weight bytes per position and row
    const auto rz = rsrc(static_cast<const char*>(a.wts[DIR]) +
                             (PAIR ? nidx * plane : (nidx * a.cw + (a.cw == 1 ? 0 : ci)) * 3 * plane) * zb,
                         NZ * plane * zb);
    const auto rx = rsrc(static_cast<const T*>(a.x) + p * plane, plane * ES);
    const auto rzt = rsrc(static_cast<T*>(a.z) + p * plane, plane * ES);  // z, [W][H]
    const auto ry = rsrc(static_cast<T*>(a.y) + p * plane, plane * ES);
    // this plane's state map of the direction, [S][L] (one plane's bytes)
    const auto rst = rsrc(STATES ? a.st + DIR * a.st_ld + p * plane : a.st, STATES ? plane * 4 : 0);
    // the tile's source: x ([H][W]) in the horizontal phases, z ([W][H]) in T2B
    const auto rsrc_tile = MODE == 2 ? rzt : rx;
    const int tR = MODE == 2 ? W : H;  // rows of the tile source = the line length
    const int tC = MODE == 2 ? H : W;
    const int RS = Tile<T>::row_stride(tR);

    const int k0 = tid * kP;
    const bool active = valid && k0 < L;
    const int k0c = active ? k0 : L - kP;
    const uint32_t vt = static_cast<uint32_t>(k0c) * ES;
    const uint32_t vw = static_cast<uint32_t>(k0c) * zb;
    const uint32_t rowT = static_cast<uint32_t>(L) * ES;
    const uint32_t rowW = static_cast<uint32_t>(L) * zb;
    const uint32_t planeW = static_cast<uint32_t>(plane) * zb;
    const bool has_l0 = k0 > 0;
    const bool has_rP = k0 + kP < L;
    auto line_of = [&](int t) { return REV ? S - 1 - t : t; };

    // per-step inputs D steps ahead: lambda, weights, x rows (T2B, B2T),
    // the z / y row added (R2L, B2T)
    uint32_t sl[D][NW], sz[D][NZ][NZW];
    uint32_t sx[HORIZ ? 1 : D][NW], se[EXTRA_ROW ? D : 1][NW];
    auto fill = [&](auto slot, int t) {
        constexpr int s = decltype(slot)::value;
        const uint32_t i = static_cast<uint32_t>(line_of(min(t, S - 1)));
        ldw<NW, kNT>(sl[s], rl, vt, i * rowT);
        constexpr int ZAUX = LOGITS ? kNT : 0;  // weights normalised beforehand are re-read by every plane
#pragma unroll
        for (int o = 0; o < NZ; ++o) ldw<NZW, ZAUX>(sz[s][o], rz, vw, o * planeW + i * rowW);
        if constexpr (!HORIZ) ldw<NW, kNT>(sx[s], rx, vt, i * rowT);
        if constexpr (MODE == 1) ldw<NW, GSPN_SEQ4_RMW_AUX>(se[s], rzt, vt, i * rowT);
        if constexpr (MODE == 3) ldw<NW, GSPN_SEQ4_RMW_AUX>(se[s], ry, vt, i * rowT);
    };

    float h[kP];
#pragma unroll
    for (int j = 0; j < kP; ++j) h[j] = 0.0f;
    int buf = 0;

    int tk = 0;  // steps since the chunk began (chunks start at t = 0 in scan order)
    // scan step t from ring slot s; tt: the step's row in the current tile
    auto step = [&](auto slot, int t) {
        constexpr int s = decltype(slot)::value;
        const int i = line_of(t);
        const bool first = tk == 0;  // the chunk's first line: no h_{i-1}, logits unused
        tk = tk + 1 == K ? 0 : tk + 1;
        float xin[kP], extra[kP];
        if constexpr (TILE) {
            const int tt = i % TS;
            uint32_t tw[NW];
            const uint32_t* src = tile + tt * RS + (ES == 4 ? k0c : k0c / 2);
            if constexpr (NW == 4) {
                const int4v q = *reinterpret_cast<const int4v*>(src);
#pragma unroll
                for (int e = 0; e < 4; ++e) tw[e] = static_cast<uint32_t>(q[e]);
            } else {
                const int2v q = *reinterpret_cast<const int2v*>(src);
                tw[0] = static_cast<uint32_t>(q[0]);
                tw[1] = static_cast<uint32_t>(q[1]);
            }
#pragma unroll
            for (int j = 0; j < kP; ++j) {
                if constexpr (MODE == 2) {
                    xin[j] = elem<T, NW>(sx[s], j);
                    extra[j] = elem<T, NW>(tw, j);
                } else {
                    xin[j] = elem<T, NW>(tw, j);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kP; ++j) xin[j] = elem<T, NW>(sx[s], j);
        }
        if constexpr (EXTRA_ROW) {
#pragma unroll
            for (int j = 0; j < kP; ++j) extra[j] = elem<T, NW>(se[s], j);
        }
        float u[kP];
#pragma unroll
        for (int j = 0; j < kP; ++j) {
            const float lx = elem<T, NW>(sl[s], j) * xin[j];
            u[j] = MERGE && !STATES ? lx * msc : lx;
        }
        // neighbours from the previous step: inside the wave by DPP, across
        // wave edges from LDS (0 beyond the line; lanes past it hold h = 0)
        const float eleft = wave > 0 ? edges[buf][wave - 1][1] : 0.0f;
        const float eright = wave + 1 < kWaves ? edges[buf][wave + 1][0] : 0.0f;
        const float dl = from_lower_lane(h[kP - 1]);
        const float dr = from_upper_lane(h[0]);
        const float left = lane == 0 ? eleft : dl;
        const float right = lane == 63 ? eright : dr;
        float hn[kP];
        if (first) {
#pragma unroll
            for (int j = 0; j < kP; ++j) hn[j] = u[j];
        } else if constexpr (PAIR) {
            // h + w_{k-1} (h_{k-1} - h) + w_{k+1} (h_{k+1} - h) + lambda x: the
            // row-stochastic combination with the centre weight eliminated
            float dd[kP + 1];
            dd[0] = h[0] - left;
#pragma unroll
            for (int j = 1; j < kP; ++j) dd[j] = h[j] - h[j - 1];
            dd[kP] = right - h[kP - 1];
#pragma unroll
            for (int j = 0; j < kP; ++j) {
                // with states, lambda x + h fused as the long-line scan fuses
                // it, so that the kept scans of the two kernels agree bit for
                // bit (without, a product and an add measured faster)
                const float base = STATES ? __builtin_fmaf(elem<T, NW>(sl[s], j), xin[j], h[j]) : h[j] + u[j];
                hn[j] = __builtin_fmaf(pair_hi(sz[s][0][j]), dd[j + 1],
                                       __builtin_fmaf(pair_lo(sz[s][0][j]), -dd[j], base));
            }
        } else {
#pragma unroll
            for (int j = 0; j < kP; ++j) {
                float w0 = elem<TW, NZW>(sz[s][0], j), w1 = elem<TW, NZW>(sz[s][1], j),
                      w2 = elem<TW, NZW>(sz[s][2], j);
                if constexpr (LOGITS) normalise_row(w0, w1, w2, j > 0 || has_l0, j < kP - 1 || has_rP, w0, w1, w2);
                const float hl = j == 0 ? left : h[j - 1];
                const float hr = j == kP - 1 ? right : h[j + 1];
                hn[j] = __builtin_fmaf(w0, hl, __builtin_fmaf(w1, h[j], __builtin_fmaf(w2, hr, u[j])));
            }
        }
        fill(slot, t + D);
#pragma unroll
        for (int j = 0; j < kP; ++j) h[j] = active ? hn[j] : 0.0f;
        if (active) {
            float ov[kP];
#pragma unroll
            for (int j = 0; j < kP; ++j) {
                if constexpr (MERGE && STATES) ov[j] = MODE == 0 ? msc * h[j] : __builtin_fmaf(msc, h[j], extra[j]);
                else ov[j] = MODE == 0 ? h[j] : h[j] + extra[j];
            }
            uint32_t ow[NW];
            pack<T, NW>(ow, ov);
            const uint32_t soff = static_cast<uint32_t>(i) * rowT;
            if constexpr (MODE <= 1) stw<NW, GSPN_SEQ4_RMW_AUX>(ow, rzt, vt, soff);      // read back a phase later
            else if constexpr (MODE == 2) stw<NW, GSPN_SEQ4_RMW_AUX>(ow, ry, vt, soff);  // read back by B2T
            else stw<NW, kNT>(ow, ry, vt, soff);
            if constexpr (STATES) {
                // read only by a backward, after this launch
                uint32_t hw[kP];
#pragma unroll
                for (int j = 0; j < kP; ++j) hw[j] = __float_as_uint(h[j]);
                stw<kP, kNT>(hw, rst, static_cast<uint32_t>(k0c) * 4, static_cast<uint32_t>(i) * L * 4);
            }
        }
        buf ^= 1;
        if (lane == 0) edges[buf][wave][0] = h[0];
        if (lane == 63) edges[buf][wave][1] = h[kP - 1];
        __syncthreads();
    };

    // the tile block holding array column (horizontal) / z column (T2B) i
    auto block_of = [&](int t) { return (line_of(t) / TS) * TS; };
    if constexpr (TILE) tl.template load<kNT>(rsrc_tile, tR, tC, block_of(0), tid);
    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        (fill(IC<Ss>{}, Ss), ...);
    }(std::make_integer_sequence<int, D>{});

    // One iteration per tile of TS steps, its steps unrolled, so the loop
    // body has no branch and every wait for a ring slot counts exactly the
    // loads issued after it (a branch around the tile's loads made the
    // compiler drain every load in flight at each group of steps).  The next
    // block's loads are issued at the top, a whole tile ahead; the last
    // iteration reloads its own block instead of branching around them.
    for (int t0 = 0; t0 < S; t0 += TS) {
        if constexpr (TILE) {
            // every lane is past the previous block (the last step's barrier)
            tl.store(tile, tR, tid);
            __syncthreads();
            tl.template load<kNT>(rsrc_tile, tR, tC, block_of(min(t0 + TS, S - 1)), tid);
        }
        [&]<int... Js>(std::integer_sequence<int, Js...>) {
            (step(IC<Js % D>{}, t0 + Js), ...);
        }(std::make_integer_sequence<int, TS>{});
    }
}

// The phases of PH (bit m: phase m) for one plane per group of four waves.
template <typename T, typename TW, bool LOGITS, int D, bool MERGE, bool STATES, int PH>
__global__ __launch_bounds__(kLanes * kGroups, (PH & 7) ? kBlocksPerCU : 4) void seq4_kernel(const Seq4K a) {
    constexpr bool TILES = (PH & 7) != 0;  // a phase reads column tiles
    __shared__ uint32_t tiles[kGroups][TILES ? kTileDwords : 1];
    __shared__ float edge_buf[kGroups][2][kWaves][2];
    // consecutive planes (channels of one image, sharing their weights) on
    // the workgroup's groups of four waves; g is uniform in a wave
    const int g = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kLanes);
    const int tid = static_cast<int>(threadIdx.x) - g * kLanes;
    const int64_t pg = static_cast<int64_t>(blockIdx.x) * kGroups + g;
    const bool valid = pg < a.planes;
    const int64_t p = valid ? pg : a.planes - 1;
    uint32_t* tile = tiles[g];
    float (*edges)[kWaves][2] = edge_buf[g];
    Tile<T> tl;
    // the phases hand z and y from one to the next through memory: each
    // phase's stores are complete and visible to the workgroup before the
    // next phase loads them (phases in separate launches are ordered by the
    // launches)
    auto handoff = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };
    if constexpr ((PH & 1) != 0) seq_phase<T, TW, LOGITS, 0, D, MERGE, STATES>(a, p, valid, tid, tile, edges, tl);
    if constexpr ((PH & 1) != 0 && (PH & 2) != 0) handoff();
    if constexpr ((PH & 2) != 0) seq_phase<T, TW, LOGITS, 1, D, MERGE, STATES>(a, p, valid, tid, tile, edges, tl);
    if constexpr ((PH & 3) != 0 && (PH & 4) != 0) handoff();
    if constexpr ((PH & 4) != 0) seq_phase<T, TW, LOGITS, 2, D, MERGE, STATES>(a, p, valid, tid, tile, edges, tl);
    if constexpr ((PH & 7) != 0 && (PH & 8) != 0) handoff();
    if constexpr ((PH & 8) != 0) seq_phase<T, TW, LOGITS, 3, D, MERGE, STATES>(a, p, valid, tid, tile, edges, tl);
}

// How the four phases are split over launches: one launch of all four, two
// (the horizontal pair, then the vertical pair) or one per phase.
#ifndef GSPN_SEQ4_SPLIT
#define GSPN_SEQ4_SPLIT 0
#endif

template <typename T, typename TW, bool LOGITS, int D, bool MERGE, bool STATES, int PH>
hipError_t launch_phases(const Seq4K& k, int64_t planes, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((planes + kGroups - 1) / kGroups));
    hipLaunchKernelGGL((seq4_kernel<T, TW, LOGITS, D, MERGE, STATES, PH>), grid, dim3(kLanes * kGroups), 0, stream, k);
    return hipGetLastError();
}

template <typename T, typename TW, bool LOGITS, int D, bool MERGE, bool STATES>
hipError_t launch_seq4_m(const Seq4K& k, int64_t planes, hipStream_t stream) {
    hipError_t e = hipSuccess;
    if constexpr (GSPN_SEQ4_SPLIT == 0) {
        e = launch_phases<T, TW, LOGITS, D, MERGE, STATES, 15>(k, planes, stream);
    } else if constexpr (GSPN_SEQ4_SPLIT == 1) {
        e = launch_phases<T, TW, LOGITS, D, MERGE, STATES, 3>(k, planes, stream);
        if (e == hipSuccess) e = launch_phases<T, TW, LOGITS, D, MERGE, STATES, 12>(k, planes, stream);
    } else {
        e = launch_phases<T, TW, LOGITS, D, MERGE, STATES, 1>(k, planes, stream);
        if (e == hipSuccess) e = launch_phases<T, TW, LOGITS, D, MERGE, STATES, 2>(k, planes, stream);
        if (e == hipSuccess) e = launch_phases<T, TW, LOGITS, D, MERGE, STATES, 4>(k, planes, stream);
        if (e == hipSuccess) e = launch_phases<T, TW, LOGITS, D, MERGE, STATES, 8>(k, planes, stream);
    }
    return e;
}

template <typename T, typename TW, bool LOGITS, int D>
hipError_t launch_seq4_t(const Seq4K& k, int64_t planes, hipStream_t stream) {
    if (k.st) {
        if (k.merge) return launch_seq4_m<T, TW, LOGITS, D, true, true>(k, planes, stream);
        return launch_seq4_m<T, TW, LOGITS, D, false, true>(k, planes, stream);
    }
    if (k.merge) return launch_seq4_m<T, TW, LOGITS, D, true, false>(k, planes, stream);
    return launch_seq4_m<T, TW, LOGITS, D, false, false>(k, planes, stream);
}

}  // namespace

int device_compute_units() {
#ifdef GSPN_CHECK_LAUNCHES
    return 256;
#else
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cus[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 0) v = 0;
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
#endif
}

bool seq4_supported(int64_t h, int64_t w) {
    return h >= 64 && w >= 64 && h <= kLanes * kP && w <= kLanes * kP && h % 64 == 0 && w % 64 == 0;
}

hipError_t launch_seq4(const void* x, const void* const wts[4], const void* const lam[4], const float* merge,
                       void* y, void* z, int64_t n, int64_t c, int64_t cw, int64_t h, int64_t w,
                       const int64_t chunk[4], int dtype, int wdtype, int wts_are_logits, int64_t run,
                       float* states, int64_t states_ld, hipStream_t stream) {
    Seq4K k;
    k.planes = n * c;
    k.x = x;
    for (int d = 0; d < 4; ++d) {
        k.wts[d] = wts[d];
        k.lam[d] = lam[d];
        k.K[d] = static_cast<int>(chunk[d]);
    }
    k.y = y;
    k.z = z;
    k.merge = merge;
    k.st = states;
    k.st_ld = states_ld;
    k.c = c;
    k.cw = cw;
    k.H = static_cast<int>(h);
    k.W = static_cast<int>(w);
    const int64_t planes = run < n * c ? run : n * c;
    if (dtype == kF32) {
        if (wts_are_logits) return launch_seq4_t<float, float, true, 4>(k, planes, stream);
        return launch_seq4_t<float, float, false, 4>(k, planes, stream);  // channel-shared, normalised once
    }
    if (wdtype == kPairF16) return launch_seq4_t<bf16_t, WPair, false, 8>(k, planes, stream);
    return launch_seq4_t<bf16_t, bf16_t, true, 4>(k, planes, stream);
}

}  // namespace gspn
