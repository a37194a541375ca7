// coltile.hpp -- LDS column tiles of a row-major plane (internal to libgspn),
// for scans whose lines are the plane's columns (the horizontal directions,
// stepping along W): the plane-sequential kernel (seq4.hip) and the
// long-line scan (scan_lp.hpp) read x this way instead of a transposed copy.
//
// The column block [c0, c0 + TS) of every row of an R x C source matrix
// (row-major, element type T; R and C multiples of 64, R <= 1024) lands in
// LDS step-major: tile row tt (column c0 + tt) holds the R values of that
// column, RS dwords apart.  TS = ROW_BYTES / sizeof(T) columns.  fp32:
// RS = R + 4 dwords (16-byte aligned rows); bf16: rows of R/2 dwords each
// holding two consecutive source rows' values (low half the even row),
// RS = R/2 + 2.
// A row's run of ROW_BYTES is CPR chunks of 16 bytes.  Lane tid of LANES
// loads chunk g = q * LANES + tid of round q: 16 bytes of row g / CPR (fp32)
// or of rows 2 (g / CPR) and 2 (g / CPR) + 1 (bf16), from column
// 16/sizeof(T) * (g % CPR) of the block, so CPR consecutive lanes read one
// whole run of a row (whole 128-byte cache lines at ROW_BYTES = 128).
#pragma once

#include "device.hpp"

namespace gspn {
namespace coltile {

typedef int int4v __attribute__((ext_vector_type(4)));

// Dwords of an LDS tile of ROW_BYTES a row for lines of up to 1024 rows
// (both storage types).
template <int ROW_BYTES>
constexpr int tile_dwords() { return (ROW_BYTES / 2) * 514; }

// Index code of Tile::load, shared with the host replay: the byte offset in
// the source of the first 16-byte vector that chunk g loads (fp32: its row's
// run; bf16: the even row's run, the odd row's one row further), or -1 for a
// round past the matrix whose address is clamped into it (its loads repeat
// the last row and are not stored).
GSPN_HD int64_t chunk_offset(int g, int R, int C, int c0, int es, int cpr) {
    const int csh = cpr == 8 ? 3 : 2;
    if (es == 4) {
        const int r = (g >> csh) < R - 1 ? (g >> csh) : R - 1;
        return static_cast<int64_t>(r) * C * 4 + (c0 + 4 * (g & (cpr - 1))) * 4;
    }
    const int r = 2 * (g >> csh) < R - 2 ? 2 * (g >> csh) : R - 2;
    return static_cast<int64_t>(r) * C * 2 + (c0 + 8 * (g & (cpr - 1))) * 2;
}

template <typename T, int LANES, int ROW_BYTES>
struct Tile {
    static constexpr bool F32 = sizeof(T) == 4;
    static constexpr int TS = ROW_BYTES / static_cast<int>(sizeof(T));
    static constexpr int CPR = ROW_BYTES / 16;          // 16-byte chunks per row
    static constexpr int CSH = CPR == 8 ? 3 : 2;        // log2 CPR
    static constexpr int NQ = 1024 * CPR / LANES;       // chunks per lane for R = 1024
    static_assert(CPR == 4 || CPR == 8, "64- or 128-byte runs of a row");
    uint32_t q[NQ][4];

    GSPN_HD static int row_stride(int R) { return F32 ? R + 4 : R / 2 + 2; }

    // Issue the loads of column block c0 (rounds beyond R rows clamp their
    // addresses into the matrix and are not stored); AUX: the loads' cache
    // policy bits.
    template <int AUX>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t src, int R, int C, int c0, int tid) {
        const uint32_t rowb = static_cast<uint32_t>(C) * sizeof(T);
        if constexpr (F32) {
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int g = i * LANES + tid;
                const int r = min(g >> CSH, R - 1);
                const uint32_t off = static_cast<uint32_t>(r) * rowb + (c0 + 4 * (g & (CPR - 1))) * 4u;
                const int4v v = __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, AUX);
#pragma unroll
                for (int e = 0; e < 4; ++e) q[i][e] = static_cast<uint32_t>(v[e]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NQ / 2; ++i) {
                const int g = i * LANES + tid;
                const int r = min(2 * (g >> CSH), R - 2);
                const uint32_t off = static_cast<uint32_t>(r) * rowb + (c0 + 8 * (g & (CPR - 1))) * 2u;
                const int4v v0 = __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, AUX);
                const int4v v1 = __builtin_amdgcn_raw_buffer_load_b128(src, off + rowb, 0, AUX);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    q[2 * i][e] = static_cast<uint32_t>(v0[e]);
                    q[2 * i + 1][e] = static_cast<uint32_t>(v1[e]);
                }
            }
        }
    }

    // Write the loaded block into LDS (the caller makes sure no lane still
    // reads the previous block, and synchronises before the new one is read).
    __device__ __forceinline__ void store(uint32_t* lds, int R, int tid) const {
        const int RS = row_stride(R);
        if constexpr (F32) {
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int g = i * LANES + tid;
                const int r = g >> CSH;
                if (r < R) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) lds[(4 * (g & (CPR - 1)) + e) * RS + r] = q[i][e];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NQ / 2; ++i) {
                const int g = i * LANES + tid;
                const int rp = g >> CSH;
                if (2 * rp < R) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t a = q[2 * i][e >> 1];
                        const uint32_t b = q[2 * i + 1][e >> 1];
                        // low half: the even row's value, high half: the odd row's
                        const uint32_t v = (e & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                                                   : __builtin_amdgcn_perm(b, a, 0x05040100u);
                        lds[(8 * (g & (CPR - 1)) + e) * RS + rp] = v;
                    }
                }
            }
        }
    }
};

}  // namespace coltile
}  // namespace gspn
