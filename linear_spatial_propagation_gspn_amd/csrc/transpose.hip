// transpose.hip -- plane transposes that let the horizontal directions run as
// row-coalesced scans: x is transposed once into the horizontal scan frame
// (column i of the array becomes row i), the horizontal scans run on that
// copy with the same kernel as the vertical ones, and their outputs are
// folded back into y through a transposing merge.
//
// Both kernels move 64 x 64 tiles through LDS: every global access is a
// 16-byte vector (where the shapes allow) within a run of 64 consecutive
// elements along the row of the tensor it touches, and the transpose happens
// in LDS (rows padded by one element so the column reads hit different banks).
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace gspn {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

struct TileIndex {
    int64_t plane;
    int r0;  // first row of the tile in the source frame
    int c0;  // first column of the tile in the source frame
};

GSPN_HD TileIndex tile_of(int64_t blk, int R, int Cc) {
    const int tr = (R + kTile - 1) / kTile;
    const int tc = (Cc + kTile - 1) / kTile;
    const int64_t per_plane = static_cast<int64_t>(tr) * tc;
    TileIndex t;
    t.plane = blk / per_plane;
    const int64_t r = blk - t.plane * per_plane;
    t.r0 = static_cast<int>(r / tc) * kTile;
    t.c0 = static_cast<int>(r % tc) * kTile;
    return t;
}

// The global accesses of thread tid to one 64 x 64 tile of a (rows x cols)
// plane: row r, column c of the tile is element (r0 + r, c0 + c) of the
// plane.  For each tile row of the thread, 16 bytes along the row:
//   fv(r, c, off)  one 16-byte vector, tile cells (r, c .. c + VW - 1), plane
//                  elements off .. off + VW - 1 (vec: the plane's rows allow
//                  16-byte accesses);
//   fe(r, c, off)  otherwise each element inside the plane on its own;
//   fn(r, c)       and each tile cell outside it.
template <int VW, typename FV, typename FE, typename FN>
GSPN_HD void tile_accesses(int tid, int rows, int cols, int r0, int c0, bool vec, FV&& fv, FE&& fe, FN&& fn) {
    constexpr int LPR = kTile / VW;      // lanes per tile row
    constexpr int RPP = kThreads / LPR;  // rows per pass
    const int lr = tid / LPR;
    const int lc = (tid % LPR) * VW;
#pragma unroll
    for (int i = 0; i < kTile / RPP; ++i) {
        const int r = lr + i * RPP;
        const int gr = r0 + r;
        const int gc = c0 + lc;
        const int64_t off = static_cast<int64_t>(gr) * cols + gc;
        if (vec && gr < rows && gc + VW <= cols) {
            fv(r, lc, off);
        } else {
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                if (gr < rows && gc + e < cols) fe(r, lc + e, off + e);
                else fn(r, lc + e);
            }
        }
    }
}

template <typename T>
struct alignas(16) Vec16 {
    T e[16 / sizeof(T)];
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte vector load / store, with the non-temporal hint when NT (data the
// kernel touches once and nothing reads back soon).
template <bool NT, typename V>
__device__ __forceinline__ V vld(const V* p) {
    if constexpr (NT) {
        return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
    } else {
        return *p;
    }
}

template <bool NT, typename V>
__device__ __forceinline__ void vst(V* p, const V& v) {
    if constexpr (NT) {
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
    } else {
        *p = v;
    }
}

#ifndef GSPN_COMBINE_NT
#define GSPN_COMBINE_NT 1
#endif
#ifndef GSPN_TRANSPOSE_NT
#define GSPN_TRANSPOSE_NT 3  // bit 0: reads, bit 1: writes with the non-temporal hint
#endif

// Moves one 64 x 64 tile of a (rows x cols) plane between global memory and
// an fp32 LDS tile, 16 bytes per lane per access along the rows: row r, column
// c of the tile is element (r0 + r, c0 + c) of the plane.  vec: the plane's
// rows allow 16-byte accesses (cols and the base are whole vectors);
// otherwise single elements.  Elements outside the plane read as 0 / are not
// written.
template <typename T>
struct TileIO {
    static constexpr int VW = 16 / static_cast<int>(sizeof(T));  // elements per vector

    template <bool NT = false, typename F>
    static __device__ __forceinline__ void read(const T* plane, int rows, int cols, int r0, int c0, bool vec,
                                                F&& put) {
        tile_accesses<VW>(
            threadIdx.x, rows, cols, r0, c0, vec,
            [&](int r, int c, int64_t off) {
                const Vec16<T> v = vld<NT>(reinterpret_cast<const Vec16<T>*>(plane + off));
#pragma unroll
                for (int e = 0; e < VW; ++e) put(r, c + e, Store<T>::ld(&v.e[e]));
            },
            [&](int r, int c, int64_t off) { put(r, c, Store<T>::ld(plane + off)); },
            [&](int r, int c) { put(r, c, 0.0f); });
    }

    template <bool NT = false, typename F>
    static __device__ __forceinline__ void write(T* plane, int rows, int cols, int r0, int c0, bool vec, F&& get) {
        tile_accesses<VW>(
            threadIdx.x, rows, cols, r0, c0, vec,
            [&](int r, int c, int64_t off) {
                Vec16<T> v;
#pragma unroll
                for (int e = 0; e < VW; ++e) Store<T>::st(&v.e[e], get(r, c + e, plane + off + e));
                vst<NT>(reinterpret_cast<Vec16<T>*>(plane + off), v);
            },
            [&](int r, int c, int64_t off) { Store<T>::st(plane + off, get(r, c, plane + off)); },
            [&](int, int) {});
    }
};

// dst[p][c][r] = src[p][r][c] for planes of R x Cc.
template <typename T>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                             int R, int Cc, int vec_src, int vec_dst) {
    __shared__ float tile[kTile][kTile + 1];
    const TileIndex ti = tile_of(blockIdx.x, R, Cc);
    const int64_t plane = static_cast<int64_t>(R) * Cc;
    TileIO<T>::template read<(GSPN_TRANSPOSE_NT & 1) != 0>(src + ti.plane * plane, R, Cc, ti.r0, ti.c0, vec_src,
                    [&](int r, int c, float v) { tile[r][c] = v; });
    __syncthreads();
    // destination plane is Cc x R: its row c holds source column c
    TileIO<T>::template write<(GSPN_TRANSPOSE_NT & 2) != 0>(dst + ti.plane * plane, Cc, R, ti.c0, ti.r0, vec_dst,
                     [&](int c, int r, const T*) { return tile[r][c]; });
}

// Offset of the merge weight of direction row k and channel ch in a [4][..]
// array whose rows lie mld floats apart (mld = the channel count, or more for
// a channel range of a wider tensor).
GSPN_HD int64_t merge_index(int k, int64_t ch, int64_t mld) { return k * mld + ch; }

// For planes of R x Cc in the array frame:
//   y[p][r][c] = ((m2 z2[p][c][r] + m3 z3[p][c][r]) + m0 b[p][r][c]) + m1 a[p][r][c]
// where b is y itself (accumulate), a separate source y0, or absent; a, z2,
// z3 may each be absent (NULL) and z2, z3 are in the transposed frame
// (Cc x R planes); m0..m3 are the learnable merge weights merge[k][ch] of
// the plane's channel ch = p % nch (row k at merge + k * mld), or 1 without
// merge weights.  The sources
// other than y are of type TS (the storage type, or fp32 states).  Every
// source is read into the LDS tile with row-vector accesses of its own
// frame; y is read completely before it is written, so it may be updated in
// place.
template <typename T, typename TS>
__global__ __launch_bounds__(kThreads) void combine_kernel(T* y, const TS* __restrict__ y0, const TS* __restrict__ a,
                                                           const TS* __restrict__ z2, const TS* __restrict__ z3,
                                                           int R, int Cc, int accumulate, int vec_y, int vec_s,
                                                           int vec_z, const float* __restrict__ merge, int64_t nch,
                                                           int64_t mld) {
    __shared__ float tile[kTile][kTile + 1];
    const TileIndex ti = tile_of(blockIdx.x, R, Cc);
    const int64_t plane = static_cast<int64_t>(R) * Cc;
    float m[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if (merge) {
        const int64_t ch = ti.plane % nch;
#pragma unroll
        for (int k = 0; k < 4; ++k) m[k] = merge[merge_index(k, ch, mld)];
    }
    bool any = false;
    auto add_t = [&](const TS* z, float wt) {  // transposed source: its row c is column c of the tile
        if (any) __syncthreads();
        const bool first = !any;
        TileIO<TS>::template read<GSPN_COMBINE_NT != 0>(z + ti.plane * plane, Cc, R, ti.c0, ti.r0, vec_z,
                        [&](int c, int r, float v) { tile[r][c] = first ? wt * v : tile[r][c] + wt * v; });
        any = true;
    };
    auto add_a = [&](const auto* src, int vec, float wt) {  // array-frame source (y itself or a TS source)
        using E = std::remove_cv_t<std::remove_pointer_t<decltype(src)>>;
        if (any) __syncthreads();
        const bool first = !any;
        TileIO<E>::template read<GSPN_COMBINE_NT != 0>(src + ti.plane * plane, R, Cc, ti.r0, ti.c0, vec,
                        [&](int r, int c, float v) { tile[r][c] = first ? wt * v : tile[r][c] + wt * v; });
        any = true;
    };
    if (z2) add_t(z2, m[2]);
    if (z3) add_t(z3, m[3]);
    if (y0) add_a(y0, vec_s, m[0]);
    else if (accumulate) add_a(static_cast<const T*>(y), vec_y, m[0]);
    if (a) add_a(a, vec_s, m[1]);
    __syncthreads();
    TileIO<T>::template write<GSPN_COMBINE_NT != 0>(y + ti.plane * plane, R, Cc, ti.r0, ti.c0, vec_y,
                                                    [&](int r, int c, const T*) { return any ? tile[r][c] : 0.0f; });
}

#ifdef GSPN_CHECK_LAUNCHES
// Host replay of one tile pass of every block over the planes at `base`
// (R x Cc planes, or Cc x R when frame_t), as the kernels below call TileIO:
// each access must lie in base's buffer, vectors on 16 bytes, and the LDS
// cell inside the 64 x 64 tile.
template <typename T>
void replay_tiles(const char* kernel, const char* what, const void* base, int64_t nblocks, int R, int Cc,
                  bool frame_t, bool vec) {
    if (!base) return;
    const check::Region reg = check::region_of(base, kernel, what);
    constexpr int VW = TileIO<T>::VW;
    const int64_t plane = static_cast<int64_t>(R) * Cc;
    const int rows = frame_t ? Cc : R;
    const int cols = frame_t ? R : Cc;
    int64_t bad = 0, n = 0;
    auto cell = [&](int r, int c) {
        if (r < 0 || r >= kTile || c < 0 || c >= kTile) ++bad;
    };
    auto acc = [&](const T* pl, int64_t off, int64_t nb, bool vector) {
        ++n;
        const uint64_t a = reinterpret_cast<uint64_t>(pl + off);
        if (!check::in_region(reg, pl, off * static_cast<int64_t>(sizeof(T)), nb) || (vector && a % 16 != 0)) {
            if (bad++ == 0)
                check::violation(kernel, what, "access of %lld bytes at %p outside [%p, %p) or misaligned",
                                 static_cast<long long>(nb), reinterpret_cast<void*>(a),
                                 reinterpret_cast<void*>(reg.lo), reinterpret_cast<void*>(reg.hi));
        }
    };
    for (int64_t b = 0; b < nblocks; ++b) {
        const TileIndex ti = tile_of(b, R, Cc);
        const T* pl = static_cast<const T*>(base) + ti.plane * plane;
        for (int tid = 0; tid < kThreads; ++tid) {
            tile_accesses<VW>(
                tid, rows, cols, frame_t ? ti.c0 : ti.r0, frame_t ? ti.r0 : ti.c0, vec,
                [&](int r, int c, int64_t off) {
                    cell(r, c);
                    cell(r, c + VW - 1);
                    acc(pl, off, 16, true);
                },
                [&](int r, int c, int64_t off) {
                    cell(r, c);
                    acc(pl, off, sizeof(T), false);
                },
                [&](int r, int c) { cell(r, c); });
        }
    }
    if (bad) check::violation(kernel, what, "%lld bad accesses", static_cast<long long>(bad));
    check::count_accesses(n);
}

// The merge weights a combine block reads: those of channel plane % nch in
// each of the four rows, k < 4.
void replay_merge(const char* kernel, const float* merge, int64_t nch, int64_t mld, int64_t nblocks, int R,
                  int Cc) {
    if (!merge) return;
    const check::Region reg = check::region_of(merge, kernel, "merge");
    for (int64_t b = 0; b < nblocks; ++b) {
        const int64_t ch = tile_of(b, R, Cc).plane % nch;
        for (int k = 0; k < 4; ++k)
            if (!check::in_region(reg, merge, merge_index(k, ch, mld) * 4, 4)) {
                check::violation(kernel, "merge", "weight (%d, %lld) outside the buffer", k,
                                 static_cast<long long>(ch));
                return;
            }
    }
}

template <typename T, typename TS>
void replay_combine(int64_t nblocks, const T* y, const TS* y0, const TS* a, const TS* z2, const TS* z3, int R,
                    int Cc, int accumulate, int vec_y, int vec_s, int vec_z, const float* merge, int64_t nch,
                    int64_t mld) {
    const char* k = "combine_kernel";
    replay_merge(k, merge, nch, mld, nblocks, R, Cc);
    replay_tiles<TS>(k, "z2", z2, nblocks, R, Cc, true, vec_z);
    replay_tiles<TS>(k, "z3", z3, nblocks, R, Cc, true, vec_z);
    if (y0) replay_tiles<TS>(k, "y0", y0, nblocks, R, Cc, false, vec_s);
    else if (accumulate) replay_tiles<T>(k, "y (read)", y, nblocks, R, Cc, false, vec_y);
    replay_tiles<TS>(k, "a", a, nblocks, R, Cc, false, vec_s);
    replay_tiles<T>(k, "y", y, nblocks, R, Cc, false, vec_y);
    check::replayed(k, kThreads, sizeof(float) * kTile * (kTile + 1));
}
#endif

int64_t tiles_for(int64_t planes, int R, int Cc) {
    return planes * ((R + kTile - 1) / kTile) * ((Cc + kTile - 1) / kTile);
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

hipError_t launch_transpose(const void* src, void* dst, int64_t planes, int R, int Cc, int dtype,
                            hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(tiles_for(planes, R, Cc)));
    const int vw = dtype == kF32 ? 4 : 8;
    const int vs = (Cc % vw == 0) && aligned16(src);
    const int vd = (R % vw == 0) && aligned16(dst);
#ifdef GSPN_CHECK_LAUNCHES
    if (dtype == kF32) {
        replay_tiles<float>("transpose_kernel", "src", src, grid.x, R, Cc, false, vs);
        replay_tiles<float>("transpose_kernel", "dst", dst, grid.x, R, Cc, true, vd);
    } else {
        replay_tiles<bf16_t>("transpose_kernel", "src", src, grid.x, R, Cc, false, vs);
        replay_tiles<bf16_t>("transpose_kernel", "dst", dst, grid.x, R, Cc, true, vd);
    }
    check::replayed("transpose_kernel", kThreads, sizeof(float) * kTile * (kTile + 1));
#endif
    if (dtype == kF32) {
        hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(kThreads), 0, stream,
                           static_cast<const float*>(src), static_cast<float*>(dst), R, Cc, vs, vd);
    } else {
        hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(kThreads), 0, stream,
                           static_cast<const bf16_t*>(src), static_cast<bf16_t*>(dst), R, Cc, vs, vd);
    }
    return hipGetLastError();
}

hipError_t launch_combine(void* y, const void* a, const void* z2, const void* z3, int64_t planes, int R,
                          int Cc, int accumulate, int dtype, hipStream_t stream, const float* merge, int64_t nch,
                          int64_t mld) {
    if (mld <= 0) mld = nch;
    const dim3 grid(static_cast<unsigned>(tiles_for(planes, R, Cc)));
    const int vw = dtype == kF32 ? 4 : 8;
    const int vy = (Cc % vw == 0) && aligned16(y);
    const int vs = vy && (!a || aligned16(a));
    const int vz = (R % vw == 0) && (!z2 || aligned16(z2)) && (!z3 || aligned16(z3));
#ifdef GSPN_CHECK_LAUNCHES
    if (dtype == kF32) {
        replay_combine<float, float>(grid.x, static_cast<const float*>(y), nullptr, static_cast<const float*>(a),
                                     static_cast<const float*>(z2), static_cast<const float*>(z3), R, Cc, accumulate,
                                     vs, vs, vz, merge, nch, mld);
    } else {
        replay_combine<bf16_t, bf16_t>(grid.x, static_cast<const bf16_t*>(y), nullptr, static_cast<const bf16_t*>(a),
                                       static_cast<const bf16_t*>(z2), static_cast<const bf16_t*>(z3), R, Cc,
                                       accumulate, vs, vs, vz, merge, nch, mld);
    }
#endif
    if (dtype == kF32) {
        hipLaunchKernelGGL((combine_kernel<float, float>), grid, dim3(kThreads), 0, stream, static_cast<float*>(y),
                           static_cast<const float*>(nullptr), static_cast<const float*>(a),
                           static_cast<const float*>(z2), static_cast<const float*>(z3), R, Cc, accumulate, vs, vs,
                           vz, merge, nch, mld);
    } else {
        hipLaunchKernelGGL((combine_kernel<bf16_t, bf16_t>), grid, dim3(kThreads), 0, stream,
                           static_cast<bf16_t*>(y), static_cast<const bf16_t*>(nullptr),
                           static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(z2),
                           static_cast<const bf16_t*>(z3), R, Cc, accumulate, vs, vs, vz, merge, nch, mld);
    }
    return hipGetLastError();
}

hipError_t launch_combine_states(void* y, const float* s0, const float* s1, const float* s2, const float* s3,
                                 int64_t planes, int R, int Cc, int dtype, hipStream_t stream, const float* merge,
                                 int64_t nch, int64_t mld) {
    if (mld <= 0) mld = nch;
    const dim3 grid(static_cast<unsigned>(tiles_for(planes, R, Cc)));
    const int vy = (Cc % (dtype == kF32 ? 4 : 8) == 0) && aligned16(y);
    const int vs = (Cc % 4 == 0) && aligned16(s0) && aligned16(s1);
    const int vz = (R % 4 == 0) && aligned16(s2) && aligned16(s3);
#ifdef GSPN_CHECK_LAUNCHES
    if (dtype == kF32) {
        replay_combine<float, float>(grid.x, static_cast<const float*>(y), s0, s1, s2, s3, R, Cc, 0, vy, vs, vz,
                                     merge, nch, mld);
    } else {
        replay_combine<bf16_t, float>(grid.x, static_cast<const bf16_t*>(y), s0, s1, s2, s3, R, Cc, 0, vy, vs, vz,
                                      merge, nch, mld);
    }
#endif
    if (dtype == kF32) {
        hipLaunchKernelGGL((combine_kernel<float, float>), grid, dim3(kThreads), 0, stream, static_cast<float*>(y),
                           s0, s1, s2, s3, R, Cc, 0, vy, vs, vz, merge, nch, mld);
    } else {
        hipLaunchKernelGGL((combine_kernel<bf16_t, float>), grid, dim3(kThreads), 0, stream,
                           static_cast<bf16_t*>(y), s0, s1, s2, s3, R, Cc, 0, vy, vs, vz, merge, nch, mld);
    }
    return hipGetLastError();
}

}  // namespace gspn
