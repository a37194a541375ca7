// wgrad.hip -- weight gradients of the 1x1 projections of the compressive
// proxy (GSPN-2 notes, "Optimisation 2"): for out = W . in, dL/dW[o][c] is
// the sum over images and pixels of dL/dout[o] * in[c].  Both gradients the
// proxy backward needs have this form with one narrow factor (C_proxy <= 16
// channels) and one wide one (C channels):
//   dL/dw_up[c][k]   = sum gy[c] * y_p[k]      (wide gy, narrow y_p)
//   dL/dw_down[k][c] = sum dx_p[k] * x[c]      (wide x, narrow dx_p)
// computed as G[c][k] = sum big[c] * small[k] and stored transposed where
// needed.  The pass over gy also yields dL/dy_p = w_up^T gy, a narrow-output
// projection of the same tiles, folded into the same kernel.
#include "device.hpp"
#include "launch.hpp"

namespace gspn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// The wide tensor's tiles are read once per pass: non-temporal loads.
__device__ __forceinline__ uint4 ld_once(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ __bf16 as_bf(uint32_t bits16) {
    return __builtin_bit_cast(__bf16, static_cast<uint16_t>(bits16));
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int k) {
    return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
}

// ---------------------------------------------------------------------------
// Weight gradients of the projections: G[c][k] = sum over images and pixels
// of big[n][c][p] * small[n][k][p] (big: c channels, small: k <= 16
// channels).  Each wave (or workgroup, on the VALU path) sums one slot, a
// run of pixels, into part[slot][c][k]; wgrad_reduce_kernel then adds the
// slots in a fixed order, so the result does not depend on scheduling.

// bf16 on the matrix cores, one wave per slot of tiles of 128 pixels.  The
// big tensor is read as the narrow-output projection reads it (lane (q, g)
// holds 8 pixels 8q.. of channels 8g..8g+7 of each 32-channel block) and,
// with PROJ, projected the same way (out[k][p] = sum_c wt[k][c] big[c][p]).
// The weight-gradient product needs pixels along K instead, so each block
// goes through the wave's own LDS tile (32 rows of 128 pixels, one 16-byte
// pad per row so the transposed reads hit 16 distinct bank quads):
// v_mfma_f32_16x16x32_bf16 with M = 16 channels, N = 16 columns of small
// (k < 16, the rest zero), K = 32 pixels; lane l reads channel l % 16 and
// pixels 8 (l / 16) .. + 7 of each 32-pixel step, and the small tensor's
// row l % 16 at the same pixels.  The accumulators (two 16 x 16 tiles per
// block) stay in registers across the slot's tiles.
// Element offsets of wgrad_mfma's accesses (shared with the host replay):
// tile t of 128 pixels, lane (q, g), 32-channel block starting at k0.
struct WgTile {
    int64_t ni, px0;
};
GSPN_HD WgTile wg_tile(int64_t t, int64_t hw) {
    const int64_t per_img = hw / 128;
    const int64_t ni = t / per_img;
    return WgTile{ni, (t - ni * per_img) * 128};
}
// first of the 8 channels lane group g loads in the block at k0 (clamped
// into the tensor; the values of clamped channels are replaced by zeros)
GSPN_HD int wg_channel(int k0, int g, int cin) { return k0 + 8 * g < cin ? k0 + 8 * g : cin - 8; }
GSPN_HD int64_t wg_big(const WgTile& t, int64_t hw, int cin, int q, int ch) {
    return t.ni * cin * hw + t.px0 + 8 * q + static_cast<int64_t>(ch) * hw;
}
GSPN_HD int64_t wg_small(const WgTile& t, int64_t hw, int kk, int q, int g, int s) {
    return (t.ni * kk + (q < kk ? q : kk - 1)) * hw + t.px0 + 8 * g + 32 * s;
}
GSPN_HD int64_t wg_out(const WgTile& t, int64_t hw, int kk, int q, int o) {
    return t.ni * kk * hw + t.px0 + 8 * q + static_cast<int64_t>(o) * hw;
}
GSPN_HD int64_t wg_part(int64_t slot, int cin, int kk, int q, int c) {
    return slot * cin * kk + static_cast<int64_t>(c) * kk + q;
}

template <int NS, bool PROJ>
__global__ __launch_bounds__(256) GSPN_WAVES_PER_EU(2) void wgrad_mfma(const bf16_t* __restrict__ big, const bf16_t* __restrict__ small,
                                                  const bf16_t* __restrict__ wt, bf16_t* __restrict__ pout,
                                                  float* __restrict__ part, int64_t tiles, int64_t per_slot,
                                                  int64_t hw, int cin, int kk) {
    constexpr int PX = 8;
    constexpr int WPX = 16 * PX;   // pixels per tile
    constexpr int ROW = WPX / 8 + 1;  // uint4 per LDS row, with the pad
    __shared__ uint4 tile_lds[kThreads / 64][32 * ROW];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t slot = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wv;
    const int64_t t0 = slot * per_slot;
    if (t0 >= tiles) return;
    const int64_t t1 = t0 + per_slot < tiles ? t0 + per_slot : tiles;
    const int q = lane & 15;
    const int g = lane >> 4;
    const bool qok = q < kk;
    uint4* lt = tile_lds[wv];
    // channel group blockIdx.y: channels c0 .. c0 + cl - 1 (one group with PROJ)
    const int c0 = PROJ ? 0 : static_cast<int>(blockIdx.y) * 32 * NS;
    const int cl = PROJ ? cin : (cin - c0 < 32 * NS ? cin - c0 : 32 * NS);

    struct Block {
        uint4 a;   // PROJ: 8 weights (bf16) of output row q
        uint4 v[8];
        bool ok;
    };
    floatx4 gacc[2 * NS];
#pragma unroll
    for (int j = 0; j < 2 * NS; ++j) gacc[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t t = t0; t < t1; ++t) {
        const WgTile tl = wg_tile(t, hw);
        // the small tensor's row q at pixels 32 s + 8 g, s = 0..3 (lanes
        // q >= kk read row kk - 1: their result columns are not stored)
        bf16x8 bs[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            bs[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(small + wg_small(tl, hw, kk, q, g, s)));
        const bf16_t* wrow = PROJ ? wt + static_cast<int64_t>(qok ? q : kk - 1) * cin : nullptr;
        const bf16_t* src = big + wg_big(tl, hw, cin, q, c0);  // channel c0 + ch at src + ch * hw
        // the lane's channel group made opaque per tile: otherwise the 8 NS
        // channel offsets, the same for every tile, are hoisted out of the
        // tile loop and held in 16 NS registers
        int gt = g;
        asm volatile("" : "+v"(gt));
        auto fetch = [&](int k0, Block& b) {
            b.ok = k0 + 8 * gt < cl;
            const int cc = wg_channel(k0, gt, cl);
            if constexpr (PROJ) b.a = *reinterpret_cast<const uint4*>(wrow + cc);
#pragma unroll
            for (int e = 0; e < 8; ++e) b.v[e] = ld_once(reinterpret_cast<const uint4*>(src + static_cast<int64_t>(cc + e) * hw));
        };
        floatx4 acc[PX];
#pragma unroll
        for (int j = 0; j < PX; ++j) acc[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        auto consume = [&](const Block& b, int i) {
            if constexpr (PROJ) {
                const bool use = b.ok && qok;
                const uint32_t aw[4] = {use ? b.a.x : 0u, use ? b.a.y : 0u, use ? b.a.z : 0u, use ? b.a.w : 0u};
                bf16x8 a;
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = as_bf((e & 1) ? (aw[e >> 1] >> 16) : (aw[e >> 1] & 0xffffu));
#pragma unroll
                for (int j = 0; j < PX; ++j) {
                    bf16x8 bv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t word = b.ok ? word_of(b.v[e], j >> 1) : 0u;
                        bv[e] = as_bf((j & 1) ? (word >> 16) : (word & 0xffffu));
                    }
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[j], 0, 0, 0);
                }
            }
            // rows 8g + e of the block, pixels 8q .. 8q + 7 (channels past
            // c_in hold clamped copies: their result rows are not stored).
            // Lanes exchange data through the wave's own rows: the fences
            // keep the compiler from moving these accesses across each
            // other, and the LDS runs one wave's accesses in order.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int e = 0; e < 8; ++e) lt[(8 * g + e) * ROW + q] = b.v[e];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 a = __builtin_bit_cast(bf16x8, lt[(16 * m + q) * ROW + 4 * s + g]);
                    gacc[2 * i + m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bs[s], gacc[2 * i + m], 0, 0, 0);
                }
            }
        };
        Block b[2];
        fetch(0, b[0]);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i + 1 < NS) fetch(32 * (i + 1), b[(i + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            consume(b[i & 1], i);
        }
        if constexpr (PROJ) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = g * 4 + i;
                if (o < kk) {
                    uint32_t w[PX / 2];
#pragma unroll
                    for (int k = 0; k < PX / 2; ++k) w[k] = pack_bf16x2(acc[2 * k][i], acc[2 * k + 1][i]);
                    *reinterpret_cast<uint4*>(pout + wg_out(tl, hw, kk, q, o)) = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
    }
    // lane holds rows 4g + r (channels 32 i + 16 m + 4g + r) of column q
    if (qok) {
#pragma unroll
        for (int j = 0; j < 2 * NS; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 32 * (j >> 1) + 16 * (j & 1) + 4 * g + r;
                if (c < cl) part[wg_part(slot, cin, kk, q, c0 + c)] = gacc[j][r];
            }
        }
    }
}

// Any storage type and shape: one workgroup per (channel, slot), each lane
// striding over the slot's pixels for 8 columns of small at a time, then a
// fixed-order tree sum over the workgroup.
template <typename T>
__global__ __launch_bounds__(256) void wgrad_partial_kernel(const T* __restrict__ big, const T* __restrict__ small,
                                                            float* __restrict__ part, int64_t hw, int64_t cin,
                                                            int64_t kk, int64_t total, int64_t per_slot,
                                                            int64_t slots) {
    __shared__ float red[8][256];
    const int tid = threadIdx.x;
    const int64_t slot = blockIdx.x % slots;
    const int64_t ci = blockIdx.x / slots;
    const int64_t e0 = slot * per_slot;
    const int64_t e1 = e0 + per_slot < total ? e0 + per_slot : total;
    for (int64_t k0 = 0; k0 < kk; k0 += 8) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        for (int64_t e = e0 + tid; e < e1; e += 256) {
            const int64_t ni = e / hw;
            const int64_t p = e - ni * hw;
            const float a = Store<T>::ld(big + (ni * cin + ci) * hw + p);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (k0 + j < kk) acc[j] = __builtin_fmaf(a, Store<T>::ld(small + (ni * kk + k0 + j) * hw + p), acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) red[j][tid] = acc[j];
        __syncthreads();
        for (int s = 128; s > 0; s >>= 1) {
            if (tid < s) {
#pragma unroll
                for (int j = 0; j < 8; ++j) red[j][tid] += red[j][tid + s];
            }
            __syncthreads();
        }
        if (tid < 8 && k0 + tid < kk) part[(slot * cin + ci) * kk + k0 + tid] = red[tid][0];
        __syncthreads();
    }
}

// out[c * sc + k * sk] = sum over slots of part[slot][c][k], slots added in
// order of their residue mod 16, then the 16 residues in order.
__global__ __launch_bounds__(1024) void wgrad_reduce_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                            int64_t slots, int64_t count, int64_t kk, int64_t sc,
                                                            int64_t sk) {
    __shared__ float red[16][64];
    const int col = threadIdx.x & 63;
    const int r = threadIdx.x >> 6;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 64 + col;
    float acc = 0.0f;
    if (e < count) {
        for (int64_t s = r; s < slots; s += 16) acc += part[s * count + e];
    }
    red[r][col] = acc;
    __syncthreads();
    if (r == 0 && e < count) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) t += red[i][col];
        out[(e / kk) * sc + (e % kk) * sk] = t;
    }
}

bool aligned_to(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

#ifdef GSPN_CHECK_LAUNCHES
// Host replays of the weight-gradient kernels: every access each lane makes,
// at the offsets the kernels compute, checked against its buffer.
void replay_wgrad_mfma(const void* big, const void* small, const void* wt, const void* pout, const float* part,
                       int64_t tiles, int64_t per_slot, int64_t slots, int64_t hw, int cin, int kk, int ns,
                       int groups) {
    const char* kn = "wgrad_mfma";
    const check::Region rb = check::region_of(big, kn, "big");
    const check::Region rs = check::region_of(small, kn, "small");
    const check::Region rp = check::region_of(part, kn, "partials");
    check::Region rw, ro;
    if (wt) {
        rw = check::region_of(wt, kn, "weights");
        ro = check::region_of(pout, kn, "projection");
    }
    int64_t bad = 0, n = 0;
    for (int grp = 0; grp < groups; ++grp) {
        const int c0 = grp * 32 * ns;
        const int cl = cin - c0 < 32 * ns ? cin - c0 : 32 * ns;
        for (int64_t slot = 0; slot < slots; ++slot) {
            const int64_t t0 = slot * per_slot;
            const int64_t t1 = t0 + per_slot < tiles ? t0 + per_slot : tiles;
            for (int64_t t = t0; t < t1; ++t) {
                const WgTile tl = wg_tile(t, hw);
                for (int lane = 0; lane < 64; ++lane) {
                    const int q = lane & 15, g = lane >> 4;
                    for (int s = 0; s < 4; ++s, ++n)
                        if (!check::in_region(rs, small, wg_small(tl, hw, kk, q, g, s) * 2, 16)) ++bad;
                    for (int i = 0; i < ns; ++i) {
                        const int cc = wg_channel(32 * i, g, cl);
                        if (wt) {
                            const int64_t wo = static_cast<int64_t>(q < kk ? q : kk - 1) * cin + cc;
                            ++n;
                            if (!check::in_region(rw, wt, wo * 2, 16) ||
                                (reinterpret_cast<uint64_t>(wt) + wo * 2) % 16)
                                ++bad;
                        }
                        for (int e = 0; e < 8; ++e, ++n)
                            if (!check::in_region(rb, big, wg_big(tl, hw, cin, q, c0 + cc + e) * 2, 16)) ++bad;
                    }
                    if (wt)
                        for (int i = 0; i < 4; ++i, ++n)
                            if (4 * g + i < kk &&
                                !check::in_region(ro, pout, wg_out(tl, hw, kk, q, 4 * g + i) * 2, 16))
                                ++bad;
                }
            }
            for (int q = 0; q < kk; ++q)
                for (int c = 0; c < cl; ++c, ++n)
                    if (!check::in_region(rp, part, wg_part(slot, cin, kk, q, c0 + c) * 4, 4)) ++bad;
        }
    }
    if (bad) check::violation(kn, "accesses", "%lld bad", static_cast<long long>(bad));
    check::count_accesses(n);
}

void replay_wgrad_partial(const void* big, const void* small, const float* part, int64_t hw, int64_t cin, int64_t kk,
                          int64_t total, int64_t per_slot, int64_t slots, int es) {
    const char* kn = "wgrad_partial_kernel";
    const check::Region rb = check::region_of(big, kn, "big");
    const check::Region rs = check::region_of(small, kn, "small");
    const check::Region rp = check::region_of(part, kn, "partials");
    int64_t bad = 0, n = 0;
    for (int64_t slot = 0; slot < slots; ++slot) {
        const int64_t e0 = slot * per_slot;
        const int64_t e1 = e0 + per_slot < total ? e0 + per_slot : total;
        for (int64_t e = e0; e < e1; ++e) {
            const int64_t ni = e / hw, p = e - ni * hw;
            for (int64_t ci = 0; ci < cin; ++ci, ++n)
                if (!check::in_region(rb, big, ((ni * cin + ci) * hw + p) * es, es)) ++bad;
            for (int64_t k = 0; k < kk; ++k, ++n)
                if (!check::in_region(rs, small, ((ni * kk + k) * hw + p) * es, es)) ++bad;
        }
        for (int64_t ci = 0; ci < cin; ++ci)
            for (int64_t k = 0; k < kk; ++k, ++n)
                if (!check::in_region(rp, part, ((slot * cin + ci) * kk + k) * 4, 4)) ++bad;
    }
    if (bad) check::violation(kn, "accesses", "%lld bad", static_cast<long long>(bad));
    check::count_accesses(n);
}

void replay_wgrad_reduce(const float* part, const float* out, int64_t slots, int64_t count, int64_t kk, int64_t sc,
                         int64_t sk) {
    const char* kn = "wgrad_reduce_kernel";
    const check::Region rp = check::region_of(part, kn, "partials");
    const check::Region ro = check::region_of(out, kn, "gradient");
    int64_t bad = 0;
    for (int64_t e = 0; e < count; ++e) {
        for (int64_t s = 0; s < slots; ++s)
            if (!check::in_region(rp, part, (s * count + e) * 4, 4)) ++bad;
        if (!check::in_region(ro, out, ((e / kk) * sc + (e % kk) * sk) * 4, 4)) ++bad;
    }
    if (bad) check::violation(kn, "accesses", "%lld bad", static_cast<long long>(bad));
    check::count_accesses(count * (slots + 1));
}
#endif

}  // namespace

int64_t wgrad_slots(int64_t n, int64_t hw) {
    const int64_t t = (n * hw + 127) / 128;
    return t < 1 ? 1 : (t > kWgradMaxSlots ? kWgradMaxSlots : t);
}

hipError_t launch_project_wgrad(int64_t n, int64_t c, int64_t hw, int64_t k, const void* big, const void* small,
                                const void* wt, void* pout, float* part, int dtype, hipStream_t stream,
                                int64_t* slots_used) {
    const int64_t total = n * hw;
    if (dtype == kBF16 && hw % 128 == 0 && c % 8 == 0 && c < (int64_t{1} << 24) && k >= 1 && k <= 16 &&
        aligned_to(big, 16) && aligned_to(small, 16)) {
        // the projection folded in when every channel fits one wave's registers
        const bool fold = wt && c <= 32 * kWgradMaxBlocks && aligned_to(wt, 16) && aligned_to(pout, 16);
        if (wt && !fold) {
            const hipError_t e = launch_project(n, c, hw, k, big, wt, pout, dtype, stream);
            if (e != hipSuccess) return e;
        }
        const int ns = static_cast<int>(c <= 32 * kWgradMaxBlocks ? (c + 31) / 32 : kWgradMaxBlocks);
        const int groups = static_cast<int>((c + 32 * ns - 1) / (32 * ns));
        const int64_t tiles = total / 128;
        const int64_t per_slot = (tiles + kWgradMaxSlots - 1) / kWgradMaxSlots;
        const int64_t slots = (tiles + per_slot - 1) / per_slot;
        constexpr int per = kThreads / 64;
        const dim3 grid(static_cast<unsigned>((slots + per - 1) / per), static_cast<unsigned>(groups));
        const auto* b = static_cast<const bf16_t*>(big);
        const auto* sm = static_cast<const bf16_t*>(small);
        const auto* w = fold ? static_cast<const bf16_t*>(wt) : nullptr;
        auto* po = fold ? static_cast<bf16_t*>(pout) : nullptr;
        const int ci = static_cast<int>(c), kk = static_cast<int>(k);
#ifdef GSPN_CHECK_LAUNCHES
        replay_wgrad_mfma(big, small, w, po, part, tiles, per_slot, slots, hw, ci, kk, ns, groups);
        check::replayed("wgrad_mfma", kThreads, int64_t{per} * 32 * 17 * 16);
#endif
        switch (ns * 2 + (fold ? 1 : 0)) {
#define GSPN_WG(k)                                                                                                  \
    case 2 * k:                                                                                                     \
        hipLaunchKernelGGL((wgrad_mfma<k, false>), grid, dim3(kThreads), 0, stream, b, sm, w, po, part,   \
                           tiles, per_slot, hw, ci, kk);                                                            \
        break;                                                                                                      \
    case 2 * k + 1:                                                                                                 \
        hipLaunchKernelGGL((wgrad_mfma<k, true>), grid, dim3(kThreads), 0, stream, b, sm, w, po, part,    \
                           tiles, per_slot, hw, ci, kk);                                                            \
        break;
            GSPN_WG(1) GSPN_WG(2) GSPN_WG(3) GSPN_WG(4) GSPN_WG(5) GSPN_WG(6) GSPN_WG(7) GSPN_WG(8) GSPN_WG(9)
            GSPN_WG(10)
#undef GSPN_WG
            default:
                return hipErrorInvalidValue;
        }
        *slots_used = slots;
        return hipGetLastError();
    }
    if (wt) {
        const hipError_t e = launch_project(n, c, hw, k, big, wt, pout, dtype, stream);
        if (e != hipSuccess) return e;
    }
    int64_t s0 = wgrad_slots(n, hw);
    const int64_t cap = int64_t{0x7fffffff} / (c > 0 ? c : 1);
    if (s0 > cap) s0 = cap;
    const int64_t per_slot = (total + s0 - 1) / s0;
    const int64_t slots = (total + per_slot - 1) / per_slot;
    const dim3 grid(static_cast<unsigned>(slots * c));
#ifdef GSPN_CHECK_LAUNCHES
    replay_wgrad_partial(big, small, part, hw, c, k, total, per_slot, slots, dtype == kF32 ? 4 : 2);
    check::replayed("wgrad_partial_kernel", 256, int64_t{8} * 256 * 4);
#endif
    if (dtype == kF32) {
        hipLaunchKernelGGL(wgrad_partial_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(big),
                           static_cast<const float*>(small), part, hw, c, k, total, per_slot, slots);
    } else {
        hipLaunchKernelGGL(wgrad_partial_kernel<bf16_t>, grid, dim3(256), 0, stream, static_cast<const bf16_t*>(big),
                           static_cast<const bf16_t*>(small), part, hw, c, k, total, per_slot, slots);
    }
    *slots_used = slots;
    return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const float* part, int64_t slots, int64_t c, int64_t k, float* out, int64_t sc,
                               int64_t sk, hipStream_t stream) {
    const int64_t count = c * k;
    const dim3 grid(static_cast<unsigned>((count + 63) / 64));
#ifdef GSPN_CHECK_LAUNCHES
    replay_wgrad_reduce(part, out, slots, count, k, sc, sk);
    check::replayed("wgrad_reduce_kernel", 1024, int64_t{16} * 64 * 4);
#endif
    hipLaunchKernelGGL(wgrad_reduce_kernel, grid, dim3(1024), 0, stream, part, out, slots, count, k, sc, sk);
    return hipGetLastError();
}

}  // namespace gspn
