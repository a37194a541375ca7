// project.hip -- the 1x1 projection between channel spaces (GSPN-2 notes,
// "Optimisation 2", compressive channel proxy):
//   out[n][o][p] = sum_c weight[o][c] * in[n][c][p]   (no bias, fp32 accumulate)
//
// bf16 storage runs on the matrix cores (gfx950 bf16 MFMA, fp32 accumulate):
//  - narrow output (c_out <= 16, c_in % 8 == 0, e.g. C -> C_proxy):
//    v_mfma_f32_16x16x32_bf16 with M = output channels, N = 16 pixels, K = 32
//    input channels per instruction.  A wave covers 128 pixels: each lane
//    loads 8 pixels of 8 input channels with 16-byte loads (16 lanes make one
//    256-byte run of a channel row) and its 8 weights with one 16-byte load,
//    and feeds eight MFMAs, one per pixel of its group (64 pixels and 8-byte
//    loads where the pixel count is not a multiple of 128).
//  - narrow input (c_in <= 8, e.g. C_proxy -> C): v_mfma_f32_32x32x8_bf16
//    with M = 32 output channels, N = 32 pixels, K = 8.  A wave covers 128
//    pixels as four interleaved quarters, so each lane ends with four
//    adjacent pixels of 16 output channels and stores them as one 8-byte
//    vector (32 lanes make one 256-byte run of an output row; 64 pixels and
//    dwords where the pixel count is not a multiple of 128).
// Longer runs per channel row measured faster on MI355X: each wave touches
// every channel row of its pixels once, so fewer, longer runs per row cut
// the rows opened per byte moved.
// Operand layouts (checked on gfx950): lane l holds row l % M of A and column
// l % M of B, with k = (l / M) * KE + e for its KE elements; the 16x16 result
// holds rows (l/16)*4 + i of column l % 16, the 32x32 result rows
// (i/4)*8 + (l/32)*4 + i%4 of column l % 32.
// Everything else (fp32 storage, other channel counts, ragged pixel counts)
// takes a VALU kernel: one lane per pixel, 8 output channels per pass.
#include "device.hpp"
#include "launch.hpp"

namespace gspn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#ifndef GSPN_PROJ_NT
#define GSPN_PROJ_NT 1  // bit 0: activation loads, bit 1: output stores (measured slower)
#endif

// Activation loads and output stores: each touched once per projection;
// with GSPN_PROJ_NT they carry the non-temporal hint.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ldx(const uint2* p) {
    if constexpr ((GSPN_PROJ_NT & 1) != 0) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        return make_uint2(v.x, v.y);
    } else {
        return *p;
    }
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldx(const uint4* p) {
    if constexpr ((GSPN_PROJ_NT & 1) != 0) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}
__device__ __forceinline__ void stx(uint4* p, uint4 v) {
    if constexpr ((GSPN_PROJ_NT & 2) != 0) {
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
    } else {
        *p = v;
    }
}
__device__ __forceinline__ void stx(uint2* p, uint2 v) {
    if constexpr ((GSPN_PROJ_NT & 2) != 0) {
        __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
    } else {
        *p = v;
    }
}
__device__ __forceinline__ void stx(uint32_t* p, uint32_t v) {
    if constexpr ((GSPN_PROJ_NT & 2) != 0) {
        __builtin_nontemporal_store(v, p);
    } else {
        *p = v;
    }
}

__device__ __forceinline__ __bf16 as_bf(uint32_t bits16) {
    return __builtin_bit_cast(__bf16, static_cast<uint16_t>(bits16));
}

// Narrow output: c_out <= 16.  Requires hw % (16 * PX) == 0, c_in % 8 == 0,
// 2 * PX-byte aligned rows and a 16-byte aligned weight matrix.  A wave
// covers 16 * PX pixels, each lane PX consecutive pixels of 8 channels, so 16
// lanes read one run of 32 * PX bytes of a channel row.  Each 32-channel
// block's loads are issued before the previous block's MFMAs (double buffer);
// channel indices past c_in are clamped into the tensor and their values
// replaced by zeros, so no load sits behind a branch.
#ifndef GSPN_PROJ_THREADS
#define GSPN_PROJ_THREADS 256
#endif
#ifndef GSPN_PROJ_PX
#define GSPN_PROJ_PX 8
#endif

template <int PX>
struct PixVec;
template <>
struct PixVec<4> {
    using T = uint2;
    static __device__ __forceinline__ uint32_t word(const T& v, int k) { return k == 0 ? v.x : v.y; }
};
template <>
struct PixVec<8> {
    using T = uint4;
    static __device__ __forceinline__ uint32_t word(const T& v, int k) {
        return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
    }
};

template <int PX, int NS>
__global__ __launch_bounds__(GSPN_PROJ_THREADS) void project_narrow_out_mfma(const bf16_t* __restrict__ in,
                                                                              const bf16_t* __restrict__ wt,
                                                                              bf16_t* __restrict__ out, int64_t waves,
                                                                              int64_t hw, int cin, int cout) {
    using PV = PixVec<PX>;
    using VT = typename PV::T;
    constexpr int WPX = 16 * PX;  // pixels per wave
    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (wave >= waves) return;
    const int64_t per_img = hw / WPX;
    const int64_t ni = wave / per_img;
    const int64_t px0 = (wave - ni * per_img) * WPX;
    const int q = lane & 15;  // pixel group: pixels px0 + PX q .. + PX - 1; output row of A
    const int g = lane >> 4;  // k-group: channels 8g .. 8g+7 of each 32-channel step
    const bf16_t* src = in + ni * cin * hw + px0 + PX * q;
    const bf16_t* wrow = wt + static_cast<int64_t>(q < cout ? q : cout - 1) * cin;
    const bool qok = q < cout;

    struct Block {
        uint4 a;   // 8 weights (bf16) of output row q
        VT v[8];   // PX pixels of 8 channels
        bool ok;   // the channels exist
    };
    auto fetch = [&](int k0, Block& b) {
        const int c0 = k0 + 8 * g;
        b.ok = c0 < cin;
        const int cc = b.ok ? c0 : cin - 8;  // clamped into the tensor (cin % 8 == 0)
        b.a = *reinterpret_cast<const uint4*>(wrow + cc);
#pragma unroll
        for (int e = 0; e < 8; ++e) b.v[e] = ldx(reinterpret_cast<const VT*>(src + static_cast<int64_t>(cc + e) * hw));
    };

    floatx4 acc[PX];
#pragma unroll
    for (int j = 0; j < PX; ++j) acc[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    auto consume = [&](const Block& b) {
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
                const uint32_t word = b.ok ? PV::word(b.v[e], j >> 1) : 0u;
                bv[e] = as_bf((j & 1) ? (word >> 16) : (word & 0xffffu));
            }
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[j], 0, 0, 0);
        }
    };

    if constexpr (NS > 0) {
        // cin <= 32 NS, the block count known here: the loop unrolls into one
        // straight sequence, in which every MFMA waits only for its own block
        // (a loop's back edge makes the compiler wait for every load in
        // flight at its head)
        Block b[2];
        fetch(0, b[0]);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i + 1 < NS) fetch(32 * (i + 1), b[(i + 1) & 1]);
            // keep the next block's loads ahead of this block's wait (the
            // scheduler would otherwise sink them below it)
            __builtin_amdgcn_sched_barrier(0);
            consume(b[i & 1]);
        }
    } else {
        Block b0, b1;
        fetch(0, b0);
        int k0 = 0;
        for (; k0 + 32 < cin; k0 += 64) {
            fetch(k0 + 32, b1);
            consume(b0);
            fetch(k0 + 64, b0);  // past c_in it reads clamped channels and yields zeros
            consume(b1);
        }
        if (k0 < cin) consume(b0);
    }

    // lane holds output rows (l/16)*4 + i for pixels px0 + PX q + j
    bf16_t* dst = out + ni * cout * hw + px0 + PX * q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int o = g * 4 + i;
        if (o < cout) {
            uint32_t w[PX / 2];
#pragma unroll
            for (int k = 0; k < PX / 2; ++k) w[k] = pack_bf16x2(acc[2 * k][i], acc[2 * k + 1][i]);
            bf16_t* d = dst + static_cast<int64_t>(o) * hw;
            if constexpr (PX == 4) {
                stx(reinterpret_cast<uint2*>(d), make_uint2(w[0], w[1]));
            } else {
                stx(reinterpret_cast<uint4*>(d), make_uint4(w[0], w[1], w[2], w[3]));
            }
        }
    }
}

// Narrow input: c_in <= 8.  Requires hw % (32 * PQ) == 0 and 2 * PQ-byte
// aligned rows.  A wave covers 32 * PQ pixels: lane n holds PQ consecutive
// pixels, one MFMA per pixel of its group, so each lane stores PQ adjacent
// pixels of an output row at once (32 lanes make one run of 64 * PQ bytes).
#ifndef GSPN_PROJ_PQ
#define GSPN_PROJ_PQ 4
#endif

template <int PQ>
__global__ __launch_bounds__(256) void project_narrow_in_mfma(const bf16_t* __restrict__ in,
                                                              const bf16_t* __restrict__ wt,
                                                              bf16_t* __restrict__ out, int64_t waves,
                                                              int64_t hw, int cin, int cout) {
    static_assert(PQ == 2 || PQ == 4, "2 or 4 pixels per lane");
    constexpr int WPX = 32 * PQ;  // pixels per wave
    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (wave >= waves) return;
    const int64_t per_img = hw / WPX;
    const int64_t ni = wave / per_img;
    const int64_t px0 = (wave - ni * per_img) * WPX;
    const int n = lane & 31;  // pixel group: pixels px0 + PQ n .. + PQ - 1; output row of A
    const int g = lane >> 5;  // k-group: input channels 4g .. 4g+3
    const bf16_t* src = in + ni * cin * hw + px0 + PQ * n;

    short4v b[PQ];  // B operand of each pixel of the group
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = 4 * g + e;
        const bf16_t* row = src + static_cast<int64_t>(c < cin ? c : cin - 1) * hw;
        uint32_t words[PQ / 2];
        if constexpr (PQ == 2) {
            words[0] = *reinterpret_cast<const uint32_t*>(row);
        } else {
            const uint2 v = *reinterpret_cast<const uint2*>(row);
            words[0] = v.x;
            words[1] = v.y;
        }
#pragma unroll
        for (int k = 0; k < PQ; ++k) {
            const uint32_t word = c < cin ? words[k >> 1] : 0u;
            b[k][e] = static_cast<short>((k & 1) ? (word >> 16) : (word & 0xffffu));
        }
    }
    bf16_t* dst = out + ni * cout * hw + px0 + PQ * n;
    for (int o0 = 0; o0 < cout; o0 += 32) {
        short4v a;
        const int orow = o0 + n;
        const int oc = orow < cout ? orow : cout - 1;  // clamped: loads stay unguarded
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 4 * g + e;
            const bf16_t v = wt[oc * cin + (c < cin ? c : cin - 1)];
            a[e] = static_cast<short>((orow < cout && c < cin) ? v : 0);
        }
        floatx16 acc[PQ];
#pragma unroll
        for (int k = 0; k < PQ; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b[k], floatx16{}, 0, 0, 0);
        // lane holds output rows (i/4)*8 + (l/32)*4 + i%4 for its pixel group
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int o = o0 + (i / 4) * 8 + g * 4 + (i % 4);
            if (o < cout) {
                bf16_t* d = dst + static_cast<int64_t>(o) * hw;
                if constexpr (PQ == 2) {
                    stx(reinterpret_cast<uint32_t*>(d), pack_bf16x2(acc[0][i], acc[1][i]));
                } else {
                    stx(reinterpret_cast<uint2*>(d), make_uint2(pack_bf16x2(acc[0][i], acc[1][i]),
                                                                pack_bf16x2(acc[2][i], acc[3][i])));
                }
            }
        }
    }
}

// VALU projection: one lane per pixel, OB output channels per pass over the
// input channels (weights are wave-uniform and come through the scalar cache).
template <typename T, int OB>
__global__ __launch_bounds__(256) void project_kernel(const T* __restrict__ in, const T* __restrict__ wt,
                                                      T* __restrict__ out, int64_t n, int64_t cin,
                                                      int64_t hw, int64_t cout) {
    const int64_t total = n * hw;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
         e += stride) {
        const int64_t ni = e / hw;
        const int64_t pix = e - ni * hw;
        const T* src = in + ni * cin * hw + pix;
        T* dst = out + ni * cout * hw + pix;
        for (int64_t o0 = 0; o0 < cout; o0 += OB) {
            float acc[OB];
#pragma unroll
            for (int oo = 0; oo < OB; ++oo) acc[oo] = 0.0f;
            for (int64_t ci = 0; ci < cin; ++ci) {
                const float v = Store<T>::ld(src + ci * hw);
#pragma unroll
                for (int oo = 0; oo < OB; ++oo) {
                    if (o0 + oo < cout)
                        acc[oo] = __builtin_fmaf(Store<T>::ld(wt + (o0 + oo) * cin + ci), v, acc[oo]);
                }
            }
#pragma unroll
            for (int oo = 0; oo < OB; ++oo)
                if (o0 + oo < cout) Store<T>::st(dst + (o0 + oo) * hw, acc[oo]);
        }
    }
}

bool aligned_to(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

}  // namespace

hipError_t launch_project(int64_t n, int64_t c_in, int64_t hw, int64_t c_out, const void* in,
                          const void* weight, void* out, int dtype, hipStream_t stream) {
    if (dtype == kBF16 && hw % 64 == 0 && c_in <= 1 << 20 && c_out <= 1 << 20) {
        const int64_t waves = n * (hw / 64);
        const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
        constexpr int PX = GSPN_PROJ_PX;
        if (c_out <= 16 && c_in % 8 == 0 && hw % (16 * PX) == 0 && aligned_to(in, 2 * PX) &&
            aligned_to(out, 2 * PX) && aligned_to(weight, 16)) {
            constexpr int per = GSPN_PROJ_THREADS / 64;
            const int64_t w2 = n * (hw / (16 * PX));
            const dim3 g2(static_cast<unsigned>((w2 + per - 1) / per));
            const auto* src = static_cast<const bf16_t*>(in);
            const auto* wts = static_cast<const bf16_t*>(weight);
            auto* dst = static_cast<bf16_t*>(out);
            const int ci = static_cast<int>(c_in), co = static_cast<int>(c_out);
            switch ((c_in + 31) / 32) {  // unrolled instances for up to 512 input channels
#define GSPN_PROJ_NS(k) \
    case k: hipLaunchKernelGGL((project_narrow_out_mfma<PX, k>), g2, dim3(GSPN_PROJ_THREADS), 0, stream, src, wts, dst, w2, hw, ci, co); break;
                GSPN_PROJ_NS(1) GSPN_PROJ_NS(2) GSPN_PROJ_NS(3) GSPN_PROJ_NS(4) GSPN_PROJ_NS(5) GSPN_PROJ_NS(6)
                GSPN_PROJ_NS(7) GSPN_PROJ_NS(8) GSPN_PROJ_NS(9) GSPN_PROJ_NS(10) GSPN_PROJ_NS(11) GSPN_PROJ_NS(12)
                GSPN_PROJ_NS(13) GSPN_PROJ_NS(14) GSPN_PROJ_NS(15) GSPN_PROJ_NS(16)
#undef GSPN_PROJ_NS
                default:
                    hipLaunchKernelGGL((project_narrow_out_mfma<PX, 0>), g2, dim3(GSPN_PROJ_THREADS), 0, stream, src,
                                       wts, dst, w2, hw, ci, co);
            }
            return hipGetLastError();
        }
        if (c_out <= 16 && c_in % 8 == 0 && aligned_to(in, 8) && aligned_to(out, 8) && aligned_to(weight, 16)) {
            constexpr int per = GSPN_PROJ_THREADS / 64;
            const dim3 g2(static_cast<unsigned>((waves + per - 1) / per));
            hipLaunchKernelGGL((project_narrow_out_mfma<4, 0>), g2, dim3(GSPN_PROJ_THREADS), 0, stream,
                               static_cast<const bf16_t*>(in), static_cast<const bf16_t*>(weight),
                               static_cast<bf16_t*>(out), waves, hw, static_cast<int>(c_in),
                               static_cast<int>(c_out));
            return hipGetLastError();
        }
        constexpr int PQ = GSPN_PROJ_PQ;
        if (c_in <= 8 && hw % (32 * PQ) == 0 && aligned_to(in, 2 * PQ) && aligned_to(out, 2 * PQ)) {
            const int64_t w2 = n * (hw / (32 * PQ));
            hipLaunchKernelGGL(project_narrow_in_mfma<PQ>, dim3(static_cast<unsigned>((w2 + 3) / 4)), dim3(256), 0,
                               stream, static_cast<const bf16_t*>(in), static_cast<const bf16_t*>(weight),
                               static_cast<bf16_t*>(out), w2, hw, static_cast<int>(c_in), static_cast<int>(c_out));
            return hipGetLastError();
        }
        if (c_in <= 8 && aligned_to(in, 4) && aligned_to(out, 4)) {
            hipLaunchKernelGGL(project_narrow_in_mfma<2>, grid, dim3(256), 0, stream,
                               static_cast<const bf16_t*>(in), static_cast<const bf16_t*>(weight),
                               static_cast<bf16_t*>(out), waves, hw, static_cast<int>(c_in),
                               static_cast<int>(c_out));
            return hipGetLastError();
        }
    }
    const int64_t total = n * hw;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    if (blocks < 1) blocks = 1;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (dtype == kF32) {
        hipLaunchKernelGGL((project_kernel<float, 8>), grid, dim3(256), 0, stream,
                           static_cast<const float*>(in), static_cast<const float*>(weight),
                           static_cast<float*>(out), n, c_in, hw, c_out);
    } else {
        hipLaunchKernelGGL((project_kernel<bf16_t, 8>), grid, dim3(256), 0, stream,
                           static_cast<const bf16_t*>(in), static_cast<const bf16_t*>(weight),
                           static_cast<bf16_t*>(out), n, c_in, hw, c_out);
    }
    return hipGetLastError();
}

}  // namespace gspn
