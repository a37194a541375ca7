// device.hpp -- small device-side helpers shared by the libgspn kernels:
// storage-type loads/stores (fp32, bf16 widened exactly, rounded to nearest
// even on store) and the sigmoid row normalisation of one tridiagonal row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gspn {

using bf16_t = uint16_t;  // bf16 storage as raw bits

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// gfx950 has a native round-to-nearest-even fp32 -> bf16 conversion
// (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float v) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(v));
}

// Two values rounded the same way, packed low-half first in one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    typedef float f32x2_v __attribute__((ext_vector_type(2)));
    const f32x2_v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

template <typename T>
struct Store;

template <>
struct Store<float> {
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
    static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};

template <>
struct Store<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Pre-normalised channel-shared weights for 16-bit storage: one 32-bit word
// per position holding w_{k-1} (low half) and w_{k+1} (high half) as IEEE
// half precision; the centre weight is recovered as 1 - w_{k-1} - w_{k+1} in
// fp32, so every row still sums to 1.  (fp16 keeps 11 significant bits over
// the weights' range [0, 1].)  WPair tags this format as a weight type.
struct WPair {};

__device__ __forceinline__ uint32_t pack_pair(float wl, float wr) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(wl))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(wr))) << 16);
}

__device__ __forceinline__ float pair_lo(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b & 0xffffu)));
}

__device__ __forceinline__ float pair_hi(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b >> 16)));
}

// Element loads / stores with the non-temporal hint, for data a kernel
// touches once (widened / rounded like Store<T>).
template <typename T>
__device__ __forceinline__ float ld_stream(const T* p) {
    if constexpr (sizeof(T) == 4) {
        return __builtin_nontemporal_load(reinterpret_cast<const float*>(p));
    } else {
        return bf16_to_f32(__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p)));
    }
}

template <typename T>
__device__ __forceinline__ void st_stream(T* p, float v) {
    if constexpr (sizeof(T) == 4) {
        __builtin_nontemporal_store(v, reinterpret_cast<float*>(p));
    } else {
        __builtin_nontemporal_store(f32_to_bf16(v), reinterpret_cast<uint16_t*>(p));
    }
}

// 1 / d to within about half an ulp: the hardware reciprocal (1 ulp) refined
// by one Newton step.
__device__ __forceinline__ float recip(float d) {
    float r = __builtin_amdgcn_rcpf(d);
    float e = __builtin_fmaf(-d, r, 1.0f);
    return __builtin_fmaf(r, e, r);
}

// Logistic sigmoid 1 / (1 + e^{-z}).  e^{-z} is evaluated as 2^{-z log2 e}
// with the hardware exp2; it saturates to +inf for z below about -88, which
// gives sigmoid = 0, and to 0 for large z, which gives 1.
__device__ __forceinline__ float sigmoid(float z) {
    const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// Row normalisation of one tridiagonal row (GSPN summary page, "Approach":
// sigmoid then division by the row sum, so the row sums to 1).  has_l /
// has_r say whether the neighbours k-1 / k+1 exist on the line; a missing
// neighbour gets weight exactly 0 and is left out of the sum.
__device__ __forceinline__ void normalise_row(float z0, float z1, float z2, bool has_l, bool has_r,
                                              float& w0, float& w1, float& w2) {
    const float s0 = has_l ? sigmoid(z0) : 0.0f;
    const float s1 = sigmoid(z1);
    const float s2 = has_r ? sigmoid(z2) : 0.0f;
    const float r = recip((s0 + s1) + s2);
    w0 = s0 * r;
    w1 = s1 * r;
    w2 = s2 * r;
}

}  // namespace gspn
