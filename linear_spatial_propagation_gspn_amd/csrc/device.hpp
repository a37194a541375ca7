// device.hpp -- small device-side helpers shared by the libgspn kernels:
// storage-type loads/stores (fp32, bf16 widened exactly, rounded to nearest
// even on store) and the sigmoid row normalisation of one tridiagonal row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "check.hpp"

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

// Logistic sigmoid 1 / (1 + e^{-z}), to within about 2 ulp over the range
// where it is a normal number.  e^{-z} is 2^{-z log2 e}; the product -z log2 e
// is rounded to fp32, and that rounding alone would cost up to |z| ulp of
// relative error in e^{-z} (20 ulp at z = -20).  Its exact error is recovered
// with one fma (the TwoProduct identity of Ogita, Rump and Oishi, "Accurate
// sum and dot product", 2005), the error of the fp32 constant is added, and
// both enter as the first-order factor 2^err ~ 1 + err ln 2.  The hardware
// exp2 and reciprocal (1 ulp each) finish it (a Newton step on the
// reciprocal measured no more accurate: 3.4 ulp at most on the normalised
// weights either way, mean 0.57 ulp, over z in [-20, 20]).  z is first
// clamped to [-87, 87] (keeping its sign; NaN compares false and passes
// through), which keeps the exponent and its correction finite: the result
// saturates at about 2^-125.5 and 1 - 2^-126 there (a row whose every
// sigmoid is that small is normalised by normalise_row_s's exact fallback);
// NaN propagates.
__device__ __forceinline__ float sigmoid(float z) {
    constexpr float kL2E = 1.44269502162933349609375f;   // log2 e rounded to fp32
    constexpr float kL2ELoLn2 = 1.33497577e-08f;          // (log2 e - kL2E) ln 2
    constexpr float kLn2 = 0.693147182464599609375f;
    const float zc = __builtin_fabsf(z) > 87.0f ? __builtin_copysignf(87.0f, z) : z;
    const float t = -zc * kL2E;
    // (exact remainder of the rounded product + the constant's error) ln 2
    const float c = __builtin_fmaf(__builtin_fmaf(-zc, kL2E, -t), kLn2, -zc * kL2ELoLn2);
    const float e = __builtin_amdgcn_exp2f(t);
    return __builtin_amdgcn_rcpf(1.0f + __builtin_fmaf(e, c, e));
}

// Row normalisation of one tridiagonal row (GSPN summary page, "Approach":
// sigmoid then division by the row sum, so the row sums to 1), keeping the
// sigmoids s (the backward's Jacobian needs them).  has_l / has_r say whether
// the neighbours k-1 / k+1 exist on the line; a missing neighbour gets weight
// exactly 0 and is left out of the sum.  When every sigmoid of the row is
// below 2^-100 (every existing logit below about -69) the sum could underflow,
// so the weights are taken as e^{z_o - max z} / sum instead: there
// 1 + e^{z} rounds to 1 in fp32, so sigmoid(z) = e^{z} and the two forms agree
// to fp32 precision.  That branch is not taken for ordinary logits.
__device__ __forceinline__ void normalise_row_s(float z0, float z1, float z2, bool has_l, bool has_r, float& s0,
                                                float& s1, float& s2, float& w0, float& w1, float& w2) {
    s0 = has_l ? sigmoid(z0) : 0.0f;
    s1 = sigmoid(z1);
    s2 = has_r ? sigmoid(z2) : 0.0f;
    const float sum = (s0 + s1) + s2;
    const float r = recip(sum);
    w0 = s0 * r;
    w1 = s1 * r;
    w2 = s2 * r;
    if (sum < 0x1p-100f) {
        constexpr float kL2E = 1.44269502162933349609375f;
        const float m = __builtin_fmaxf(__builtin_fmaxf(has_l ? z0 : z1, z1), has_r ? z2 : z1);
        const float e0 = has_l ? __builtin_amdgcn_exp2f((z0 - m) * kL2E) : 0.0f;
        const float e1 = __builtin_amdgcn_exp2f((z1 - m) * kL2E);
        const float e2 = has_r ? __builtin_amdgcn_exp2f((z2 - m) * kL2E) : 0.0f;
        const float re = recip((e0 + e1) + e2);  // the largest term is 1: the sum lies in [1, 3]
        w0 = e0 * re;
        w1 = e1 * re;
        w2 = e2 * re;
    }
}

__device__ __forceinline__ void normalise_row(float z0, float z1, float z2, bool has_l, bool has_r, float& w0,
                                              float& w1, float& w2) {
    float s0, s1, s2;
    normalise_row_s(z0, z1, z2, has_l, has_r, s0, s1, s2, w0, w1, w2);
}

}  // namespace gspn
