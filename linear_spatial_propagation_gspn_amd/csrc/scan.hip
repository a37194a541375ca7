// scan.hip -- the line-scan kernel: one workgroup runs one (plane, chunk)
// line scan with h held in registers.
//
// What it computes (GSPN-2 paper notes, "2D spatial propagation recap"):
//   h_i[k] = sum_{o in {-1,0,+1}, 0 <= k+o < L} w_i[k,o] h_{i-1}[k+o]
//            + lambda_i[k] x_i[k]
// for the lines i of one direction in scan order, with h = 0 before the
// first line of the scan and of every chunk ("Optimisation 1": independent
// (chunk, n, c) blocks).  w_i is the sigmoid row normalisation of the three
// logits at (i, k) (GSPN summary page, "Approach").
//
// Mapping on gfx950: a workgroup owns one line of L positions; each lane owns
// P contiguous positions, so a step reads P contiguous values per stream and
// the whole line is one coalesced row of the scan-frame tensors.  h stays in
// VGPRs for the whole scan; the two values a lane needs from its neighbours
// (h[k0-1] and h[k0+P]) go through a double-buffered LDS edge array with one
// barrier per step.  The inputs of the next D steps are prefetched into a
// register ring so that HBM latency overlaps the serial chain of steps.
#include "device.hpp"
#include "launch.hpp"

namespace gspn {
namespace {

constexpr int kMaxThreads = 1024;

struct ScanK {
    const void* x;
    const void* wts;
    const void* lam;
    void* out;
    int64_t c;
    int64_t cw;
    int S;          // scan steps
    int L;          // line length
    int K;          // steps per chunk
    int nchunks;
    int reverse;
    int logits;     // wts holds logits (1) or normalised weights (0)
    int accumulate;
    int vec_frame;  // scan-frame tensors (wts, lam) allow P-wide vector access
    int vec_arr;    // array-frame tensors (x, out) allow P-wide vector access (vertical only)
};

template <typename T, int P>
struct alignas(sizeof(T) * P) VecT {
    T e[P];
};

// P values of a line starting at position k0; positions >= L read as 0.
template <typename T, int P>
__device__ __forceinline__ void load_run(const T* __restrict__ base, int k0, int L, bool vec,
                                         float (&dst)[P]) {
    if (vec) {
        const VecT<T, P> v = *reinterpret_cast<const VecT<T, P>*>(base + k0);
#pragma unroll
        for (int j = 0; j < P; ++j) dst[j] = Store<T>::ld(&v.e[j]);
    } else {
#pragma unroll
        for (int j = 0; j < P; ++j) dst[j] = (k0 + j < L) ? Store<T>::ld(base + k0 + j) : 0.0f;
    }
}

template <typename T, int P>
__device__ __forceinline__ void store_run(T* __restrict__ base, int k0, int L, bool vec,
                                          const float (&src)[P]) {
    if (vec) {
        VecT<T, P> v;
#pragma unroll
        for (int j = 0; j < P; ++j) Store<T>::st(&v.e[j], src[j]);
        *reinterpret_cast<VecT<T, P>*>(base + k0) = v;
    } else {
#pragma unroll
        for (int j = 0; j < P; ++j)
            if (k0 + j < L) Store<T>::st(base + k0 + j, src[j]);
    }
}

template <typename T, int P, int D, bool HORIZ, int MAXT>
__global__ __launch_bounds__(MAXT) void scan_kernel(const ScanK a) {
    // [buffer][0 = first position, 1 = last position][thread]
    __shared__ float s_edge[2][2][kMaxThreads];

    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int64_t blk = blockIdx.x;
    const int64_t p = blk / a.nchunks;           // plane n * c + ci
    const int q = static_cast<int>(blk - p * a.nchunks);
    const int64_t nidx = p / a.c;
    const int64_t ci = p - nidx * a.c;
    const int S = a.S;
    const int L = a.L;
    const int64_t plane = static_cast<int64_t>(S) * L;

    const T* __restrict__ xp = static_cast<const T*>(a.x) + p * plane;
    const T* __restrict__ lp = static_cast<const T*>(a.lam) + p * plane;
    const T* __restrict__ zp =
        static_cast<const T*>(a.wts) + (nidx * a.cw + (a.cw == 1 ? 0 : ci)) * 3 * plane;
    T* __restrict__ op = static_cast<T*>(a.out) + p * plane;

    const int k0 = tid * P;
    const int t0 = q * a.K;
    const int t1 = min(t0 + a.K, S);
    const bool vf = a.vec_frame && (k0 + P <= L);
    const bool va = !HORIZ && a.vec_arr && (k0 + P <= L);
    const bool acc = a.accumulate != 0;

    // Register ring: inputs of the steps t .. t+D-1.
    float rz[D][3][P];
    float rl[D][P];
    float rx[D][P];
    float ry[D][P];

    auto fetch = [&](int slot, int t) {
        if (t >= t1) return;
        const int i = a.reverse ? S - 1 - t : t;
        const int64_t lo = static_cast<int64_t>(i) * L;
#pragma unroll
        for (int o = 0; o < 3; ++o) load_run<T, P>(zp + o * plane + lo, k0, L, vf, rz[slot][o]);
        load_run<T, P>(lp + lo, k0, L, vf, rl[slot]);
        if (HORIZ) {
            // array element (row k, column i); rows are S long
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const int k = k0 + j;
                const int64_t ao = static_cast<int64_t>(k) * S + i;
                rx[slot][j] = (k < L) ? Store<T>::ld(xp + ao) : 0.0f;
                ry[slot][j] = (acc && k < L) ? Store<T>::ld(op + ao) : 0.0f;
            }
        } else {
            load_run<T, P>(xp + lo, k0, L, va, rx[slot]);
            if (acc) load_run<T, P>(op + lo, k0, L, va, ry[slot]);
        }
    };

    float h[P];
#pragma unroll
    for (int j = 0; j < P; ++j) h[j] = 0.0f;

#pragma unroll
    for (int s = 0; s < D; ++s) fetch(s, t0 + s);

    int buf = 0;
    for (int tb = t0; tb < t1; tb += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int t = tb + s;
            if (t < t1) {
                const int i = a.reverse ? S - 1 - t : t;
                const bool first = (t == t0);
                float left = 0.0f, right = 0.0f;
                if (!first) {
                    left = tid > 0 ? s_edge[buf][1][tid - 1] : 0.0f;
                    right = tid + 1 < nt ? s_edge[buf][0][tid + 1] : 0.0f;
                }
                float hn[P];
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const int k = k0 + j;
                    float u = rl[s][j] * rx[s][j];
                    if (!first) {
                        float w0, w1, w2;
                        const bool has_l = k > 0;
                        const bool has_r = k + 1 < L;
                        if (a.logits) {
                            normalise_row(rz[s][0][j], rz[s][1][j], rz[s][2][j], has_l, has_r, w0,
                                          w1, w2);
                        } else {
                            w0 = has_l ? rz[s][0][j] : 0.0f;
                            w1 = rz[s][1][j];
                            w2 = has_r ? rz[s][2][j] : 0.0f;
                        }
                        const float hl = (j == 0) ? left : h[j - 1];
                        const float hr = (j == P - 1) ? right : h[j + 1];
                        u = __builtin_fmaf(w0, hl, __builtin_fmaf(w1, h[j], __builtin_fmaf(w2, hr, u)));
                    }
                    hn[j] = (k < L) ? u : 0.0f;
                }
                // write out (or accumulate into) the output line
                float ov[P];
#pragma unroll
                for (int j = 0; j < P; ++j) ov[j] = acc ? ry[s][j] + hn[j] : hn[j];
                if (HORIZ) {
#pragma unroll
                    for (int j = 0; j < P; ++j) {
                        const int k = k0 + j;
                        if (k < L) Store<T>::st(op + static_cast<int64_t>(k) * S + i, ov[j]);
                    }
                } else {
                    store_run<T, P>(op + static_cast<int64_t>(i) * L, k0, L, va, ov);
                }
#pragma unroll
                for (int j = 0; j < P; ++j) h[j] = hn[j];

                fetch(s, t + D);

                buf ^= 1;
                s_edge[buf][0][tid] = h[0];
                s_edge[buf][1][tid] = h[P - 1];
                __syncthreads();
            }
        }
    }
}

template <typename T, int P, int D, bool HORIZ, int MAXT>
hipError_t launch_t(const ScanK& k, int64_t nblocks, int nthreads, hipStream_t stream) {
    hipLaunchKernelGGL((scan_kernel<T, P, D, HORIZ, MAXT>), dim3(static_cast<unsigned>(nblocks)),
                       dim3(nthreads), 0, stream, k);
    return hipGetLastError();
}

template <typename T, bool HORIZ>
hipError_t dispatch_p(int P, const ScanK& k, int64_t nblocks, int nthreads, hipStream_t stream) {
    // Up to 256 lanes: a 4-deep prefetch ring fits the register budget.
    // Longer lines (> 2048 positions) take up to 1024 lanes of 8 positions
    // with a 2-deep ring so that 16 waves still fit a CU's registers.
    if (nthreads > 256) return launch_t<T, 8, 2, HORIZ, 1024>(k, nblocks, nthreads, stream);
    switch (P) {
        case 1: return launch_t<T, 1, 4, HORIZ, 256>(k, nblocks, nthreads, stream);
        case 2: return launch_t<T, 2, 4, HORIZ, 256>(k, nblocks, nthreads, stream);
        case 4: return launch_t<T, 4, 4, HORIZ, 256>(k, nblocks, nthreads, stream);
        default: return launch_t<T, 8, 4, HORIZ, 256>(k, nblocks, nthreads, stream);
    }
}

bool aligned_to(const void* ptr, size_t bytes) {
    return (reinterpret_cast<uintptr_t>(ptr) % bytes) == 0;
}

}  // namespace

hipError_t launch_scan(const ScanParams& p, hipStream_t stream) {
    const bool horiz = (p.dir == 2 || p.dir == 3);
    const int S = static_cast<int>(horiz ? p.w : p.h);
    const int L = static_cast<int>(horiz ? p.h : p.w);
    // positions per lane: keep a workgroup at <= 256 lanes where the line
    // allows it, up to 1024 lanes for the longest lines
    int P = 1;
    while (P < 8 && (L + P - 1) / P > 256) P *= 2;
    const int lanes = (L + P - 1) / P;
    const int nthreads = ((lanes + 63) / 64) * 64;
    const size_t esz = p.dtype == kF32 ? 4 : 2;

    ScanK k;
    k.x = p.x;
    k.wts = p.wts;
    k.lam = p.lam;
    k.out = p.out;
    k.c = p.c;
    k.cw = p.cw;
    k.S = S;
    k.L = L;
    k.K = static_cast<int>(p.chunk);
    k.nchunks = (S + k.K - 1) / k.K;
    k.reverse = (p.dir == 1 || p.dir == 3) ? 1 : 0;
    k.logits = p.wts_are_logits ? 1 : 0;
    k.accumulate = p.accumulate ? 1 : 0;
    k.vec_frame = (L % P == 0) && aligned_to(p.wts, esz * P) && aligned_to(p.lam, esz * P);
    k.vec_arr = (L % P == 0) && aligned_to(p.x, esz * P) && aligned_to(p.out, esz * P);
    const int64_t nblocks = p.n * p.c * k.nchunks;

    if (p.dtype == kF32) {
        return horiz ? dispatch_p<float, true>(P, k, nblocks, nthreads, stream)
                     : dispatch_p<float, false>(P, k, nblocks, nthreads, stream);
    }
    return horiz ? dispatch_p<bf16_t, true>(P, k, nblocks, nthreads, stream)
                 : dispatch_p<bf16_t, false>(P, k, nblocks, nthreads, stream);
}

}  // namespace gspn
