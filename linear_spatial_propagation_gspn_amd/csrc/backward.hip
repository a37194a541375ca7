// backward.hip -- the adjoint line scan: gradients of the four-direction
// propagation with respect to x, lambda and the logits.
//
// The pages define the forward propagation (GSPN-2 paper notes, "2D spatial
// propagation recap"; chunks from "Optimisation 1", channel-shared logits
// from "Optimisation 2") and report backward runtimes (GSPN-2 summary page,
// "Experimental setup"); the gradient is its exact derivative.  In the scan
// frame of a direction, with u_t = lambda_t * x_t and
// h_t = M_t h_{t-1} + u_t ((M_t v)[k] = sum_o w_t[k,o] v[k+o], no M_t at a
// chunk's first step), and g_t = dL/dy at line t:
//   a_t          = g_t + M_{t+1}^T a_{t+1}        (backwards in t, per chunk)
//   dlambda_t[k] = a_t[k] x_t[k]
//   dx_t[k]     += a_t[k] lambda_t[k]             (summed over the directions)
//   dw_t[k,o]    = a_t[k] h_{t-1}[k+o]            (not at a chunk's first step)
//   dz_t[k,q]    = w_q (1 - s_q) (dw_q - sum_o dw_o w_o),  s_q = sigmoid(z_q)
// (M^T v)[k] = w[k+1,-1] v[k+1] + w[k,0] v[k] + w[k-1,+1] v[k-1], so each lane
// publishes the products w[k,-1] a[k] and w[k,+1] a[k] of its outer positions
// for its neighbours, the same one-barrier LDS edge exchange as the forward.
//
// One workgroup per (direction, plane, chunk) line in vertical form: the
// horizontal directions run on x and dL/dy transposed into their scan frame,
// reading the forward states h recomputed beforehand into separate maps.  The
// per-step inputs of the next D steps are in flight (ring slots refilled as
// soon as read, compile-time slot indices, addresses clamped instead of
// guarded).  Streams touched once carry the non-temporal hint when the
// lines are whole cache lines.
#include <utility>

#include "device.hpp"
#include "launch.hpp"

namespace gspn {
namespace {

template <int V>
using IC = std::integral_constant<int, V>;

// steps in flight: 4 for one position and channel per lane, else 2
// (register budget)
template <int P, int G>
constexpr int adj_depth() { return (P == 1 && G == 1) ? 4 : 2; }

// channels per workgroup for channel-shared logits (fewer for two positions
// per lane: register budget; with the learnable merge's extra state the
// four-channel groups spill a few registers, and still measured faster than
// groups of two)
template <int P>
constexpr int shared_group() { return P == 1 ? 4 : 2; }

struct AdjK {
    const void* x;    // [planes][S][L] (x, or x transposed for horizontal)
    const void* g;    // dL/dy in the same frame
    const void* lam;  // [planes][S][L]
    const void* z;    // logits [n][cw][3][S][L]
    const float* hs;  // forward states [planes][S][L], fp32
    void* dlam;       // [planes][S][L]
    void* dz;         // [n][cw][3][S][L] in the storage type, or fp32 sums for shared logits
    void* dx;         // this direction's dx term [planes][S][L]
    int64_t c;
    int64_t cw;
    int S;
    int L;
    int K;
    int nchunks;
    int reverse;
    int shared;  // dz holds fp32 channel sums of weight-gradient differences (atomic adds; groups of shared_group<P>() channels)
    const float* mscale;  // learnable merge weight of each channel for this direction ([c]), or null for 1
    float* dmerge;        // its gradient [c] (fp32 atomic adds), or null
};

struct Adj4K {
    AdjK d[4];
    int64_t blocks[4];
};

// One (plane group, chunk) line of one direction.  G channels of the same
// image run together (G > 1 only for channel-shared logits): the logits of a
// position are normalised once for all of them, and the logit gradient, which
// sums over channels, is accumulated over the G channels in registers before
// it leaves the workgroup (one atomic add per logit and G channels).
// MERGE: learnable merge weights or their gradient are in play.  With a
// merge weight m for (direction, channel), the direction's output enters y as
// m h, so its adjoint input is m g: the adjoint a runs on g itself and every
// gradient it feeds is scaled by m, while
// dL/dm = sum_t <g_t, h_t> = sum_t <a_t, lambda_t x_t> (the adjoint identity
// of the linear recurrence, per chunk) is summed on the way.  Without MERGE
// none of this costs registers.
// NT: the streams touched once carry the non-temporal hint; only for lines
// of whole 128-byte cache lines (for shorter, unaligned rows the hint makes
// consecutive steps fetch their shared lines twice).
template <typename T, bool NT>
__device__ __forceinline__ float ld_once(const T* p) {
    if constexpr (NT) return ld_stream(p);
    else return Store<T>::ld(p);
}
template <typename T, bool NT>
__device__ __forceinline__ void st_once(T* p, float v) {
    if constexpr (NT) st_stream(p, v);
    else Store<T>::st(p, v);
}

template <typename T, int P, int G, bool MERGE, bool NT>
__device__ __forceinline__ void adj_line(const AdjK& a, int64_t pg, int q, float* edge_raw) {
    constexpr int D = adj_depth<P, G>();
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int S = a.S;
    const int L = a.L;
    const int64_t plane = static_cast<int64_t>(S) * L;
    const int64_t groups = (a.c + G - 1) / G;
    const int64_t nidx = pg / groups;
    const int64_t c0 = (pg - nidx * groups) * G;  // first channel of the group
    const int64_t p0 = nidx * a.c + c0;           // its plane
    int gc[G];                                    // channel offset of each member, clamped
    bool gok[G];
    float msc[G];                                 // merge weight of each member (MERGE)
    float dm[G];                                  // this lane's share of dL/dm (MERGE)
#pragma unroll
    for (int g = 0; g < G; ++g) {
        gok[g] = c0 + g < a.c;
        gc[g] = gok[g] ? g : 0;
        msc[g] = (MERGE && a.mscale) ? a.mscale[c0 + gc[g]] : 1.0f;
        dm[g] = 0.0f;
    }
    const T* xp = static_cast<const T*>(a.x) + p0 * plane;
    const T* gp = static_cast<const T*>(a.g) + p0 * plane;
    const T* lp = static_cast<const T*>(a.lam) + p0 * plane;
    const float* hp = a.hs + p0 * plane;
    const int64_t zplane = (nidx * a.cw + (a.cw == 1 ? 0 : c0)) * 3 * plane;
    const T* zp = static_cast<const T*>(a.z) + zplane;
    T* dlp = static_cast<T*>(a.dlam) + p0 * plane;
    T* dxp = static_cast<T*>(a.dx) + p0 * plane;

    auto edge = [&](int b, int side, int g, int lane) -> float& {
        return edge_raw[((b * 2 + side) * G + g) * nt + lane];
    };

    const int k0 = tid * P;
    int kk[P];
    bool kin[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        kk[j] = min(k0 + j, L - 1);
        kin[j] = k0 + j < L;
    }
    const int kl = max(k0 - 1, 0);      // left neighbour of the first position (clamped)
    const int kr = min(k0 + P, L - 1);  // right neighbour of the last position (clamped)

    const int t0 = q * a.K;
    const int t1 = min(t0 + a.K, S);
    const bool rev = a.reverse != 0;
    auto line_of = [&](int t) { return rev ? S - 1 - t : t; };

    // ring: per step and channel g, x, lambda and h_{t-1} at the positions
    // and their two outer neighbours; the three logits (shared by the group)
    float rg[D][G][P], rx[D][G][P], rl[D][G][P], rh[D][G][P + 2], rz[D][3][P];
    auto fill = [&](auto slot, int t) {
        constexpr int s = decltype(slot)::value;
        const int tc = max(t, t0);
        const int64_t lo = static_cast<int64_t>(line_of(tc)) * L;
        const int64_t hlo = static_cast<int64_t>(line_of(max(tc - 1, t0))) * L;  // h_{t-1} (clamped)
#pragma unroll
        for (int j = 0; j < P; ++j) {
#pragma unroll
            for (int o = 0; o < 3; ++o) {
                // per-channel logits are read once; a channel group's shared logits are re-read
                rz[s][o][j] = G == 1 ? ld_once<T, NT>(zp + o * plane + lo + kk[j]) : Store<T>::ld(zp + o * plane + lo + kk[j]);
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t go = gc[g] * plane;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                rg[s][g][j] = ld_once<T, NT>(gp + go + lo + kk[j]);
                rx[s][g][j] = Store<T>::ld(xp + go + lo + kk[j]);
                rl[s][g][j] = ld_once<T, NT>(lp + go + lo + kk[j]);
                rh[s][g][j + 1] = hp[go + hlo + kk[j]];
            }
            rh[s][g][0] = hp[go + hlo + kl];
            rh[s][g][P + 1] = hp[go + hlo + kr];
        }
    };

    float qn0[G][P];  // w_{t+1}[k,-1] a_{t+1}[k]  (for position k-1)
    float qn1[G][P];  // w_{t+1}[k, 0] a_{t+1}[k]
    float qn2[G][P];  // w_{t+1}[k,+1] a_{t+1}[k]  (for position k+1)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < P; ++j) qn0[g][j] = qn1[g][j] = qn2[g][j] = 0.0f;
    int buf = 0;

    auto step = [&](auto slot, auto lastc, int t) {
        constexpr int s = decltype(slot)::value;
        constexpr bool LAST = decltype(lastc)::value != 0;  // t = t1 - 1: no line after it in the chunk
        const bool first = (t == t0);  // chunk's first line: logits unused, no h_{t-1}
        const int i = line_of(t);
        const int64_t lo = static_cast<int64_t>(i) * L;
        // this line's weights (and sigmoids), shared by the group
        float w[3][P], sg[3][P];
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const bool has_l = k0 + j > 0;
            const bool has_r = k0 + j + 1 < L;
            const float s0 = has_l ? sigmoid(rz[s][0][j]) : 0.0f;
            const float s1 = sigmoid(rz[s][1][j]);
            const float s2 = has_r ? sigmoid(rz[s][2][j]) : 0.0f;
            const float r = recip((s0 + s1) + s2);
            sg[0][j] = s0;
            sg[1][j] = s1;
            sg[2][j] = s2;
            w[0][j] = s0 * r;
            w[1][j] = s1 * r;
            w[2][j] = s2 * r;
        }
        float dw[P][3];  // weight gradient summed over the group
#pragma unroll
        for (int j = 0; j < P; ++j) dw[j][0] = dw[j][1] = dw[j][2] = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float right_in = 0.0f, left_in = 0.0f;  // products from the neighbour lanes
            if constexpr (!LAST) {
                right_in = tid + 1 < nt ? edge(buf, 0, g, tid + 1) : 0.0f;  // w[k0+P,-1] a[k0+P]
                left_in = tid > 0 ? edge(buf, 1, g, tid - 1) : 0.0f;        // w[k0-1,+1] a[k0-1]
            }
            float a_t[P];
#pragma unroll
            for (int j = 0; j < P; ++j) {
                float v = rg[s][g][j];
                if constexpr (!LAST) {
                    const float from_r = (j == P - 1) ? right_in : qn0[g][j + 1];
                    const float from_l = (j == 0) ? left_in : qn2[g][j - 1];
                    v += (qn1[g][j] + from_r) + from_l;
                }
                a_t[j] = (kin[j] && gok[g]) ? v : 0.0f;
            }
            const int64_t go = gc[g] * plane;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                float am = a_t[j];
                if constexpr (MERGE) {
                    am = a_t[j] * msc[g];  // the adjoint of the merged output
                    dm[g] = __builtin_fmaf(a_t[j], rl[s][g][j] * rx[s][g][j], dm[g]);
                }
                if (kin[j] && gok[g]) {
                    st_once<T, NT>(dlp + go + lo + k0 + j, am * rx[s][g][j]);
                    st_once<T, NT>(dxp + go + lo + k0 + j, am * rl[s][g][j]);
                }
#pragma unroll
                for (int o = 0; o < 3; ++o) dw[j][o] += am * rh[s][g][j + o];  // h_{t-1}[k+o-1]
                qn0[g][j] = first ? 0.0f : w[0][j] * a_t[j];
                qn1[g][j] = first ? 0.0f : w[1][j] * a_t[j];
                qn2[g][j] = first ? 0.0f : w[2][j] * a_t[j];
            }
        }
        // logit gradient of this line (none on a chunk's first line).  For
        // shared logits only the channel sums of dw_{-1} - dw_0 and
        // dw_{+1} - dw_0 leave the workgroup: the normalisation's Jacobian
        // ignores a common shift of the dw, and it is the same for every
        // channel, so it is applied once to the sums afterwards.
        if (a.shared) {
            if (!first) {
                float* dzs = static_cast<float*>(a.dz) + nidx * 3 * plane;
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    if (kin[j]) {
                        atomicAdd(dzs + lo + k0 + j, dw[j][0] - dw[j][1]);
                        atomicAdd(dzs + plane + lo + k0 + j, dw[j][2] - dw[j][1]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < P; ++j) {
                float dz[3] = {0.0f, 0.0f, 0.0f};
                if (!first) {
                    const float dot = (dw[j][0] * w[0][j] + dw[j][1] * w[1][j]) + dw[j][2] * w[2][j];
#pragma unroll
                    for (int o = 0; o < 3; ++o) dz[o] = w[o][j] * (1.0f - sg[o][j]) * (dw[j][o] - dot);
                    if (k0 + j == 0) dz[0] = 0.0f;
                    if (k0 + j + 1 >= L) dz[2] = 0.0f;
                    if (L == 1) dz[1] = 0.0f;  // a single neighbour: w = [1] whatever its logit
                }
                if (kin[j]) {
                    T* dzp = static_cast<T*>(a.dz) + zplane;
#pragma unroll
                    for (int o = 0; o < 3; ++o) st_once<T, NT>(dzp + o * plane + lo + k0 + j, dz[o]);
                }
            }
        }
        fill(slot, t - D);
        buf ^= 1;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            edge(buf, 0, g, tid) = qn0[g][0];
            edge(buf, 1, g, tid) = qn2[g][P - 1];
        }
        __syncthreads();
    };

    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        (fill(IC<Ss>{}, t1 - 1 - Ss), ...);
    }(std::make_integer_sequence<int, D>{});
    step(IC<0>{}, IC<1>{}, t1 - 1);
    int t = t1 - 2;
    for (; t - (D - 1) >= t0; t -= D) {
        [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
            (step(IC<(Ss + 1) % D>{}, IC<0>{}, t - Ss), ...);
        }(std::make_integer_sequence<int, D>{});
    }
    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        ((t - Ss >= t0 ? step(IC<(Ss + 1) % D>{}, IC<0>{}, t - Ss) : void()), ...);
    }(std::make_integer_sequence<int, D - 1>{});

    if (MERGE && a.dmerge) {
        // sum over the wave, one atomic add per wave and member
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float v = dm[g];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
            if ((tid & 63) == 0 && gok[g]) atomicAdd(a.dmerge + c0 + g, v);
        }
    }
}

template <typename T, int P, int G, bool MERGE, bool NT>
__global__ __launch_bounds__(1024) void adj4_kernel(const Adj4K a) {
    extern __shared__ float s_edge_raw[];
    int dir = 0;
    int64_t idx = blockIdx.x;
    while (dir < 3 && idx >= a.blocks[dir]) {
        idx -= a.blocks[dir];
        ++dir;
    }
    const AdjK& k = a.d[dir];
    const int64_t pg = idx / k.nchunks;
    const int q = static_cast<int>(idx - pg * k.nchunks);
    adj_line<T, P, G, MERGE, NT>(k, pg, q, s_edge_raw);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) p[e] = 0.0f;
}

// Shared logits: dlogits from the channel sums e_{-1} = sum (dw_{-1} - dw_0)
// and e_{+1} = sum (dw_{+1} - dw_0) that the adjoints left in planes 0 and 1
// of src ([n][3][S][L] fp32; plane 2 unused).  With the shared weights w and
// sigmoids s of the position, dz_q = w_q (1 - s_q) (e_q - sum_o w_o e_o),
// e_0 = 0: the same value as summing each channel's dz, since that Jacobian
// is linear, equal for all channels and blind to a common shift of the dw
// (the w sum to 1).  One thread per position of the n * S * L.
template <typename T>
__global__ __launch_bounds__(256) void finish_shared_dz_kernel(const float* __restrict__ src,
                                                               const T* __restrict__ z, T* __restrict__ dz,
                                                               int64_t n, int S, int L) {
    const int64_t plane = static_cast<int64_t>(S) * L;
    const int64_t total = n * plane;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t img = e / plane;
        const int64_t r = e - img * plane;
        const int k = static_cast<int>(r % L);
        const int64_t base = img * 3 * plane + r;
        const bool has_l = k > 0;
        const bool has_r = k + 1 < L;
        const float s0 = has_l ? sigmoid(Store<T>::ld(z + base)) : 0.0f;
        const float s1 = sigmoid(Store<T>::ld(z + base + plane));
        const float s2 = has_r ? sigmoid(Store<T>::ld(z + base + 2 * plane)) : 0.0f;
        const float rr = recip((s0 + s1) + s2);
        const float w0 = s0 * rr, w1 = s1 * rr, w2 = s2 * rr;
        const float e0 = src[base], e2 = src[base + plane];
        const float dot = w0 * e0 + w2 * e2;
        float d0 = w0 * (1.0f - s0) * (e0 - dot);
        float d1 = w1 * (1.0f - s1) * (0.0f - dot);
        float d2 = w2 * (1.0f - s2) * (e2 - dot);
        if (!has_l) d0 = 0.0f;
        if (!has_r) d2 = 0.0f;
        if (L == 1) d1 = 0.0f;  // a single neighbour: w = [1] whatever its logit
        Store<T>::st(dz + base, d0);
        Store<T>::st(dz + base + plane, d1);
        Store<T>::st(dz + base + 2 * plane, d2);
    }
}

unsigned grid_for(int64_t total) {
    int64_t b = (total + 255) / 256;
    if (b > 256 * 64) b = 256 * 64;
    if (b < 1) b = 1;
    return static_cast<unsigned>(b);
}

}  // namespace

hipError_t launch_adjoint4(const AdjointParams (&p)[4], hipStream_t stream) {
    Adj4K k;
    int maxL = 1;
    int64_t total = 0;
    const bool shared = p[0].shared != 0;
    bool merge = false;
    for (int d = 0; d < 4; ++d) {
        maxL = p[d].L > maxL ? static_cast<int>(p[d].L) : maxL;
        merge = merge || p[d].mscale || p[d].dmerge;
    }
    const int P = maxL <= 1024 ? 1 : 2;  // lines of at most 2048 positions
    const int G = !shared ? 1 : (P == 1 ? shared_group<1>() : shared_group<2>());
    for (int d = 0; d < 4; ++d) {
        AdjK& a = k.d[d];
        a.x = p[d].x;
        a.g = p[d].g;
        a.lam = p[d].lam;
        a.z = p[d].logits;
        a.hs = static_cast<const float*>(p[d].hs);
        a.dlam = p[d].dlam;
        a.dz = p[d].dz;
        a.dx = p[d].dx;
        a.c = p[d].c;
        a.cw = p[d].cw;
        a.S = static_cast<int>(p[d].S);
        a.L = static_cast<int>(p[d].L);
        a.K = static_cast<int>(p[d].chunk);
        a.nchunks = static_cast<int>((p[d].S + p[d].chunk - 1) / p[d].chunk);
        a.reverse = p[d].reverse;
        a.shared = p[d].shared;
        a.mscale = p[d].mscale;
        a.dmerge = p[d].dmerge;
        k.blocks[d] = p[d].n * ((p[d].c + G - 1) / G) * a.nchunks;
        total += k.blocks[d];
    }
    const int lanes = ((maxL + P - 1) / P + 63) / 64 * 64;
    const size_t lds = 4 * sizeof(float) * static_cast<size_t>(G) * static_cast<size_t>(lanes);
    const dim3 grid(static_cast<unsigned>(total));
    const bool f32 = p[0].dtype == kF32;
    // non-temporal streams only when every line is a whole number of cache lines
    bool nt = true;
    for (int d = 0; d < 4; ++d) nt = nt && (p[d].L * (f32 ? 4 : 2)) % 128 == 0;
#define GSPN_ADJ_LAUNCH(PP, GG, MM)                                                                               \
    do {                                                                                                          \
        if (f32) {                                                                                                \
            if (nt) hipLaunchKernelGGL((adj4_kernel<float, PP, GG, MM, true>), grid, dim3(lanes), lds, stream, k);  \
            else hipLaunchKernelGGL((adj4_kernel<float, PP, GG, MM, false>), grid, dim3(lanes), lds, stream, k);    \
        } else {                                                                                                  \
            if (nt) hipLaunchKernelGGL((adj4_kernel<bf16_t, PP, GG, MM, true>), grid, dim3(lanes), lds, stream, k); \
            else hipLaunchKernelGGL((adj4_kernel<bf16_t, PP, GG, MM, false>), grid, dim3(lanes), lds, stream, k);   \
        }                                                                                                         \
    } while (0)
#define GSPN_ADJ_LAUNCH_P(PP, MM)                                                                                 \
    do {                                                                                                          \
        if (shared) GSPN_ADJ_LAUNCH(PP, shared_group<PP>(), MM);                                                  \
        else GSPN_ADJ_LAUNCH(PP, 1, MM);                                                                          \
    } while (0)
    if (P == 1) {
        if (merge) GSPN_ADJ_LAUNCH_P(1, true);
        else GSPN_ADJ_LAUNCH_P(1, false);
    } else {
        if (merge) GSPN_ADJ_LAUNCH_P(2, true);
        else GSPN_ADJ_LAUNCH_P(2, false);
    }
#undef GSPN_ADJ_LAUNCH_P
#undef GSPN_ADJ_LAUNCH
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_finish_shared_dz(const float* sums, const void* logits, void* dlogits, int64_t n, int64_t S,
                                   int64_t L, int dtype, hipStream_t stream) {
    const unsigned grid = grid_for(n * S * L);
    if (dtype == kF32) {
        hipLaunchKernelGGL(finish_shared_dz_kernel<float>, dim3(grid), dim3(256), 0, stream, sums,
                           static_cast<const float*>(logits), static_cast<float*>(dlogits), n, static_cast<int>(S),
                           static_cast<int>(L));
    } else {
        hipLaunchKernelGGL(finish_shared_dz_kernel<bf16_t>, dim3(grid), dim3(256), 0, stream, sums,
                           static_cast<const bf16_t*>(logits), static_cast<bf16_t*>(dlogits), n,
                           static_cast<int>(S), static_cast<int>(L));
    }
    return hipGetLastError();
}

}  // namespace gspn
