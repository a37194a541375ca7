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

// steps in flight in the banded adjoint: its workgroups of four waves run
// one a CU, so the registers a deeper ring takes cost no occupancy
#ifndef GSPN_ADJ_BAND_DEPTH
#define GSPN_ADJ_BAND_DEPTH 8
#endif
template <int P, int G>
constexpr int adj_band_depth() { return GSPN_ADJ_BAND_DEPTH * 2 / (P * G) > 1 ? GSPN_ADJ_BAND_DEPTH * 2 / (P * G) : 2; }

// channels one banded workgroup runs together for channel-shared logits
// (their logit gradient summed in registers before its atomic adds).  One:
// groups of 2 and 4 halve and quarter the workgroups and the steps in
// flight, and measured slower (proxy-space adjoint 2.18 and 3.16 ms against
// 1.85) for all the atomics they save.
#ifndef GSPN_ADJ_BAND_G
#define GSPN_ADJ_BAND_G 1
#endif

// channels per workgroup for channel-shared logits (fewer for two positions
// per lane: register budget).  A 1024-lane workgroup leaves 128 registers a
// lane.  Without merge weights groups of three fit them (four spill 8 bytes
// a lane): wide adjoint 13.7-13.8 ms against 14.8-15.4 for four and 15.9-16.0
// for two.  With the learnable merge's extra state three spill 20 bytes and
// four 68, so groups of two (16.1-16.2 ms, against 16.9-17.0 for three and
// 21.2-21.5 for four).
#ifndef GSPN_ADJ_G1
#define GSPN_ADJ_G1 3
#endif
#ifndef GSPN_ADJ_G1_MERGE
#define GSPN_ADJ_G1_MERGE 2
#endif
#ifndef GSPN_ADJ_G2
#define GSPN_ADJ_G2 2
#endif
#ifndef GSPN_ADJ_P
#define GSPN_ADJ_P 1
#endif
template <int P, bool MERGE>
constexpr int shared_group() { return P == 1 ? (MERGE ? GSPN_ADJ_G1_MERGE : GSPN_ADJ_G1) : GSPN_ADJ_G2; }

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
    int shared;  // dz holds fp32 channel sums of weight-gradient differences (atomic adds; groups of shared_group<P, MERGE>() channels)
    const float* mscale;  // learnable merge weight of each channel for this direction ([c]), or null for 1
    float* dmerge;        // its gradient [c] (fp32 atomic adds), or null
};

struct Adj4K {
    AdjK d[4];
    int64_t blocks[4];
};

// Index code of adj_line and adj4_kernel, shared with the host replay.

// Direction and index within it of block b (consecutive ranges).
GSPN_HD void adj4_block(const Adj4K& a, int64_t b, int& dir, int64_t& idx) {
    dir = 0;
    idx = b;
    while (dir < 3 && idx >= a.blocks[dir]) {
        idx -= a.blocks[dir];
        ++dir;
    }
}

// Channel group pg of a direction: its image, first channel and plane, and
// the offset of its logits ([n][cw][3][S][L]) in elements.
struct AdjGroup {
    int64_t nidx, c0, p0, zplane;
};

GSPN_HD AdjGroup adj_group(const AdjK& a, int64_t pg, int G, int64_t plane) {
    const int64_t groups = (a.c + G - 1) / G;
    AdjGroup r;
    r.nidx = pg / groups;
    r.c0 = (pg - r.nidx * groups) * G;
    r.p0 = r.nidx * a.c + r.c0;
    r.zplane = (r.nidx * a.cw + (a.cw == 1 ? 0 : r.c0)) * 3 * plane;
    return r;
}

// Member g of the group exists; its channel offset (0 when it does not).
GSPN_HD bool adj_member_ok(const AdjK& a, int64_t c0, int g) { return c0 + g < a.c; }
GSPN_HD int adj_member(const AdjK& a, int64_t c0, int g) { return adj_member_ok(a, c0, g) ? g : 0; }

// Position k clamped into the line (addresses of lanes past its end), and
// the clamped left / right neighbours of a lane's positions k0 .. k0 + P - 1.
// Both ends clamp: a lane past the line's end would otherwise read its left
// neighbour beyond the row, and beyond the buffer on the last row of the
// last plane.
GSPN_HD int adj_clamp(int k, int L) { return k < L - 1 ? k : L - 1; }
GSPN_HD int adj_left(int k0, int L) { return adj_clamp(k0 - 1 > 0 ? k0 - 1 : 0, L); }
GSPN_HD int adj_right(int k0, int P, int L) { return adj_clamp(k0 + P, L); }

// Index of one LDS edge value: buffer b, side (0: left, 1: right), member g, lane.
GSPN_HD int adj_edge(int b, int side, int G, int g, int nt, int lane) { return ((b * 2 + side) * G + g) * nt + lane; }

// Row of step t, and the rows a fill for step t reads: step t clamped to the
// chunk's first step t0, and the step before that (h_{t-1}, clamped too).
GSPN_HD int adj_row(int t, int S, bool rev) { return rev ? S - 1 - t : t; }
struct AdjFill {
    int64_t lo, hlo;  // element offsets of the two rows
};
GSPN_HD AdjFill adj_fill(int t, int t0, int S, int L, bool rev) {
    const int tc = t > t0 ? t : t0;
    const int tp = tc - 1 > t0 ? tc - 1 : t0;
    return {static_cast<int64_t>(adj_row(tc, S, rev)) * L, static_cast<int64_t>(adj_row(tp, S, rev)) * L};
}

// A band of the banded adjoint (few, long lines): the workgroup's lanes
// cover positions r0 .. r0 + nt P - 1 of the line (its segment
// [o_lo, o_hi) plus a halo on each side) for the steps tb_lo .. tb_hi - 1.
// The products w a of the step above the band come from qin (rows o of
// qstride floats; null: the band holds the chunk's last step), those of its
// bottom step go to qout (null: none wanted).  Only the segment's own
// positions store anything.
struct AdjBand {
    int r0, o_lo, o_hi, tb_lo, tb_hi;
    int64_t qstride;  // floats between the rows o of one channel's products
    int64_t mstride;  // floats between the products of consecutive channels
    const float* qin;
    float* qout;
};

// Position k clamped into the line at both ends (band lanes may start
// before position 0).
GSPN_HD int adj_clamp2(int k, int L) { return k < 0 ? 0 : (k < L - 1 ? k : L - 1); }
// First position of an aligned group of P (k and L multiples of P, L >= P)
// clamped to the line's last group.
GSPN_HD int adj_group_start(int k, int P, int L) { return k < 0 ? 0 : (k < L - P ? k : L - P); }

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

// P (2 or 4) neighbouring positions in one load or store (VEC: the group
// starts at a multiple of P in a line whose length is one, so its address
// is aligned to the group's size).
template <typename T, int P, bool NT>
__device__ __forceinline__ void ld_vec(const T* p, float (&v)[P]) {
    static_assert(P == 2 || P == 4, "pairs or quads");
    if constexpr (sizeof(T) == 4) {
        typedef float fv __attribute__((ext_vector_type(P)));
        const fv q = NT ? __builtin_nontemporal_load(reinterpret_cast<const fv*>(p)) : *reinterpret_cast<const fv*>(p);
#pragma unroll
        for (int j = 0; j < P; ++j) v[j] = q[j];
    } else {
        typedef uint32_t uv __attribute__((ext_vector_type(P / 2)));
        const uv q = NT ? __builtin_nontemporal_load(reinterpret_cast<const uv*>(p)) : *reinterpret_cast<const uv*>(p);
#pragma unroll
        for (int j = 0; j < P; ++j) v[j] = __uint_as_float((j & 1) ? (q[j >> 1] & 0xffff0000u) : (q[j >> 1] << 16));
    }
}
template <typename T, int P, bool NT>
__device__ __forceinline__ void st_vec(T* p, const float (&v)[P]) {
    static_assert(P == 2 || P == 4, "pairs or quads");
    if constexpr (sizeof(T) == 4) {
        typedef float fv __attribute__((ext_vector_type(P)));
        fv q;
#pragma unroll
        for (int j = 0; j < P; ++j) q[j] = v[j];
        if constexpr (NT) __builtin_nontemporal_store(q, reinterpret_cast<fv*>(p));
        else *reinterpret_cast<fv*>(p) = q;
    } else {
        typedef uint32_t uv __attribute__((ext_vector_type(P / 2)));
        uv q;
#pragma unroll
        for (int j = 0; j < P / 2; ++j) q[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        if constexpr (NT) __builtin_nontemporal_store(q, reinterpret_cast<uv*>(p));
        else *reinterpret_cast<uv*>(p) = q;
    }
}

template <typename T, int P, int G, bool MERGE, bool NT, bool BAND = false, bool VEC = false>
__device__ __forceinline__ void adj_line(const AdjK& a, int64_t pg, int q, float* edge_raw,
                                         const AdjBand& bd = AdjBand{}) {
    static_assert(!VEC || (BAND && (P == 2 || P == 4)), "pairs or quads of positions in the banded adjoint");
    constexpr int D = BAND ? adj_band_depth<P, G>() : adj_depth<P, G>();
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int S = a.S;
    const int L = a.L;
    const int64_t plane = static_cast<int64_t>(S) * L;
    const AdjGroup grp = adj_group(a, pg, G, plane);
    const int64_t nidx = grp.nidx;
    const int64_t c0 = grp.c0;  // first channel of the group
    const int64_t p0 = grp.p0;  // its plane
    int gc[G];                  // channel offset of each member, clamped
    bool gok[G];
    float msc[G];               // merge weight of each member (MERGE)
    float dm[G];                // this lane's share of dL/dm (MERGE)
#pragma unroll
    for (int g = 0; g < G; ++g) {
        gok[g] = adj_member_ok(a, c0, g);
        gc[g] = adj_member(a, c0, g);
        msc[g] = (MERGE && a.mscale) ? a.mscale[c0 + gc[g]] : 1.0f;
        dm[g] = 0.0f;
    }
    const T* xp = static_cast<const T*>(a.x) + p0 * plane;
    const T* gp = static_cast<const T*>(a.g) + p0 * plane;
    const T* lp = static_cast<const T*>(a.lam) + p0 * plane;
    const float* hp = a.hs + p0 * plane;
    const int64_t zplane = grp.zplane;
    const T* zp = static_cast<const T*>(a.z) + zplane;
    T* dlp = static_cast<T*>(a.dlam) + p0 * plane;
    T* dxp = static_cast<T*>(a.dx) + p0 * plane;

    auto edge = [&](int b, int side, int g, int lane) -> float& {
        return edge_raw[adj_edge(b, side, G, g, nt, lane)];
    };

    const int k0 = (BAND ? bd.r0 : 0) + tid * P;
    int kk[P];
    bool kin[P];  // in the line
    bool own[P];  // stored by this workgroup (BAND: in its segment)
#pragma unroll
    for (int j = 0; j < P; ++j) {
        kk[j] = BAND ? adj_clamp2(k0 + j, L) : adj_clamp(k0 + j, L);
        kin[j] = (!BAND || k0 + j >= 0) && k0 + j < L;
        own[j] = BAND ? (kin[j] && k0 + j >= bd.o_lo && k0 + j < bd.o_hi) : kin[j];
    }
    // left neighbour of the first position, right one of the last (clamped)
    const int kl = BAND ? adj_clamp2(k0 - 1, L) : adj_left(k0, L);
    const int kr = BAND ? adj_clamp2(k0 + P, L) : adj_right(k0, P, L);
    // VEC: the group's first position, clamped to the line's last group
    const int kp = adj_group_start(k0, P, L);

    const int t0 = q * a.K;
    const int t1 = min(t0 + a.K, S);
    const int ttop = BAND ? bd.tb_hi : t1;  // one past this launch's first (highest) step
    const int tbot = BAND ? bd.tb_lo : t0;  // its last step
    const bool rev = a.reverse != 0;
    auto line_of = [&](int t) { return adj_row(t, S, rev); };

    // ring: per step and channel g, x, lambda and h_{t-1} at the positions
    // and their two outer neighbours; the three logits (shared by the group)
    float rg[D][G][P], rx[D][G][P], rl[D][G][P], rh[D][G][P + 2], rz[D][3][P];
    auto fill = [&](auto slot, int t) {
        constexpr int s = decltype(slot)::value;
        const AdjFill f = adj_fill(t, t0, S, L, rev);
        const int64_t lo = f.lo;
        const int64_t hlo = f.hlo;  // h_{t-1} (clamped)
        if constexpr (VEC) {
#pragma unroll
            for (int o = 0; o < 3; ++o) ld_vec<T, P, NT>(zp + o * plane + lo + kp, rz[s][o]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int64_t go = gc[g] * plane;
                ld_vec<T, P, NT>(gp + go + lo + kp, rg[s][g]);
                ld_vec<T, P, NT>(xp + go + lo + kp, rx[s][g]);
                ld_vec<T, P, NT>(lp + go + lo + kp, rl[s][g]);
                float hv[P];
                ld_vec<float, P, false>(hp + go + hlo + kp, hv);
#pragma unroll
                for (int j = 0; j < P; ++j) rh[s][g][j + 1] = hv[j];
                rh[s][g][0] = hp[go + hlo + kl];
                rh[s][g][P + 1] = hp[go + hlo + kr];
            }
            return;
        }
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
                rx[s][g][j] = ld_once<T, NT>(xp + go + lo + kk[j]);
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
            normalise_row_s(rz[s][0][j], rz[s][1][j], rz[s][2][j], has_l, has_r, sg[0][j], sg[1][j], sg[2][j],
                            w[0][j], w[1][j], w[2][j]);
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
            if constexpr (VEC) {
                // the group's positions are all the segment's, or none
                float vl[P], vd[P];
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const float m = MERGE ? a_t[j] * msc[g] : a_t[j];
                    vl[j] = m * rx[s][g][j];
                    vd[j] = m * rl[s][g][j];
                }
                if (own[0] && gok[g]) {
                    st_vec<T, P, NT>(dlp + go + lo + k0, vl);
                    st_vec<T, P, NT>(dxp + go + lo + k0, vd);
                }
            }
#pragma unroll
            for (int j = 0; j < P; ++j) {
                float am = a_t[j];
                if constexpr (MERGE) {
                    am = a_t[j] * msc[g];  // the adjoint of the merged output
                    if (!BAND || own[j]) dm[g] = __builtin_fmaf(a_t[j], rl[s][g][j] * rx[s][g][j], dm[g]);
                }
                if (!VEC && own[j] && gok[g]) {
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
                    if (own[j]) {
                        atomicAdd(dzs + lo + k0 + j, dw[j][0] - dw[j][1]);
                        atomicAdd(dzs + plane + lo + k0 + j, dw[j][2] - dw[j][1]);
                    }
                }
            }
        } else {
            float dzv[P][3];
#pragma unroll
            for (int j = 0; j < P; ++j) {
                float* dz = dzv[j];
                dz[0] = dz[1] = dz[2] = 0.0f;
                if (!first) {
                    const float dot = (dw[j][0] * w[0][j] + dw[j][1] * w[1][j]) + dw[j][2] * w[2][j];
#pragma unroll
                    for (int o = 0; o < 3; ++o) dz[o] = w[o][j] * (1.0f - sg[o][j]) * (dw[j][o] - dot);
                    if (k0 + j == 0) dz[0] = 0.0f;
                    if (k0 + j + 1 >= L) dz[2] = 0.0f;
                    if (L == 1) dz[1] = 0.0f;  // a single neighbour: w = [1] whatever its logit
                }
                if (!VEC && own[j]) {
                    T* dzp = static_cast<T*>(a.dz) + zplane;
#pragma unroll
                    for (int o = 0; o < 3; ++o) st_once<T, NT>(dzp + o * plane + lo + k0 + j, dz[o]);
                }
            }
            if constexpr (VEC) {
                if (own[0]) {
                    T* dzp = static_cast<T*>(a.dz) + zplane;
#pragma unroll
                    for (int o = 0; o < 3; ++o) {
                        float v[P];
#pragma unroll
                        for (int j = 0; j < P; ++j) v[j] = dzv[j][o];
                        st_vec<T, P, NT>(dzp + o * plane + lo + k0, v);
                    }
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
        (fill(IC<Ss>{}, ttop - 1 - Ss), ...);
    }(std::make_integer_sequence<int, D>{});
    if constexpr (BAND) {
        // the products of the step above the band (none above the chunk's
        // last step), published to the neighbours like a step's own
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float* qi = bd.qin + g * bd.mstride;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const bool have = bd.qin != nullptr && kin[j] && gok[g];
                qn0[g][j] = have ? qi[kk[j]] : 0.0f;
                qn1[g][j] = have ? qi[bd.qstride + kk[j]] : 0.0f;
                qn2[g][j] = have ? qi[2 * bd.qstride + kk[j]] : 0.0f;
            }
            edge(buf, 0, g, tid) = qn0[g][0];
            edge(buf, 1, g, tid) = qn2[g][P - 1];
        }
        __syncthreads();
        step(IC<0>{}, IC<0>{}, ttop - 1);
    } else {
        step(IC<0>{}, IC<1>{}, t1 - 1);
    }
    int t = ttop - 2;
    for (; t - (D - 1) >= tbot; t -= D) {
        [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
            (step(IC<(Ss + 1) % D>{}, IC<0>{}, t - Ss), ...);
        }(std::make_integer_sequence<int, D>{});
    }
    [&]<int... Ss>(std::integer_sequence<int, Ss...>) {
        ((t - Ss >= tbot ? step(IC<(Ss + 1) % D>{}, IC<0>{}, t - Ss) : void()), ...);
    }(std::make_integer_sequence<int, D - 1>{});
    if constexpr (BAND) {
        // the products of the band's bottom step, for the band below
        if (bd.qout) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float* qo = bd.qout + g * bd.mstride;
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    if (own[j] && gok[g]) {
                        qo[k0 + j] = qn0[g][j];
                        qo[bd.qstride + k0 + j] = qn1[g][j];
                        qo[2 * bd.qstride + k0 + j] = qn2[g][j];
                    }
                }
            }
        }
    }

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
    int dir;
    int64_t idx;
    adj4_block(a, blockIdx.x, dir, idx);
    const AdjK& k = a.d[dir];
    const int64_t pg = idx / k.nchunks;
    const int q = static_cast<int>(idx - pg * k.nchunks);
    adj_line<T, P, G, MERGE, NT>(k, pg, q, s_edge_raw);
}

// The banded adjoint: a launch per band of kAdjBandHalo steps (counted down
// from each direction's last step), one workgroup of kAdjBandThreads lanes,
// two positions each, per (direction, plane, segment); a segment is
// kAdjBandSeg positions, with a halo of kAdjBandHalo on each side.  The
// coupling M^T moves information one position per step, so what the halo's
// outer edge gets wrong (its outer neighbours taken as 0) reaches at most
// kAdjBandHalo positions inwards by the band's end: the segment stays exact.
constexpr int kAdjBandSeg = 256;
constexpr int kAdjBandHalo = 128;
constexpr int kAdjBandSpan = kAdjBandSeg + 2 * kAdjBandHalo;  // positions of a workgroup
constexpr int kAdjBandThreads = kAdjBandSpan / 2;            // lanes with two positions each (four: half)

struct Adj4BandK {
    Adj4K base;           // blocks[d]: planes * nseg[d], or 0 once the direction's scan has ended
    int nseg[4];          // segments per line of each direction
    int band;             // steps S_d - (band + 1) halo .. S_d - band halo - 1 of direction d
    int64_t planes;       // planes per direction
    int64_t lmax;         // floats per row of the product buffers
    const float* qin;     // products above the band: direction d, plane p, row o at ((d planes + p) 3 + o) lmax
    float* qout;          // those of its bottom step, same layout
};

// Band of workgroup (dir, first plane p of its channel group, segment sg)
// (shared with the host replay).
GSPN_HD AdjBand adj_band(const Adj4BandK& k, int dir, int64_t p, int sg) {
    const AdjK& a = k.base.d[dir];
    AdjBand bd;
    bd.o_lo = sg * kAdjBandSeg;
    bd.o_hi = bd.o_lo + kAdjBandSeg < a.L ? bd.o_lo + kAdjBandSeg : a.L;
    bd.r0 = bd.o_lo - kAdjBandHalo;
    bd.tb_hi = a.S - k.band * kAdjBandHalo;
    bd.tb_lo = bd.tb_hi - kAdjBandHalo > 0 ? bd.tb_hi - kAdjBandHalo : 0;
    bd.qstride = k.lmax;
    bd.mstride = 3 * k.lmax;
    const int64_t off = (static_cast<int64_t>(dir) * k.planes + p) * 3 * k.lmax;
    bd.qin = k.band == 0 ? nullptr : k.qin + off;
    bd.qout = bd.tb_lo > 0 ? k.qout + off : nullptr;
    return bd;
}

// VEC: every line's length a multiple of P and every tensor aligned to P
// elements: each lane loads and stores its P positions as one vector.
template <typename T, bool MERGE, bool NT, bool VEC, int P, int G>
__global__ __launch_bounds__(kAdjBandThreads) void adj4band_kernel(const Adj4BandK k) {
    extern __shared__ float s_edge_raw[];
    int dir;
    int64_t idx;
    adj4_block(k.base, blockIdx.x, dir, idx);
    const AdjK& a = k.base.d[dir];
    const int64_t pg = idx / k.nseg[dir];  // channel group
    const int sg = static_cast<int>(idx - pg * k.nseg[dir]);
    const int64_t plane = static_cast<int64_t>(a.S) * a.L;
    adj_line<T, P, G, MERGE, NT, true, VEC>(a, pg, 0, s_edge_raw, adj_band(k, dir, adj_group(a, pg, G, plane).p0, sg));
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
        float s0, s1, s2, w0, w1, w2;
        normalise_row_s(Store<T>::ld(z + base), Store<T>::ld(z + base + plane), Store<T>::ld(z + base + 2 * plane),
                        has_l, has_r, s0, s1, s2, w0, w1, w2);
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

#ifdef GSPN_CHECK_LAUNCHES
// Host replay of adj4_kernel: for every block and thread, each access of
// every step at the offsets adj_line computes with the functions above
// (fills for steps t0 - D .. t1 - 1, clamped as the kernel clamps them;
// stores, atomics and merge accesses for the chunk's steps), and every LDS
// edge index against the launch's dynamic LDS.
static void replay_adjoint4(const Adj4K& k, int64_t nblocks, int nt, size_t lds, int es, int P, int G, int D, bool merge) {
    const char* kn = "adj4_kernel";
    int64_t bad = 0, n = 0;
    auto fail = [&](const char* what, int64_t b, int tid, int t) {
        if (bad++ < 4) check::violation(kn, what, "block %lld thread %d step %d", static_cast<long long>(b), tid, t);
    };
    check::Region rx[4], rg[4], rl[4], rz[4], rh[4], rdl[4], rdz[4], rdx[4], rms[4], rdm[4];
    for (int d = 0; d < 4; ++d) {
        const AdjK& a = k.d[d];
        rx[d] = check::region_of(a.x, kn, "x");
        rg[d] = check::region_of(a.g, kn, "dL/dy");
        rl[d] = check::region_of(a.lam, kn, "lambda");
        rz[d] = check::region_of(a.z, kn, "logits");
        rh[d] = check::region_of(a.hs, kn, "states");
        rdl[d] = check::region_of(a.dlam, kn, "dlambda");
        rdz[d] = check::region_of(a.dz, kn, "dlogits");
        rdx[d] = check::region_of(a.dx, kn, "dx");
        if (merge && a.mscale) rms[d] = check::region_of(a.mscale, kn, "merge");
        if (merge && a.dmerge) rdm[d] = check::region_of(a.dmerge, kn, "dmerge");
    }
    for (int b = 0; b < 2; ++b)
        for (int side = 0; side < 2; ++side)
            for (int g = 0; g < G; ++g)
                for (int lane = 0; lane < nt; ++lane)
                    if (static_cast<size_t>(adj_edge(b, side, G, g, nt, lane) + 1) * 4 > lds) fail("edge LDS", -1, lane, -1);
    for (int64_t b = 0; b < nblocks; ++b) {
        int dir;
        int64_t idx;
        adj4_block(k, b, dir, idx);
        const AdjK& a = k.d[dir];
        const int64_t pg = idx / a.nchunks;
        const int q = static_cast<int>(idx - pg * a.nchunks);
        const int S = a.S, L = a.L;
        const int64_t plane = static_cast<int64_t>(S) * L;
        const AdjGroup grp = adj_group(a, pg, G, plane);
        const int t0 = q * a.K;
        const int t1 = (t0 + a.K < S) ? t0 + a.K : S;
        const bool rev = a.reverse != 0;
        const int64_t pe = grp.p0 * plane * es;  // bytes to the group's first plane
        const char* zb = static_cast<const char*>(a.z) + grp.zplane * es;
        const float* hb = a.hs + grp.p0 * plane;
        for (int g = 0; g < G; ++g) {
            const bool ok = adj_member_ok(a, grp.c0, g);
            const int64_t c = grp.c0 + adj_member(a, grp.c0, g);
            if (merge && a.mscale && !check::in_region(rms[dir], a.mscale, c * 4, 4)) fail("merge weight", b, -1, -1);
            if (merge && a.dmerge && ok && !check::in_region(rdm[dir], a.dmerge, (grp.c0 + g) * 4, 4))
                fail("dmerge", b, -1, -1);
        }
        for (int tid = 0; tid < nt; ++tid) {
            const int k0 = tid * P;
            const int kl = adj_left(k0, L), kr = adj_right(k0, P, L);
            for (int t = t0 - D; t < t1; ++t) {
                const AdjFill f = adj_fill(t, t0, S, L, rev);
                for (int j = 0; j < P; ++j) {
                    const int kk = adj_clamp(k0 + j, L);
                    for (int o = 0; o < 3; ++o)
                        if (!check::in_region(rz[dir], zb, (o * plane + f.lo + kk) * es, es)) fail("logit load", b, tid, t);
                    for (int g = 0; g < G; ++g) {
                        const int64_t go = adj_member(a, grp.c0, g) * plane;
                        const int64_t e = (go + f.lo + kk) * es;
                        if (!check::in_region(rg[dir], a.g, pe + e, es)) fail("dL/dy load", b, tid, t);
                        if (!check::in_region(rx[dir], a.x, pe + e, es)) fail("x load", b, tid, t);
                        if (!check::in_region(rl[dir], a.lam, pe + e, es)) fail("lambda load", b, tid, t);
                        if (!check::in_region(rh[dir], hb, (go + f.hlo + kk) * 4, 4)) fail("state load", b, tid, t);
                    }
                }
                for (int g = 0; g < G; ++g) {
                    const int64_t go = adj_member(a, grp.c0, g) * plane;
                    if (!check::in_region(rh[dir], hb, (go + f.hlo + kl) * 4, 4)) fail("left state", b, tid, t);
                    if (!check::in_region(rh[dir], hb, (go + f.hlo + kr) * 4, 4)) fail("right state", b, tid, t);
                }
                n += P * (3 + 4 * G) + 2 * G;
                if (t < t0) continue;
                // the step's stores
                const int64_t lo = static_cast<int64_t>(adj_row(t, S, rev)) * L;
                for (int j = 0; j < P; ++j) {
                    if (k0 + j >= L) continue;
                    for (int g = 0; g < G; ++g) {
                        if (!adj_member_ok(a, grp.c0, g)) continue;
                        const int64_t e = (adj_member(a, grp.c0, g) * plane + lo + k0 + j) * es;
                        if (!check::in_region(rdl[dir], a.dlam, pe + e, es)) fail("dlambda store", b, tid, t);
                        if (!check::in_region(rdx[dir], a.dx, pe + e, es)) fail("dx store", b, tid, t);
                    }
                    if (a.shared) {
                        if (t != t0) {
                            const int64_t e = (grp.nidx * 3 * plane + lo + k0 + j) * 4;
                            if (!check::in_region(rdz[dir], a.dz, e, 4) || !check::in_region(rdz[dir], a.dz, e + plane * 4, 4))
                                fail("dlogit sum atomic", b, tid, t);
                        }
                    } else {
                        for (int o = 0; o < 3; ++o)
                            if (!check::in_region(rdz[dir], a.dz, (grp.zplane + o * plane + lo + k0 + j) * es, es))
                                fail("dlogit store", b, tid, t);
                    }
                    n += 2 * G + 3;
                }
            }
        }
    }
    if (bad) check::violation(kn, "accesses", "%lld bad", static_cast<long long>(bad));
    check::count_accesses(n);
    check::replayed(kn, 1024, 0);
}

static void replay_adjoint4_band(const Adj4BandK& k, int64_t nblocks, int es, bool merge, bool vec, int P, int G) {
    const char* kn = "adj4band_kernel";
    const int D = G == 1 ? adj_band_depth<2, 1>() : adj_band_depth<2, GSPN_ADJ_BAND_G>();
    const int nt = kAdjBandSpan / P;
    int64_t bad = 0, n = 0;
    auto fail = [&](const char* what, int64_t b, int tid, int t) {
        if (bad++ < 4) check::violation(kn, what, "block %lld thread %d step %d", static_cast<long long>(b), tid, t);
    };
    check::Region rx[4], rg[4], rl[4], rz[4], rh[4], rdl[4], rdz[4], rdx[4], rms[4], rdm[4];
    for (int d = 0; d < 4; ++d) {
        const AdjK& a = k.base.d[d];
        rx[d] = check::region_of(a.x, kn, "x");
        rg[d] = check::region_of(a.g, kn, "dL/dy");
        rl[d] = check::region_of(a.lam, kn, "lambda");
        rz[d] = check::region_of(a.z, kn, "logits");
        rh[d] = check::region_of(a.hs, kn, "states");
        rdl[d] = check::region_of(a.dlam, kn, "dlambda");
        rdz[d] = check::region_of(a.dz, kn, "dlogits");
        rdx[d] = check::region_of(a.dx, kn, "dx");
        if (merge && a.mscale) rms[d] = check::region_of(a.mscale, kn, "merge");
        if (merge && a.dmerge) rdm[d] = check::region_of(a.dmerge, kn, "dmerge");
    }
    const check::Region rqi = check::region_of(k.qin, kn, "band products in");
    const check::Region rqo = check::region_of(k.qout, kn, "band products out");
    for (int64_t b = 0; b < nblocks; ++b) {
        int dir;
        int64_t idx;
        adj4_block(k.base, b, dir, idx);
        const AdjK& a = k.base.d[dir];
        const int64_t pg = idx / k.nseg[dir];
        const int sg = static_cast<int>(idx - pg * k.nseg[dir]);
        const int S = a.S, L = a.L;
        const int64_t plane = static_cast<int64_t>(S) * L;
        const AdjGroup grp = adj_group(a, pg, G, plane);
        const AdjBand bd = adj_band(k, dir, grp.p0, sg);
        const bool rev = a.reverse != 0;
        const int64_t pe = grp.p0 * plane * es;
        const char* zb = static_cast<const char*>(a.z) + grp.zplane * es;
        const float* hb = a.hs + grp.p0 * plane;
        if (a.nchunks != 1 || bd.tb_lo >= bd.tb_hi) fail("band steps", b, -1, -1);
        for (int g = 0; g < G; ++g) {
            const bool ok = adj_member_ok(a, grp.c0, g);
            const int64_t c = grp.c0 + adj_member(a, grp.c0, g);
            if (merge && a.mscale && !check::in_region(rms[dir], a.mscale, c * 4, 4)) fail("merge weight", b, -1, -1);
            if (merge && a.dmerge && ok && !check::in_region(rdm[dir], a.dmerge, (grp.c0 + g) * 4, 4))
                fail("dmerge", b, -1, -1);
        }
        for (int tid = 0; tid < nt; ++tid) {
            const int k0 = bd.r0 + tid * P;
            const int kl = adj_clamp2(k0 - 1, L), kr = adj_clamp2(k0 + P, L);
            for (int g = 0; g < G; ++g) {
                if (!adj_member_ok(a, grp.c0, g)) continue;
                for (int j = 0; j < P; ++j) {
                    const int kk = adj_clamp2(k0 + j, L);
                    const bool kin = k0 + j >= 0 && k0 + j < L;
                    const bool own = kin && k0 + j >= bd.o_lo && k0 + j < bd.o_hi;
                    for (int o = 0; o < 3; ++o) {
                        if (bd.qin && kin &&
                            !check::in_region(rqi, bd.qin, (g * bd.mstride + o * bd.qstride + kk) * 4, 4))
                            fail("band products load", b, tid, -1);
                        if (bd.qout && own &&
                            !check::in_region(rqo, bd.qout, (g * bd.mstride + o * bd.qstride + k0 + j) * 4, 4))
                            fail("band products store", b, tid, -1);
                    }
                }
            }
            const int kp = adj_group_start(k0, P, L);
            if (vec && (k0 % P != 0 || L % P != 0)) fail("group alignment", b, tid, -1);
            for (int t = bd.tb_lo - D; t < bd.tb_hi; ++t) {
                const AdjFill f = adj_fill(t, 0, S, L, rev);
                for (int j = 0; j < P; ++j) {
                    const int kk = vec ? kp + j : adj_clamp2(k0 + j, L);
                    for (int o = 0; o < 3; ++o)
                        if (!check::in_region(rz[dir], zb, (o * plane + f.lo + kk) * es, es)) fail("logit load", b, tid, t);
                    for (int g = 0; g < G; ++g) {
                        const int64_t go = adj_member(a, grp.c0, g) * plane;
                        const int64_t e = (go + f.lo + kk) * es;
                        if (!check::in_region(rg[dir], a.g, pe + e, es)) fail("dL/dy load", b, tid, t);
                        if (!check::in_region(rx[dir], a.x, pe + e, es)) fail("x load", b, tid, t);
                        if (!check::in_region(rl[dir], a.lam, pe + e, es)) fail("lambda load", b, tid, t);
                        if (!check::in_region(rh[dir], hb, (go + f.hlo + kk) * 4, 4)) fail("state load", b, tid, t);
                    }
                }
                for (int g = 0; g < G; ++g) {
                    const int64_t go = adj_member(a, grp.c0, g) * plane;
                    if (!check::in_region(rh[dir], hb, (go + f.hlo + kl) * 4, 4)) fail("left state", b, tid, t);
                    if (!check::in_region(rh[dir], hb, (go + f.hlo + kr) * 4, 4)) fail("right state", b, tid, t);
                }
                n += P * (3 + 4 * G) + 2 * G;
                if (t < bd.tb_lo) continue;
                const int64_t lo = static_cast<int64_t>(adj_row(t, S, rev)) * L;
                for (int j = 0; j < P; ++j) {
                    const bool own = k0 + j >= 0 && k0 + j < L && k0 + j >= bd.o_lo && k0 + j < bd.o_hi;
                    if (!own) continue;
                    for (int g = 0; g < G; ++g) {
                        if (!adj_member_ok(a, grp.c0, g)) continue;
                        const int64_t e = (adj_member(a, grp.c0, g) * plane + lo + k0 + j) * es;
                        if (!check::in_region(rdl[dir], a.dlam, pe + e, es)) fail("dlambda store", b, tid, t);
                        if (!check::in_region(rdx[dir], a.dx, pe + e, es)) fail("dx store", b, tid, t);
                    }
                    if (a.shared) {
                        if (t != 0) {
                            const int64_t ez = (grp.nidx * 3 * plane + lo + k0 + j) * 4;
                            if (!check::in_region(rdz[dir], a.dz, ez, 4) ||
                                !check::in_region(rdz[dir], a.dz, ez + plane * 4, 4))
                                fail("dlogit sum atomic", b, tid, t);
                        }
                    } else {
                        for (int o = 0; o < 3; ++o)
                            if (!check::in_region(rdz[dir], a.dz, (grp.zplane + o * plane + lo + k0 + j) * es, es))
                                fail("dlogit store", b, tid, t);
                    }
                    n += 2 * G + 3;
                }
            }
        }
    }
    if (bad) check::violation(kn, "accesses", "%lld bad", static_cast<long long>(bad));
    check::count_accesses(n);
    check::replayed(kn, nt, 0);
}

static void replay_elementwise(const char* kn, const char* what, const void* base, int64_t first, int64_t end, int es) {
    const check::Region r = check::region_of(base, kn, what);
    if (end > first && (!check::in_region(r, base, first * es, es) || !check::in_region(r, base, (end - 1) * es, es)))
        check::violation(kn, what, "elements [%lld, %lld) outside the buffer", static_cast<long long>(first),
                         static_cast<long long>(end));
    check::count_accesses(end - first);
}
#endif

namespace {

AdjK adj_args(const AdjointParams& p) {
    AdjK a;
    a.x = p.x;
    a.g = p.g;
    a.lam = p.lam;
    a.z = p.logits;
    a.hs = static_cast<const float*>(p.hs);
    a.dlam = p.dlam;
    a.dz = p.dz;
    a.dx = p.dx;
    a.c = p.c;
    a.cw = p.cw;
    a.S = static_cast<int>(p.S);
    a.L = static_cast<int>(p.L);
    a.K = static_cast<int>(p.chunk);
    a.nchunks = static_cast<int>((p.S + p.chunk - 1) / p.chunk);
    a.reverse = p.reverse;
    a.shared = p.shared;
    a.mscale = p.mscale;
    a.dmerge = p.dmerge;
    return a;
}

constexpr int64_t kAdjBandMaxLines = 64;  // lines (planes x 4 directions) below which bands pay

}  // namespace

bool adjoint_band_shape(int64_t planes, int64_t h, int64_t w) {
    return planes * 4 <= kAdjBandMaxLines && h >= 2 * kAdjBandThreads && w >= 2 * kAdjBandThreads;
}

int64_t adjoint_band_floats(int64_t planes, int64_t lmax) { return 2 * 4 * 3 * planes * lmax; }

int adjoint_band_launches(const AdjointParams (&p)[4]) {
    int64_t smax = 0;
    for (int d = 0; d < 4; ++d) {
        if (p[d].chunk < p[d].S) return 0;  // chunked lines run in parallel already
        smax = p[d].S > smax ? p[d].S : smax;
    }
    // p[0] is vertical (S = h, L = w), p[2] horizontal (S = w, L = h)
    if (!adjoint_band_shape(p[0].n * p[0].c, p[0].S, p[0].L)) return 0;
    return static_cast<int>((smax + kAdjBandHalo - 1) / kAdjBandHalo);
}

hipError_t launch_adjoint4_band(const AdjointParams (&p)[4], float* qbuf, int band, hipStream_t stream) {
    Adj4BandK k;
    const int64_t planes = p[0].n * p[0].c;
    int64_t lmax = 1, total = 0;
    bool merge = false;
    for (int d = 0; d < 4; ++d) {
        lmax = p[d].L > lmax ? p[d].L : lmax;
        merge = merge || p[d].mscale || p[d].dmerge;
    }
    const int G = p[0].shared ? GSPN_ADJ_BAND_G : 1;
    const int64_t groups = p[0].n * ((p[0].c + G - 1) / G);
    for (int d = 0; d < 4; ++d) {
        k.base.d[d] = adj_args(p[d]);
        k.nseg[d] = static_cast<int>((p[d].L + kAdjBandSeg - 1) / kAdjBandSeg);
        k.base.blocks[d] = p[d].S - static_cast<int64_t>(band) * kAdjBandHalo > 0 ? groups * k.nseg[d] : 0;
        total += k.base.blocks[d];
    }
    k.band = band;
    k.planes = planes;
    k.lmax = lmax;
    k.qin = qbuf + (band & 1) * 4 * planes * 3 * lmax;
    k.qout = qbuf + ((band + 1) & 1) * 4 * planes * 3 * lmax;
    const bool f32 = p[0].dtype == kF32;
    bool nt = true;
    for (int d = 0; d < 4; ++d) nt = nt && (p[d].L * (f32 ? 4 : 2)) % 128 == 0;
    const dim3 grid(static_cast<unsigned>(total));
    // groups of P positions a lane: lines whose lengths are multiples of P,
    // every tensor aligned to P elements (quads, else pairs, else one
    // position at a time, two a lane)
    auto vec_ok = [&](int P) {
        const size_t al = static_cast<size_t>(P) * (f32 ? 4 : 2);
        bool ok = true;
        for (int d = 0; d < 4; ++d) {
            const AdjointParams& q = p[d];
            ok = ok && q.L % P == 0 && q.L >= P && reinterpret_cast<uintptr_t>(q.x) % al == 0 &&
                 reinterpret_cast<uintptr_t>(q.g) % al == 0 && reinterpret_cast<uintptr_t>(q.lam) % al == 0 &&
                 reinterpret_cast<uintptr_t>(q.logits) % al == 0 && reinterpret_cast<uintptr_t>(q.dlam) % al == 0 &&
                 reinterpret_cast<uintptr_t>(q.dx) % al == 0 && reinterpret_cast<uintptr_t>(q.hs) % (4 * P) == 0 &&
                 (q.shared || reinterpret_cast<uintptr_t>(q.dz) % al == 0);
        }
        return ok;
    };
    // (quads on workgroups of half the lanes measured slower: the proxy
    // backward's adjoint 3.9 against 1.9 ms)
    const int P = 2;
    const bool vec = vec_ok(2);
    const int threads = kAdjBandSpan / P;
    const size_t lds = 4 * sizeof(float) * threads * G;
#ifdef GSPN_CHECK_LAUNCHES
    replay_adjoint4_band(k, total, f32 ? 4 : 2, merge, vec, P, G);
#endif
#define GSPN_ADJB_LAUNCH3(TT, MM, VV, GG)                                                                           \
    do {                                                                                                            \
        if (nt) hipLaunchKernelGGL((adj4band_kernel<TT, MM, true, VV, 2, GG>), grid, dim3(threads), lds, stream, k); \
        else hipLaunchKernelGGL((adj4band_kernel<TT, MM, false, VV, 2, GG>), grid, dim3(threads), lds, stream, k);   \
    } while (0)
#define GSPN_ADJB_LAUNCH2(TT, MM, VV)                         \
    do {                                                      \
        if (G > 1) GSPN_ADJB_LAUNCH3(TT, MM, VV, GSPN_ADJ_BAND_G); \
        else GSPN_ADJB_LAUNCH3(TT, MM, VV, 1);                    \
    } while (0)
#define GSPN_ADJB_LAUNCH(TT, MM)                  \
    do {                                          \
        if (vec) GSPN_ADJB_LAUNCH2(TT, MM, true);    \
        else GSPN_ADJB_LAUNCH2(TT, MM, false);       \
    } while (0)
    if (f32) {
        if (merge) GSPN_ADJB_LAUNCH(float, true);
        else GSPN_ADJB_LAUNCH(float, false);
    } else {
        if (merge) GSPN_ADJB_LAUNCH(bf16_t, true);
        else GSPN_ADJB_LAUNCH(bf16_t, false);
    }
#undef GSPN_ADJB_LAUNCH
#undef GSPN_ADJB_LAUNCH2
#undef GSPN_ADJB_LAUNCH3
    return hipGetLastError();
}

hipError_t launch_adjoint4(const AdjointParams (&p)[4], hipStream_t stream, AdjointPlan* plan) {
    Adj4K k;
    int maxL = 1;
    int64_t total = 0;
    const bool shared = p[0].shared != 0;
    bool merge = false;
    for (int d = 0; d < 4; ++d) {
        maxL = p[d].L > maxL ? static_cast<int>(p[d].L) : maxL;
        merge = merge || p[d].mscale || p[d].dmerge;
    }
    const int P = maxL <= 1024 ? (shared ? GSPN_ADJ_P : 1) : 2;  // lines of at most 2048 positions
    const int G = !shared ? 1
                  : P == 1   ? (merge ? shared_group<1, true>() : shared_group<1, false>())
                             : (merge ? shared_group<2, true>() : shared_group<2, false>());
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
    if (plan) *plan = {P, G, nt ? 1 : 0};
#ifdef GSPN_CHECK_LAUNCHES
    {
        const int depth = (P == 1 && G == 1) ? adj_depth<1, 1>() : adj_depth<2, 2>();
        replay_adjoint4(k, total, lanes, lds, f32 ? 4 : 2, P, G, depth, merge);
    }
#endif
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
        if (shared) GSPN_ADJ_LAUNCH(PP, (shared_group<PP, MM>()), MM);                                            \
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
#ifdef GSPN_CHECK_LAUNCHES
    // grid-stride loop over [0, n)
    replay_elementwise("fill_zero_kernel", "p", p, 0, n, 4);
    check::replayed("fill_zero_kernel", 256, 0);
#endif
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_finish_shared_dz(const float* sums, const void* logits, void* dlogits, int64_t n, int64_t S,
                                   int64_t L, int dtype, hipStream_t stream) {
    const unsigned grid = grid_for(n * S * L);
#ifdef GSPN_CHECK_LAUNCHES
    // grid-stride loop over the n * S * L positions: planes 0..2 of [n][3][S][L]
    {
        const char* kn = "finish_shared_dz_kernel";
        const int es = dtype == kF32 ? 4 : 2;
        replay_elementwise(kn, "sums", sums, 0, n * 3 * S * L - S * L, 4);
        replay_elementwise(kn, "logits", logits, 0, n * 3 * S * L, es);
        replay_elementwise(kn, "dlogits", dlogits, 0, n * 3 * S * L, es);
        check::replayed(kn, 256, 0);
    }
#endif
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
