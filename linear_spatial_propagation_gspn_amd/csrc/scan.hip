// scan.hip -- launch configuration of the line-scan kernels (the kernels and
// their launch families live in scan_kernel.hpp, instantiated per storage type
// and direction family in scan_{f32,bf16,bf16pair}_{vert,horiz}.hip and
// scan4_{f32,bf16,bf16pair}.hip).
#include "scan_band.hpp"
#include "scan_kernel.hpp"
#include "scan_lp.hpp"

namespace gspn {

extern template hipError_t launch_family<float, float, false>(const ScanConfig&, bool, bool, const ScanK&,
                                                              int64_t, int, hipStream_t);
extern template hipError_t launch_family<float, float, true>(const ScanConfig&, bool, bool, const ScanK&,
                                                             int64_t, int, hipStream_t);
extern template hipError_t launch_family<bf16_t, bf16_t, false>(const ScanConfig&, bool, bool, const ScanK&,
                                                                int64_t, int, hipStream_t);
extern template hipError_t launch_family<bf16_t, bf16_t, true>(const ScanConfig&, bool, bool, const ScanK&,
                                                               int64_t, int, hipStream_t);
extern template hipError_t launch_family<bf16_t, WPair, false>(const ScanConfig&, bool, bool, const ScanK&,
                                                               int64_t, int, hipStream_t);
extern template hipError_t launch_family<bf16_t, WPair, true>(const ScanConfig&, bool, bool, const ScanK&,
                                                              int64_t, int, hipStream_t);
extern template hipError_t launch_fused4<float, float>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4<bf16_t, bf16_t>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4<bf16_t, WPair>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4v<float, float>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4v<bf16_t, bf16_t>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4v<bf16_t, WPair>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4lp<float, float, true>(const Scan4K&, int, hipStream_t);
extern template hipError_t launch_fused4lp<float, float, false>(const Scan4K&, int, hipStream_t);
extern template hipError_t launch_fused4lp<float, float, true, float, true>(const Scan4K&, int, hipStream_t);
extern template hipError_t launch_fused4lp<float, float, false, float, true>(const Scan4K&, int, hipStream_t);
extern template hipError_t launch_fused4lp<bf16_t, bf16_t, true>(const Scan4K&, int, hipStream_t);
extern template hipError_t launch_fused4v<bf16_t, bf16_t, float>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4lp<bf16_t, bf16_t, true, float>(const Scan4K&, int, hipStream_t);
extern template hipError_t launch_fused4v<bf16_t, WPair, float>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4lp<bf16_t, WPair, false, float>(const Scan4K&, int, hipStream_t);
extern template hipError_t launch_fused4lp<bf16_t, WPair, false>(const Scan4K&, int, hipStream_t);
extern template hipError_t launch_band4<float, float, true>(const BandK&, hipStream_t);
extern template hipError_t launch_band4<float, float, false>(const BandK&, hipStream_t);
extern template hipError_t launch_band4<bf16_t, bf16_t, true>(const BandK&, hipStream_t);
extern template hipError_t launch_band4<bf16_t, WPair, false>(const BandK&, hipStream_t);
extern template hipError_t launch_band4<bf16_t, WPair, false, float>(const BandK&, hipStream_t);
extern template hipError_t launch_band4<bf16_t, bf16_t, true, float>(const BandK&, hipStream_t);

namespace {

// Positions per lane for a line of L positions: one position per lane up to
// 1024 lanes (16 waves, four per SIMD, which hides the latency of each step's
// chain better than fewer, fatter lanes), then 2 or 4 for longer lines.
ScanConfig choose_config(bool horiz, int L) {
#if defined(GSPN_VERT_P)
    if (!horiz && (L + GSPN_VERT_P - 1) / GSPN_VERT_P <= 1024) return {GSPN_VERT_P};
#endif
#if defined(GSPN_HORIZ_P)
    if (horiz && (L + GSPN_HORIZ_P - 1) / GSPN_HORIZ_P <= 1024) return {GSPN_HORIZ_P};
#endif
    (void)horiz;
    ScanConfig c{1};
    while (c.P < 4 && (L + c.P - 1) / c.P > 1024) c.P *= 2;
    return c;
}

// Horizontal tile width in steps (mirrors Blocking<T, P, true>::UT).
int horiz_tile_width(size_t esz, int P) {
    const int vw = static_cast<int>(16 / esz);
    const int u = P == 1 ? GSPN_SUB_U : (P == 2 ? GSPN_SUB_U2 : 2);
    const int t0 = (16 / P) > vw ? (16 / P) : vw;
    return t0 > u ? t0 : u;
}

bool aligned_to(const void* ptr, size_t bytes) {
    return (reinterpret_cast<uintptr_t>(ptr) % bytes) == 0;
}

bool is_horiz(int dir) { return dir == 2 || dir == 3; }

ScanK make_args(const ScanParams& p, int P) {
    const bool horiz = is_horiz(p.dir);
    const int S = static_cast<int>(horiz ? p.w : p.h);
    const int L = static_cast<int>(horiz ? p.h : p.w);
    const size_t esz = p.dtype == kF32 ? 4 : 2;
    const int vw = static_cast<int>(16 / esz);
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
    k.mscale = p.mscale;
    k.xtile = p.xtile;
    // Row tiles take 16-byte accesses when every tile of every chunk starts
    // on a 16-byte column: rows and chunk starts are whole vectors apart.
    const int ut = horiz_tile_width(esz, P);
    k.vec_tile = horiz && S % vw == 0 && (k.nchunks == 1 || k.K % vw == 0) && S >= ut &&
                 aligned_to(p.x, 16) && aligned_to(p.out, 16);
    return k;
}

int lanes_for(int L, int P) { return (((L + P - 1) / P + 63) / 64) * 64; }

}  // namespace

hipError_t launch_scan(const ScanParams& p, hipStream_t stream) {
    const bool horiz = is_horiz(p.dir);
    const bool rev = (p.dir == 1 || p.dir == 3);
    const int L = static_cast<int>(horiz ? p.h : p.w);
    const ScanConfig cfg = choose_config(horiz, L);
    const ScanK k = make_args(p, cfg.P);
    const int64_t nblocks = p.n * p.c * k.nchunks;
    const int nthreads = lanes_for(L, cfg.P);
    const bool acc = p.accumulate != 0;
    if (p.dtype == kF32) {
        return horiz ? launch_family<float, float, true>(cfg, rev, acc, k, nblocks, nthreads, stream)
                     : launch_family<float, float, false>(cfg, rev, acc, k, nblocks, nthreads, stream);
    }
    if (p.wdtype == kPairF16) {
        return horiz ? launch_family<bf16_t, WPair, true>(cfg, rev, acc, k, nblocks, nthreads, stream)
                     : launch_family<bf16_t, WPair, false>(cfg, rev, acc, k, nblocks, nthreads, stream);
    }
    return horiz ? launch_family<bf16_t, bf16_t, true>(cfg, rev, acc, k, nblocks, nthreads, stream)
                 : launch_family<bf16_t, bf16_t, false>(cfg, rev, acc, k, nblocks, nthreads, stream);
}

bool fused4_supported(int64_t h, int64_t w) { return h <= 2048 && w <= 2048; }

hipError_t launch_scan4(const ScanParams (&p)[4], hipStream_t stream) {
    const int Lv = static_cast<int>(p[0].w);
    const int Lh = static_cast<int>(p[0].h);
    const int pv = Lv > 1024 ? 2 : 1;
    const int ph = Lh > 1024 ? 2 : 1;
    Scan4K k;
    for (int d = 0; d < 4; ++d) {
        k.d[d] = make_args(p[d], is_horiz(d) ? ph : pv);
        k.blocks[d] = p[d].n * p[d].c * k.d[d].nchunks;
    }
    k.interleave = (k.blocks[0] == k.blocks[1] && k.blocks[1] == k.blocks[2] &&
                    k.blocks[2] == k.blocks[3]) ? 1 : 0;
    k.group = 1;
    k.planes = p[0].n * p[0].c;
    const int lv = lanes_for(Lv, pv);
    const int lh = lanes_for(Lh, ph);
    const int nthreads = lv > lh ? lv : lh;
    if (p[0].dtype == kF32) return launch_fused4<float, float>(k, pv, ph, nthreads, stream);
    if (p[0].wdtype == kPairF16) return launch_fused4<bf16_t, WPair>(k, pv, ph, nthreads, stream);
    return launch_fused4<bf16_t, bf16_t>(k, pv, ph, nthreads, stream);
}

// The long-line kernel (scan_lp.hpp) serves every launch whose lines split
// into whole 16-byte vectors on at most lp::kMaxLanes lanes, with 16-byte
// aligned tensors: its per-step work is a fraction of the one-position-per-
// lane kernel's, which matters most when few lines run (the step latency
// decides the time) and still pays when the GPU is full.
#ifndef GSPN_LP_MAX_GROUP
#define GSPN_LP_MAX_GROUP 2
#endif
constexpr int64_t kLpGroupMinBlocks = 2048;  // workgroups left after grouping: 8 per CU

bool lp_eligible(const ScanParams (&p)[4]) {
    const int esz = p[0].dtype == kF32 ? 4 : 2;
    const int P = 16 / esz;
    for (int d = 0; d < 4; ++d) {
        const int64_t L = p[d].w;
        if (L % P != 0 || L / P > lp::kMaxLanes) return false;
        if (!aligned_to(p[d].x, 16) || !aligned_to(p[d].lam, 16) || !aligned_to(p[d].out, 16) ||
            !aligned_to(p[d].wts, 16))
            return false;
    }
    return true;
}

// The banded kernel (scan_band.hpp) serves long-line launches with so few
// lines that one workgroup per line would leave most CUs idle: one wave of
// 16-byte vectors covers a segment of half its positions plus a halo of a
// quarter on each side, and a band runs as many steps as the halo is wide.
namespace {

constexpr int64_t kBandMaxLines = 64;  // lines (planes x 4 directions) below which it pays
constexpr int kBandMaxLaunches = 32;

int band_positions(int dtype) { return 64 * GSPN_BAND_WAVES * GSPN_BAND_BYTES / (dtype == kF32 ? 4 : 2); }

}  // namespace

int band_launches(const ScanParams (&p)[4]) {
    if (!lp_eligible(p)) return 0;
    for (int d = 0; d < 4; ++d)
        if (p[d].mscale) return 0;  // merge weights are applied after the scan (launch_combine)
    // outputs in the storage type, or fp32 states
    if (p[0].odtype != -1 && p[0].odtype != p[0].dtype && p[0].odtype != kF32) return 0;
    const int span = band_positions(p[0].dtype);
    const int64_t planes = p[0].n * p[0].c;
    if (planes * 4 > kBandMaxLines) return 0;
    int smax = 0;
    for (int d = 0; d < 4; ++d) {
        if (p[d].w < span) return 0;  // lines shorter than one workgroup's span gain nothing
        smax = static_cast<int>(p[d].h > smax ? p[d].h : smax);
    }
    const int halo = span / 4;
    const int n = (smax + halo - 1) / halo;
    return n <= kBandMaxLaunches ? n : 0;
}

int64_t band_state_floats(int64_t planes, int64_t lmax) { return 2 * 4 * planes * lmax; }

hipError_t launch_scan4_band(const ScanParams (&p)[4], float* state, int index, hipStream_t stream) {
    const int P = GSPN_BAND_BYTES / (p[0].dtype == kF32 ? 4 : 2);
    const int span = band_positions(p[0].dtype);
    const int64_t planes = p[0].n * p[0].c;
    BandK b;
    b.seg = span / 2;
    b.halo = span / 4;
    b.t0 = index * b.halo;
    int64_t lmax = 0;
    for (int d = 0; d < 4; ++d) {
        b.d[d] = make_args(p[d], P);
        b.nseg[d] = (b.d[d].L + b.seg - 1) / b.seg;
        b.blocks[d] = b.t0 < b.d[d].S ? planes * b.nseg[d] : 0;
        lmax = b.d[d].L > lmax ? b.d[d].L : lmax;
    }
    b.sstride = planes * lmax;
    b.planes = planes;
    b.xcd_lines = (planes * 4) % 8 == 0;
    for (int d = 0; d < 4; ++d)
        b.xcd_lines = b.xcd_lines && b.blocks[d] > 0 && b.nseg[d] == b.nseg[0];
    b.hin = state + (index & 1) * 4 * b.sstride;
    b.hout = state + ((index + 1) & 1) * 4 * b.sstride;
    if (p[0].dtype == kF32) {
        return p[0].wts_are_logits ? launch_band4<float, float, true>(b, stream)
                                   : launch_band4<float, float, false>(b, stream);
    }
    if (p[0].odtype == kF32) {
        if (p[0].wdtype == kPairF16) return launch_band4<bf16_t, WPair, false, float>(b, stream);
        return launch_band4<bf16_t, bf16_t, true, float>(b, stream);
    }
    if (p[0].wdtype == kPairF16) return launch_band4<bf16_t, WPair, false>(b, stream);
    return launch_band4<bf16_t, bf16_t, true>(b, stream);
}

bool lp_xtile_supported(const ScanParams (&p)[4]) {
    if (p[0].dtype != kF32 || !lp_eligible(p)) return false;
    for (int d = 0; d < 4; ++d)
        if (p[d].mscale || (p[d].odtype != -1 && p[d].odtype != kF32)) return false;
    // one 256-lane workgroup a line (the tile's loaders); the horizontal
    // scans unchunked, their steps whole tiles
    const int64_t L01 = p[0].w, L23 = p[2].w;
    const int lanes = lanes_for(static_cast<int>(L01 > L23 ? L01 : L23), 4);
    if (lanes != lp::kMaxLanes) return false;
    for (int d = 2; d < 4; ++d)
        if (p[d].chunk < p[d].h || p[d].h % LpXTile::TS != 0) return false;
    // more lines than the banded kernel takes
    return band_launches(p) == 0 && p[0].n * p[0].c * 4 > kBandMaxLines;
}

hipError_t launch_scan4v(const ScanParams (&p)[4], hipStream_t stream, int* kind) {
    // the separate output maps are merged afterwards (launch_combine), which
    // applies any merge weights
    for (int d = 0; d < 4; ++d)
        if (p[d].mscale) return hipErrorInvalidValue;
    // every p[d] is a vertical-form scan (dir 0 or 1); p[0..1] share one line
    // length, p[2..3] another
    const int l01 = static_cast<int>(p[0].w);
    const int l23 = static_cast<int>(p[2].w);
    // fp32 outputs of a bf16 scan (states kept at full precision): logits or
    // half-pair weights
    const bool wide_out = p[0].dtype == kBF16 && p[0].odtype == kF32;
    if (wide_out && !((p[0].wdtype == kBF16 && p[0].wts_are_logits) || p[0].wdtype == kPairF16))
        return hipErrorInvalidValue;
    if (lp_eligible(p)) {
        const int P = p[0].dtype == kF32 ? 4 : 8;
        const int a = lanes_for(l01, P);
        const int b = lanes_for(l23, P);
        const int lanes = a > b ? a : b;
        const bool logits = p[0].wts_are_logits != 0;
        // Normalised weights are shared by every channel: when the launch is
        // large enough to fill the GPU anyway, run several channels of a line
        // in one workgroup so that their weight loads coincide.
        const int64_t planes = p[0].n * p[0].c;
        int group = 1;
        if (!logits) {
            while (group * 2 <= GSPN_LP_MAX_GROUP && group * 2 * lanes <= lp::kMaxLanes &&
                   (planes + group * 2 - 1) / (group * 2) * 4 >= kLpGroupMinBlocks)
                group *= 2;
        }
        const bool xt = p[2].xtile || p[3].xtile;
        if (xt && (!lp_xtile_supported(p) || !p[2].xtile || !p[3].xtile || p[0].xtile || p[1].xtile))
            return hipErrorInvalidValue;
        if (xt) group = 1;
        Scan4K k;
        for (int d = 0; d < 4; ++d) {
            k.d[d] = make_args(p[d], P);
            k.blocks[d] = (planes + group - 1) / group * k.d[d].nchunks;
        }
        k.interleave = (k.blocks[0] == k.blocks[1] && k.blocks[1] == k.blocks[2] &&
                        k.blocks[2] == k.blocks[3]) ? 1 : 0;
        k.group = group;
        k.planes = planes;
        const int nthreads = lanes * group;
        if (kind) *kind = 3;
        if (xt) {
            return logits ? launch_fused4lp<float, float, true, float, true>(k, nthreads, stream)
                          : launch_fused4lp<float, float, false, float, true>(k, nthreads, stream);
        }
        if (p[0].dtype == kF32) {
            return logits ? launch_fused4lp<float, float, true>(k, nthreads, stream)
                          : launch_fused4lp<float, float, false>(k, nthreads, stream);
        }
        if (p[0].wdtype == kPairF16) {
            return wide_out ? launch_fused4lp<bf16_t, WPair, false, float>(k, nthreads, stream)
                            : launch_fused4lp<bf16_t, WPair, false>(k, nthreads, stream);
        }
        if (wide_out) return launch_fused4lp<bf16_t, bf16_t, true, float>(k, nthreads, stream);
        return launch_fused4lp<bf16_t, bf16_t, true>(k, nthreads, stream);
    }
    if (kind) *kind = 2;
    const int pv = l01 > 1024 ? 2 : 1;
    const int ph = l23 > 1024 ? 2 : 1;
    Scan4K k;
    for (int d = 0; d < 4; ++d) {
        k.d[d] = make_args(p[d], d < 2 ? pv : ph);
        k.blocks[d] = p[d].n * p[d].c * k.d[d].nchunks;
    }
    k.interleave = (k.blocks[0] == k.blocks[1] && k.blocks[1] == k.blocks[2] &&
                    k.blocks[2] == k.blocks[3]) ? 1 : 0;
    k.group = 1;
    k.planes = p[0].n * p[0].c;
    const int a = lanes_for(l01, pv);
    const int b = lanes_for(l23, ph);
    const int nthreads = a > b ? a : b;
    if (p[0].dtype == kF32) return launch_fused4v<float, float>(k, pv, ph, nthreads, stream);
    if (p[0].wdtype == kPairF16) {
        return wide_out ? launch_fused4v<bf16_t, WPair, float>(k, pv, ph, nthreads, stream)
                        : launch_fused4v<bf16_t, WPair>(k, pv, ph, nthreads, stream);
    }
    if (wide_out) return launch_fused4v<bf16_t, bf16_t, float>(k, pv, ph, nthreads, stream);
    return launch_fused4v<bf16_t, bf16_t>(k, pv, ph, nthreads, stream);
}

}  // namespace gspn
