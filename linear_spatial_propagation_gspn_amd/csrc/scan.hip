// scan.hip -- launch configuration of the line-scan kernels (the kernels and
// their launch families live in scan_kernel.hpp, instantiated per storage type
// and direction family in scan_{f32,bf16}_{vert,horiz}.hip and
// scan4_{f32,bf16}.hip).
#include "scan_kernel.hpp"

namespace gspn {

extern template hipError_t launch_family<float, false>(const ScanConfig&, bool, const ScanK&, int64_t,
                                                       int, hipStream_t);
extern template hipError_t launch_family<float, true>(const ScanConfig&, bool, const ScanK&, int64_t,
                                                      int, hipStream_t);
extern template hipError_t launch_family<bf16_t, false>(const ScanConfig&, bool, const ScanK&, int64_t,
                                                        int, hipStream_t);
extern template hipError_t launch_family<bf16_t, true>(const ScanConfig&, bool, const ScanK&, int64_t,
                                                       int, hipStream_t);
extern template hipError_t launch_fused4<float>(const Scan4K&, int, int, int, hipStream_t);
extern template hipError_t launch_fused4<bf16_t>(const Scan4K&, int, int, int, hipStream_t);

namespace {

// Positions per lane and workgroup size for a line of L positions: one
// position per lane up to 1024 lanes (16 waves, four per SIMD, which hides the
// latency of each step's chain better than fewer, fatter lanes), then 2, 4
// or 8 positions per lane for longer lines.
ScanConfig choose_config(bool horiz, int L) {
#if defined(GSPN_VERT_P) && defined(GSPN_VERT_MAXT)
    if (!horiz && (L + GSPN_VERT_P - 1) / GSPN_VERT_P <= GSPN_VERT_MAXT) return {GSPN_VERT_P, GSPN_VERT_MAXT};
#endif
#if defined(GSPN_HORIZ_P) && defined(GSPN_HORIZ_MAXT)
    if (horiz && (L + GSPN_HORIZ_P - 1) / GSPN_HORIZ_P <= GSPN_HORIZ_MAXT)
        return {GSPN_HORIZ_P, GSPN_HORIZ_MAXT};
#endif
    (void)horiz;
    ScanConfig c{1, 256};
    while (c.P < 8 && (L + c.P - 1) / c.P > 1024) c.P *= 2;
    c.maxt = (L + c.P - 1) / c.P > 256 ? 1024 : 256;
    return c;
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
    k.accumulate = p.accumulate ? 1 : 0;
    k.vec_frame = (L % P == 0) && aligned_to(p.wts, esz * P) && aligned_to(p.lam, esz * P);
    k.vec_arr = (L % P == 0) && aligned_to(p.x, esz * P) && aligned_to(p.out, esz * P);
    k.vec_tile = (S % vw == 0) && aligned_to(p.x, 16) && aligned_to(p.out, 16);
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
    if (p.dtype == kF32) {
        return horiz ? launch_family<float, true>(cfg, rev, k, nblocks, nthreads, stream)
                     : launch_family<float, false>(cfg, rev, k, nblocks, nthreads, stream);
    }
    return horiz ? launch_family<bf16_t, true>(cfg, rev, k, nblocks, nthreads, stream)
                 : launch_family<bf16_t, false>(cfg, rev, k, nblocks, nthreads, stream);
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
    const int lv = lanes_for(Lv, pv);
    const int lh = lanes_for(Lh, ph);
    const int nthreads = lv > lh ? lv : lh;
    if (p[0].dtype == kF32) return launch_fused4<float>(k, pv, ph, nthreads, stream);
    return launch_fused4<bf16_t>(k, pv, ph, nthreads, stream);
}

}  // namespace gspn
