// scan.hip -- launch configuration of the line-scan kernel (the kernel and
// its launch families live in scan_kernel.hpp, instantiated per storage type
// and direction family in scan_{f32,bf16}_{vert,horiz}.hip).
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

namespace {

// Positions per lane and workgroup size for a line of L positions.
// Vertical lines: at most 256 lanes (one wave per SIMD) while P <= 8 allows,
// which leaves registers for the prefetch ring; longer lines take P = 8 on up
// to 1024 lanes.  Horizontal lines: one position per lane up to 1024 lanes,
// since the row tiles already take many registers.
ScanConfig choose_config(bool horiz, int L) {
    ScanConfig c{1, 256};
#if defined(GSPN_VERT_P) && defined(GSPN_VERT_MAXT)
    if (!horiz && (L + GSPN_VERT_P - 1) / GSPN_VERT_P <= GSPN_VERT_MAXT) return {GSPN_VERT_P, GSPN_VERT_MAXT};
#endif
#if defined(GSPN_HORIZ_P) && defined(GSPN_HORIZ_MAXT)
    if (horiz && (L + GSPN_HORIZ_P - 1) / GSPN_HORIZ_P <= GSPN_HORIZ_MAXT)
        return {GSPN_HORIZ_P, GSPN_HORIZ_MAXT};
#endif
    const int cap = horiz ? 1024 : 256;
    while (c.P < 8 && (L + c.P - 1) / c.P > cap) c.P *= 2;
    c.maxt = (horiz || (L + c.P - 1) / c.P > 256) ? 1024 : 256;
    return c;
}

bool aligned_to(const void* ptr, size_t bytes) {
    return (reinterpret_cast<uintptr_t>(ptr) % bytes) == 0;
}

}  // namespace

hipError_t launch_scan(const ScanParams& p, hipStream_t stream) {
    const bool horiz = (p.dir == 2 || p.dir == 3);
    const bool rev = (p.dir == 1 || p.dir == 3);
    const int S = static_cast<int>(horiz ? p.w : p.h);
    const int L = static_cast<int>(horiz ? p.h : p.w);
    const ScanConfig cfg = choose_config(horiz, L);
    const int lanes = (L + cfg.P - 1) / cfg.P;
    const int nthreads = ((lanes + 63) / 64) * 64;
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
    k.reverse = rev ? 1 : 0;
    k.logits = p.wts_are_logits ? 1 : 0;
    k.accumulate = p.accumulate ? 1 : 0;
    k.vec_frame = (L % cfg.P == 0) && aligned_to(p.wts, esz * cfg.P) && aligned_to(p.lam, esz * cfg.P);
    k.vec_arr = (L % cfg.P == 0) && aligned_to(p.x, esz * cfg.P) && aligned_to(p.out, esz * cfg.P);
    k.vec_tile = (S % vw == 0) && aligned_to(p.x, 16) && aligned_to(p.out, 16);
    const int64_t nblocks = p.n * p.c * k.nchunks;

    if (p.dtype == kF32) {
        return horiz ? launch_family<float, true>(cfg, rev, k, nblocks, nthreads, stream)
                     : launch_family<float, false>(cfg, rev, k, nblocks, nthreads, stream);
    }
    return horiz ? launch_family<bf16_t, true>(cfg, rev, k, nblocks, nthreads, stream)
                 : launch_family<bf16_t, false>(cfg, rev, k, nblocks, nthreads, stream);
}

}  // namespace gspn
