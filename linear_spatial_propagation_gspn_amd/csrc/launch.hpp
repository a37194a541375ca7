// launch.hpp -- host-side launchers behind the C ABI (internal to libgspn).
// Arguments reaching these functions have been validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "check.hpp"

namespace gspn {

enum Dtype { kF32 = 0, kBF16 = 1 };

// Weight formats a scan can read besides the storage type itself: fp32
// triples (kF32) or, for 16-bit storage, packed half pairs (kPairF16, see
// WPair in device.hpp).
enum WeightFormat { kPairF16 = 2 };

struct ScanParams {
    const void* x;
    const void* wts;
    const void* lam;
    void* out;
    int64_t n, c, cw, h, w;
    int dir;             // 0 T2B, 1 B2T, 2 L2R, 3 R2L
    int64_t chunk;       // steps per chunk, already clamped to [1, S]
    int wts_are_logits;
    int accumulate;
    int dtype;   // storage type of x, lam, out
    int wdtype;  // format of wts: dtype, or for weights normalised beforehand kF32 / kPairF16
    int odtype = -1;  // storage type of out: -1 = dtype; kF32 for fp32 states of bf16 scans
    const float* mscale = nullptr;  // learnable merge: weight of each channel ([c]) for this direction
    int xtile = 0;  // a vertical-form horizontal scan whose x is the array-frame plane, read through
                    // LDS column tiles by the long-line kernel (lp_xtile_supported) instead of rows of
                    // x transposed
};

hipError_t launch_scan(const ScanParams& p, hipStream_t stream);

// Whether the four-direction long-line launch can read the horizontal
// directions' x through LDS column tiles (ScanParams::xtile) for these
// vertical-form directions: fp32 storage, one 256-lane workgroup a line,
// unchunked horizontal scans of a multiple of 32 steps, 16-byte aligned
// tensors, more lines than the banded kernel takes.  p[2], p[3] describe the
// horizontal directions in vertical form with x the array-frame plane.
bool lp_xtile_supported(const ScanParams (&p)[4]);

// The four directions of one forward in one launch; p[d] describes direction d
// (each with its own output buffer, accumulate = 0).
hipError_t launch_scan4(const ScanParams (&p)[4], hipStream_t stream);
bool fused4_supported(int64_t h, int64_t w);

// Four vertical-form scans in one launch (p[d].dir in {0, 1}): used for the
// vertical directions on x and the horizontal ones on the transposed x.
// Merge weights (mscale) are not taken: the merge of the separate outputs
// applies them.
// *kind (if given) receives the kernel used: 2 = one workgroup per line,
// 3 = the long-line kernel (gspn_scan_kernel values).
hipError_t launch_scan4v(const ScanParams (&p)[4], hipStream_t stream, int* kind = nullptr);

// The same four vertical-form scans (outputs in the storage type) for
// launches of very few long lines: each line is split across workgroups and
// the scan advances in bands of steps, one launch per band.
// band_launches: the number of bands, or 0 when this path does not apply.
// state: band_state_floats(n * c, max line length) floats of scratch (fp32
// states at the band boundaries); bands run in order 0 .. band_launches - 1.
int band_launches(const ScanParams (&p)[4]);
int64_t band_state_floats(int64_t planes, int64_t lmax);
hipError_t launch_scan4_band(const ScanParams (&p)[4], float* state, int band, hipStream_t stream);

// All four directions of planes of at most 64 x 64 in one pass, y written
// once (chunk[d]: steps per chunk of direction d, clamped to [1, S_d];
// merge: learnable merge weights [4][c], or null for the plain sum).
bool plane4_supported(int64_t h, int64_t w);
hipError_t launch_plane4(const void* x, const void* const logits[4], const void* const lam[4], const float* merge,
                         void* y, int64_t n, int64_t c, int64_t cw, int64_t h, int64_t w, const int64_t chunk[4],
                         int dtype, hipStream_t stream);

// Many big planes: one workgroup per (n, c) plane runs L2R, R2L, T2B, B2T
// one after another, building y in place (seq4.hip).  Planes with both sides
// multiples of 64 in [64, 1024]; 16-byte aligned tensors.  wts[d]: logits
// (wdtype == dtype) or, for bf16, channel-shared half pairs (kPairF16);
// chunk[d] clamped to [1, S_d]; z: scratch of n*c*h*w elements of the
// storage type ([n][c][w][h], the horizontal directions' sum).
bool seq4_supported(int64_t h, int64_t w);
constexpr int64_t kSeq4MinPlanes =
#ifdef GSPN_SEQ4_MIN_PLANES
    GSPN_SEQ4_MIN_PLANES;
#else
    256;  // one workgroup per CU: fewer planes would leave CUs idle
#endif
// Runs the first `run` of the n * c planes (run <= n * c).  states: fp32
// maps of the four unweighted scans, map d at states + d * states_ld, each in
// its direction's scan frame, or null.
hipError_t launch_seq4(const void* x, const void* const wts[4], const void* const lam[4], const float* merge,
                       void* y, void* z, int64_t n, int64_t c, int64_t cw, int64_t h, int64_t w,
                       const int64_t chunk[4], int dtype, int wdtype, int wts_are_logits, int64_t run,
                       float* states, int64_t states_ld, hipStream_t stream);

// Compute units of the current device (cached per device; 0 if unknown).
int device_compute_units();

// dst[p][c][r] = src[p][r][c] for `planes` planes of R x Cc elements.
hipError_t launch_transpose(const void* src, void* dst, int64_t planes, int R, int Cc, int dtype,
                            hipStream_t stream);

// y[p][r][c] = ((m2 z2[p][c][r] + m3 z3[p][c][r]) + m0 y[p][r][c] (if accumulate)) + m1 a[p][r][c]
// over planes of R x Cc; a, z2, z3 may be NULL; z2, z3 are Cc x R planes;
// m0..m3: merge[k][p % nch] (learnable merge weights [4][nch], rows mld floats
// apart; mld = 0 means nch), or 1 if merge is null.
hipError_t launch_combine(void* y, const void* a, const void* z2, const void* z3, int64_t planes, int R,
                          int Cc, int accumulate, int dtype, hipStream_t stream, const float* merge = nullptr,
                          int64_t nch = 1, int64_t mld = 0);

// y[p][r][c] = ((m2 s2[p][c][r] + m3 s3[p][c][r]) + m0 s0[p][r][c]) + m1 s1[p][r][c]:
// the same merge from four fp32 state maps (s2, s3 in the transposed frame),
// y in the storage type.
hipError_t launch_combine_states(void* y, const float* s0, const float* s1, const float* s2, const float* s3,
                                 int64_t planes, int R, int Cc, int dtype, hipStream_t stream,
                                 const float* merge = nullptr, int64_t nch = 1, int64_t mld = 0);

// out_dtype: storage type of w_out (-1: the same as dtype; kF32 is allowed
// for bf16 logits).
hipError_t launch_normalize(int dir, int64_t n, int64_t cw, int64_t h, int64_t w,
                            const void* logits, void* w_out, int dtype, hipStream_t stream,
                            int out_dtype = -1);

// Channel-shared logits of the four directions ([n][1][3][S][L], in each
// direction's scan frame) into packed half pairs [n][S][L] (WPair format),
// one launch.
hipError_t launch_normalize_pair4(int64_t n, int64_t h, int64_t w, const void* const logits[4],
                                  void* const w_out[4], int dtype, hipStream_t stream);

hipError_t launch_merge4(const void* h0, const void* h1, const void* h2, const void* h3, void* y,
                         int64_t numel, int dtype, hipStream_t stream);


// One direction of the adjoint scan, in vertical form (horizontal directions
// on x and dL/dy transposed into their scan frame).  hs: the direction's
// forward states in fp32; dz: logits gradient in the storage type, or
// (shared) fp32 channel sums of the weight-gradient differences
// dw_{-1} - dw_0 and dw_{+1} - dw_0, planes 0 and 1 of [n][3][S][L], that the
// kernel adds into (launch_finish_shared_dz turns them into dlogits).
struct AdjointParams {
    const void* x;
    const void* g;
    const void* lam;
    const void* logits;
    const void* hs;
    void* dlam;
    void* dz;
    void* dx;
    int64_t n, c, cw, S, L;
    int64_t chunk;  // clamped to [1, S]
    int reverse;
    int shared;
    int dtype;
    const float* mscale = nullptr;  // learnable merge: weight of each channel ([c]) for this direction
    float* dmerge = nullptr;        // its gradient [c], fp32, added into (null: not wanted)
};

// What launch_adjoint4 ran: positions per lane, channels per workgroup (the
// shared-logit gradient is summed over them) and whether the streams touched
// once carry the non-temporal hint.
struct AdjointPlan {
    int positions;
    int group;
    int nontemporal;
};
hipError_t launch_adjoint4(const AdjointParams (&p)[4], hipStream_t stream, AdjointPlan* plan = nullptr);

// The same adjoint for launches of very few long, unchunked lines: each line
// is split across workgroups (segments with halos) and the adjoint advances
// in bands of steps, one launch per band, bands 0 .. adjoint_band_launches
// - 1 in order.  adjoint_band_launches: the number of bands, or 0 when this
// path does not apply (chunked lines, more than 16 planes, sides under 512).
// qbuf: adjoint_band_floats(n * c, max(h, w)) floats of scratch, which the
// workspace holds whenever adjoint_band_shape(n * c, h, w).
bool adjoint_band_shape(int64_t planes, int64_t h, int64_t w);
int64_t adjoint_band_floats(int64_t planes, int64_t lmax);
int adjoint_band_launches(const AdjointParams (&p)[4]);
hipError_t launch_adjoint4_band(const AdjointParams (&p)[4], float* qbuf, int band, hipStream_t stream);

// All four directions' adjoint for planes of at most 64 x 64, one workgroup
// per plane (x, gy and dx in the array frame; the per-direction tensors in
// each direction's scan frame; dz as in AdjointParams: the storage type, or
// fp32 difference sums when shared).  The launch first recomputes the
// forward's fp32 states into hs (workspace, each direction's scan frame),
// then runs the adjoint on them.  dx is written, dmerge (if given) added into.
struct AdjPlaneParams {
    const void* x;
    const void* g;
    const void* z[4];
    const void* lam[4];
    float* hs[4];
    void* dlam[4];
    void* dz[4];
    void* dx;
    const float* merge;
    float* dmerge;
    int64_t n, c, cw, h, w;
    int64_t chunk[4];  // clamped to [1, S_d]
    int shared;
    int dtype;
};
hipError_t launch_adjplane(const AdjPlaneParams& p, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
// Shared logits: dlogits (storage type, [n][3][S][L]) from the channel sums
// of the weight-gradient differences that the adjoints added into sums
// (planes 0 and 1 of [n][3][S][L] fp32) and the logits themselves.
hipError_t launch_finish_shared_dz(const float* sums, const void* logits, void* dlogits, int64_t n, int64_t S,
                                   int64_t L, int dtype, hipStream_t stream);

hipError_t launch_project(int64_t n, int64_t c_in, int64_t hw, int64_t c_out, const void* in,
                          const void* weight, void* out, int dtype, hipStream_t stream);

// Weight gradients of the projections, in two launches.  First
// launch_project_wgrad: with wt (weights [k][c]) given, pout = wt . big as
// launch_project computes it; in every case the partial sums of
// G[c][j] = sum over images and pixels of big[n][c][p] * small[n][j][p]
// (big [n][c][hw], small [n][k][hw]) over at most wgrad_slots(n, hw) runs of
// pixels into part ([slots][c][k] fp32), *slots_used receiving the count.
// Then launch_wgrad_reduce: out[c * sc + j * sk] = sum over the slots, in a
// fixed order.  bf16 with hw % 128 == 0, c % 8 == 0, k <= 16 and 16-byte
// aligned tensors runs on the matrix cores, in groups of at most
// 32 kWgradMaxBlocks channels (for c up to that, with the projection folded
// into the same pass over big); everything else on the VALU.
constexpr int64_t kWgradMaxSlots = 2048;
constexpr int kWgradMaxBlocks = 10;
int64_t wgrad_slots(int64_t n, int64_t hw);
hipError_t launch_project_wgrad(int64_t n, int64_t c, int64_t hw, int64_t k, const void* big, const void* small,
                                const void* wt, void* pout, float* part, int dtype, hipStream_t stream,
                                int64_t* slots_used);
hipError_t launch_wgrad_reduce(const float* part, int64_t slots, int64_t c, int64_t k, float* out, int64_t sc,
                               int64_t sk, hipStream_t stream);

// The allocation-free forward's scratch (noalloc.hip): a static device array
// of kNoallocScratchBytes per GPU; *out receives the current device's copy
// (its address looked up on that device's first call, then cached).
constexpr int64_t kNoallocScratchBytes = int64_t{64} << 20;
hipError_t noalloc_scratch(void** out);

}  // namespace gspn
