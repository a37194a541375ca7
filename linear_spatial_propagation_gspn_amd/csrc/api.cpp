// api.cpp -- the C ABI of libgspn (declared in include/gspn.h): host-side
// validation of every argument, then kernel launches on the caller's stream.
// Validation never touches the device; nothing here allocates, frees or
// synchronises.
#include "../../include/gspn.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "launch.hpp"

namespace {

using gspn::kBF16;
using gspn::kF32;

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxElems = int64_t{1} << 58;

bool valid_dtype(int dt) { return dt == GSPN_F32 || dt == GSPN_BF16; }
bool valid_layout(int l) { return l == GSPN_LAYOUT_SCAN || l == GSPN_LAYOUT_ARRAY; }
size_t elem_size(int dt) { return dt == GSPN_F32 ? 4 : 2; }
bool valid_dir(int d) { return d >= GSPN_T2B && d <= GSPN_R2L; }
bool horizontal(int d) { return d == GSPN_L2R || d == GSPN_R2L; }

// Product of non-negative dims without overflow; -1 when it exceeds kMaxElems.
int64_t checked_product(std::initializer_list<int64_t> dims) {
    int64_t p = 1;
    for (int64_t d : dims) {
        if (d == 0) return 0;
    }
    for (int64_t d : dims) {
        if (d > kMaxElems / p) return -1;
        p *= d;
    }
    return p;
}

bool dims_ok(std::initializer_list<int64_t> dims) {
    for (int64_t d : dims)
        if (d < 0 || d > kMaxDim) return false;
    return checked_product(dims) >= 0;
}

// The long-line scan reading the horizontal directions' x through LDS
// column tiles instead of a transposed copy (a build parameter, so that the
// two can be measured against each other).
#ifndef GSPN_XTILE
#define GSPN_XTILE 1
#endif
constexpr bool xtile_enabled() { return GSPN_XTILE != 0; }

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

gspn_status from_hip(hipError_t e) { return e == hipSuccess ? GSPN_OK : GSPN_ERR_HIP; }

// Optional event timing of the launches of one forward call: a pair of HIP
// events around each launch, read back by finish().
struct Timer {
    static constexpr int kMax = 128;
    hipStream_t st = nullptr;
    int count = 0;
    int stage[kMax] = {};
    hipEvent_t a[kMax] = {};
    hipEvent_t b[kMax] = {};
    int scan_kernel = GSPN_SCAN_NONE;
    gspn_adjoint_plan adjoint = {0, 0, 0, 0};

    ~Timer() {
        for (int i = 0; i < count; ++i) {
            (void)hipEventDestroy(a[i]);
            (void)hipEventDestroy(b[i]);
        }
    }
    // Records the opening event of a launch of stage s.
    hipError_t open(int s) {
        if (count >= kMax) return hipErrorInvalidValue;
        hipError_t e = hipEventCreate(&a[count]);
        if (e != hipSuccess) return e;
        e = hipEventCreate(&b[count]);
        if (e != hipSuccess) {
            (void)hipEventDestroy(a[count]);
            return e;
        }
        stage[count] = s;
        ++count;
        return hipEventRecord(a[count - 1], st);
    }
    hipError_t close() { return hipEventRecord(b[count - 1], st); }
    // Waits for the last event and sums the durations per stage.
    hipError_t finish(gspn_stage_times* t) {
        for (int s = 0; s < GSPN_NUM_STAGES; ++s) {
            t->ms[s] = 0.0f;
            t->launches[s] = 0;
        }
        t->scan_kernel = scan_kernel;
        t->adjoint = adjoint;
        if (count == 0) return hipSuccess;
        hipError_t e = hipEventSynchronize(b[count - 1]);
        if (e != hipSuccess) return e;
        for (int i = 0; i < count; ++i) {
            float ms = 0.0f;
            e = hipEventElapsedTime(&ms, a[i], b[i]);
            if (e != hipSuccess) return e;
            t->ms[stage[i]] += ms;
            t->launches[stage[i]] += 1;
        }
        return hipSuccess;
    }
};

// Runs one launch, bracketed by timing events when a timer is given.
template <typename F>
hipError_t timed(Timer* t, int stage, F&& launch) {
    if (!t) return launch();
    hipError_t e = t->open(stage);
    if (e != hipSuccess) return e;
    const hipError_t el = launch();
    e = t->close();
    return el != hipSuccess ? el : e;
}

struct ScanCheck {
    gspn_status st;
    int64_t chunk;  // clamped to [1, S]
};

// Shared validation of one scan direction's arguments.
ScanCheck check_scan(int dir, int64_t chunk_len, int64_t n, int64_t c, int64_t h, int64_t w,
                     int64_t cw, int dtype, bool* empty) {
    *empty = false;
    if (!valid_dtype(dtype)) return {GSPN_ERR_BAD_DTYPE, 0};
    if (!valid_dir(dir)) return {GSPN_ERR_BAD_DIRECTION, 0};
    if (!dims_ok({n, c, h, w})) return {GSPN_ERR_BAD_SHAPE, 0};
    if (chunk_len < 0) return {GSPN_ERR_BAD_CHUNK, 0};
    if (!(cw == 1 || cw == c)) return {GSPN_ERR_BAD_WEIGHT_CHANNELS, 0};
    if (checked_product({n, c, h, w}) == 0) {
        *empty = true;
        return {GSPN_OK, 0};
    }
    const int64_t S = horizontal(dir) ? w : h;
    const int64_t L = horizontal(dir) ? h : w;
    if (L > GSPN_MAX_LINE) return {GSPN_ERR_UNSUPPORTED, 0};
    const int64_t K = (chunk_len == 0 || chunk_len >= S) ? S : chunk_len;
    const int64_t nchunks = (S + K - 1) / K;
    if (n * c > INT_MAX / nchunks) return {GSPN_ERR_UNSUPPORTED, 0};
    return {GSPN_OK, K};
}

// GSPN_LAYOUT_ARRAY: bytes of the scan-frame copies of the two horizontal
// directions' logits ([n][cw][3][w][h] each) and lambdas ([n][c][w][h] each)
// in the storage type, rounded up to 4 bytes; -1 if that overflows.
int64_t layout_copy_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int dtype) {
    const int64_t nhw = checked_product({n, h, w});
    if (nhw < 0) return -1;
    const int64_t elems = 2 * (3 * cw + c);  // <= 8 c, so elems * nhw < 2^61
    const int64_t es = static_cast<int64_t>(elem_size(dtype));
    if (nhw > 0 && elems > (INT64_MAX / 2) / es / nhw) return -1;
    return (elems * nhw * es + 3) / 4 * 4;
}

// The four-direction launches run a workgroup per (plane, chunk) of every
// direction: the total must fit one launch's grid.
// Bands of the fp32-state forward for very few long lines (0: the
// four-direction launch instead).  A forward keeping its states and a
// backward recomputing them take the same condition, so both run the same
// kernel and the states agree bit for bit.
int state_bands(const gspn::ScanParams (&p)[4], int64_t n, int64_t c, int64_t h, int64_t w) {
    return gspn::adjoint_band_shape(n * c, h, w) ? gspn::band_launches(p) : 0;
}

int64_t adjoint_band_bytes(int64_t n, int64_t c, int64_t h, int64_t w) {
    return gspn::adjoint_band_shape(n * c, h, w) ? gspn::adjoint_band_floats(n * c, h > w ? h : w) * 4 : 0;
}

bool fused_grid_ok(int64_t n, int64_t c, int64_t h, int64_t w, const int64_t chunks[4]) {
    int64_t total = 0;
    for (int d = 0; d < 4; ++d) {
        const int64_t S = horizontal(d) ? w : h;
        total += n * c * ((S + chunks[d] - 1) / chunks[d]);  // each term <= INT_MAX (check_scan)
    }
    return total <= INT_MAX;
}

}  // namespace

extern "C" {

const char* gspn_status_string(int status) {
    switch (status) {
        case GSPN_OK: return "GSPN_OK";
        case GSPN_ERR_NULL_POINTER: return "GSPN_ERR_NULL_POINTER: a required pointer is NULL";
        case GSPN_ERR_BAD_SHAPE: return "GSPN_ERR_BAD_SHAPE: a dimension is negative or too large";
        case GSPN_ERR_BAD_DIRECTION: return "GSPN_ERR_BAD_DIRECTION: direction is not 0..3";
        case GSPN_ERR_BAD_DTYPE: return "GSPN_ERR_BAD_DTYPE: dtype is not GSPN_F32 or GSPN_BF16";
        case GSPN_ERR_BAD_CHUNK: return "GSPN_ERR_BAD_CHUNK: chunk_len is negative";
        case GSPN_ERR_BAD_WEIGHT_CHANNELS:
            return "GSPN_ERR_BAD_WEIGHT_CHANNELS: weight channels must be 1 or C";
        case GSPN_ERR_MISALIGNED: return "GSPN_ERR_MISALIGNED: a pointer is not aligned to its element size";
        case GSPN_ERR_ALIASING: return "GSPN_ERR_ALIASING: an output overlaps an input";
        case GSPN_ERR_UNSUPPORTED:
            return "GSPN_ERR_UNSUPPORTED: line longer than GSPN_MAX_LINE or grid too large";
        case GSPN_ERR_HIP: return "GSPN_ERR_HIP: a HIP launch failed";
        case GSPN_ERR_WORKSPACE: return "GSPN_ERR_WORKSPACE: the workspace is smaller than required";
        case GSPN_ERR_BAD_LAYOUT: return "GSPN_ERR_BAD_LAYOUT: layout is not GSPN_LAYOUT_SCAN or GSPN_LAYOUT_ARRAY";
        default: return "unknown gspn_status";
    }
}

int gspn_abi_version(void) { return GSPN_ABI_VERSION; }

gspn_status gspn_normalize_weights(int dir, int64_t n, int64_t cw, int64_t h, int64_t w,
                                   const void* logits, void* w_out, int dtype, void* stream) {
    if (!valid_dtype(dtype)) return GSPN_ERR_BAD_DTYPE;
    if (!valid_dir(dir)) return GSPN_ERR_BAD_DIRECTION;
    if (!dims_ok({n, cw, 3, h, w})) return GSPN_ERR_BAD_SHAPE;
    const int64_t total = checked_product({n, cw, 3, h, w});
    if (total == 0) return GSPN_OK;
    if (!logits || !w_out) return GSPN_ERR_NULL_POINTER;
    const size_t es = elem_size(dtype);
    if (!aligned(logits, es) || !aligned(w_out, es)) return GSPN_ERR_MISALIGNED;
    const int64_t bytes = total * static_cast<int64_t>(es);
    if (overlap(logits, bytes, w_out, bytes)) return GSPN_ERR_ALIASING;
    return from_hip(gspn::launch_normalize(dir, n, cw, h, w, logits, w_out, dtype, as_stream(stream)));
}

gspn_status gspn_scan_fwd(int dir, int64_t chunk_len, int64_t n, int64_t c, int64_t h, int64_t w,
                          int64_t cw, const void* x, const void* wts, int wts_are_logits,
                          const void* lam, void* out, int accumulate, int dtype, void* stream) {
    bool empty = false;
    const ScanCheck ck = check_scan(dir, chunk_len, n, c, h, w, cw, dtype, &empty);
    if (ck.st != GSPN_OK || empty) return ck.st;
    if (!x || !wts || !lam || !out) return GSPN_ERR_NULL_POINTER;
    const size_t es = elem_size(dtype);
    if (!aligned(x, es) || !aligned(wts, es) || !aligned(lam, es) || !aligned(out, es))
        return GSPN_ERR_MISALIGNED;
    const int64_t xb = n * c * h * w * static_cast<int64_t>(es);
    const int64_t wb = n * cw * 3 * h * w * static_cast<int64_t>(es);
    if (overlap(out, xb, x, xb) || overlap(out, xb, wts, wb) || overlap(out, xb, lam, xb))
        return GSPN_ERR_ALIASING;
    gspn::ScanParams p;
    p.x = x;
    p.wts = wts;
    p.lam = lam;
    p.out = out;
    p.n = n;
    p.c = c;
    p.cw = cw;
    p.h = h;
    p.w = w;
    p.dir = dir;
    p.chunk = ck.chunk;
    p.wts_are_logits = wts_are_logits ? 1 : 0;
    p.accumulate = accumulate ? 1 : 0;
    p.dtype = dtype;
    p.wdtype = dtype;
    return from_hip(gspn::launch_scan(p, as_stream(stream)));
}

gspn_status gspn_merge4(const void* h0, const void* h1, const void* h2, const void* h3, void* y,
                        int64_t numel, int dtype, void* stream) {
    if (!valid_dtype(dtype)) return GSPN_ERR_BAD_DTYPE;
    if (numel < 0 || numel >= kMaxElems) return GSPN_ERR_BAD_SHAPE;
    if (numel == 0) return GSPN_OK;
    if (!h0 || !h1 || !h2 || !h3 || !y) return GSPN_ERR_NULL_POINTER;
    const size_t es = elem_size(dtype);
    if (!aligned(h0, es) || !aligned(h1, es) || !aligned(h2, es) || !aligned(h3, es) || !aligned(y, es))
        return GSPN_ERR_MISALIGNED;
    const int64_t b = numel * static_cast<int64_t>(es);
    if (overlap(y, b, h0, b) || overlap(y, b, h1, b) || overlap(y, b, h2, b) || overlap(y, b, h3, b))
        return GSPN_ERR_ALIASING;
    return from_hip(gspn::launch_merge4(h0, h1, h2, h3, y, numel, dtype, as_stream(stream)));
}

gspn_status gspn_proxy_project(int64_t n, int64_t c_in, int64_t h, int64_t w, int64_t c_out,
                               const void* in, const void* weight, void* out, int dtype,
                               void* stream) {
    if (!valid_dtype(dtype)) return GSPN_ERR_BAD_DTYPE;
    if (!dims_ok({n, c_in, h, w}) || !dims_ok({n, c_out, h, w}) || !dims_ok({c_out, c_in}))
        return GSPN_ERR_BAD_SHAPE;
    const int64_t out_elems = checked_product({n, c_out, h, w});
    if (out_elems == 0) return GSPN_OK;
    if (c_in == 0) return GSPN_ERR_BAD_SHAPE;
    if (!in || !weight || !out) return GSPN_ERR_NULL_POINTER;
    const size_t es = elem_size(dtype);
    if (!aligned(in, es) || !aligned(weight, es) || !aligned(out, es)) return GSPN_ERR_MISALIGNED;
    const int64_t ob = out_elems * static_cast<int64_t>(es);
    const int64_t ib = n * c_in * h * w * static_cast<int64_t>(es);
    const int64_t wb = c_out * c_in * static_cast<int64_t>(es);
    if (overlap(out, ob, in, ib) || overlap(out, ob, weight, wb)) return GSPN_ERR_ALIASING;
    return from_hip(gspn::launch_project(n, c_in, h * w, c_out, in, weight, out, dtype, as_stream(stream)));
}

gspn_status gspn_scan4_fwd(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                           int64_t chunk_len, const void* x, const void* const logits[4],
                           const void* const lam[4], void* const out[4], int dtype, void* stream) {
    int64_t chunks[4];
    for (int d = 0; d < 4; ++d) {
        bool empty = false;
        const ScanCheck ck = check_scan(d, chunk_len, n, c, h, w, cw, dtype, &empty);
        if (ck.st != GSPN_OK || empty) return ck.st;
        chunks[d] = ck.chunk;
    }
    if (!gspn::fused4_supported(h, w) || !fused_grid_ok(n, c, h, w, chunks)) return GSPN_ERR_UNSUPPORTED;
    if (!x || !logits || !lam || !out) return GSPN_ERR_NULL_POINTER;
    for (int d = 0; d < 4; ++d)
        if (!logits[d] || !lam[d] || !out[d]) return GSPN_ERR_NULL_POINTER;
    const size_t es = elem_size(dtype);
    if (!aligned(x, es)) return GSPN_ERR_MISALIGNED;
    for (int d = 0; d < 4; ++d)
        if (!aligned(logits[d], es) || !aligned(lam[d], es) || !aligned(out[d], es))
            return GSPN_ERR_MISALIGNED;
    const int64_t xb = n * c * h * w * static_cast<int64_t>(es);
    const int64_t wb = n * cw * 3 * h * w * static_cast<int64_t>(es);
    for (int d = 0; d < 4; ++d) {
        if (overlap(out[d], xb, x, xb)) return GSPN_ERR_ALIASING;
        for (int e = 0; e < 4; ++e) {
            if (overlap(out[d], xb, logits[e], wb) || overlap(out[d], xb, lam[e], xb))
                return GSPN_ERR_ALIASING;
            if (e != d && overlap(out[d], xb, out[e], xb)) return GSPN_ERR_ALIASING;
        }
    }
    gspn::ScanParams p[4];
    for (int d = 0; d < 4; ++d) {
        p[d].x = x;
        p[d].wts = logits[d];
        p[d].lam = lam[d];
        p[d].out = out[d];
        p[d].n = n;
        p[d].c = c;
        p[d].cw = cw;
        p[d].h = h;
        p[d].w = w;
        p[d].dir = d;
        p[d].chunk = chunks[d];
        p[d].wts_are_logits = 1;
        p[d].accumulate = 0;
        p[d].dtype = dtype;
        p[d].wdtype = dtype;
    }
    return from_hip(gspn::launch_scan4(p, as_stream(stream)));
}

int64_t gspn_forward4_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                                      int dtype, int layout) {
    if (!valid_dtype(dtype) || !valid_layout(layout) || !dims_ok({n, c, h, w}) || !(cw == 1 || cw == c)) return -1;
    const int64_t elems = checked_product({n, c, h, w});
    const int64_t maps = 4 * elems * static_cast<int64_t>(elem_size(dtype));
    // channel-shared weights over several channels, normalised once per
    // direction: fp32 triples for fp32 storage, packed half pairs for bf16
    const int64_t per_dir = checked_product({n, h, w}) * (dtype == GSPN_F32 ? 3 * 4 : 4);
    const int64_t weights = (cw == 1 && c > 1) ? 4 * per_dir : 0;
    // fp32 states at band boundaries for the banded scan of very few lines
    const int64_t states = gspn::band_state_floats(checked_product({n, c}), h > w ? h : w) * 4;
    const int64_t base = (maps + weights + 3) / 4 * 4 + states;
    if (layout == GSPN_LAYOUT_SCAN) return base;
    // then the scan-frame copies of the horizontal logits and lambdas
    const int64_t lc = layout_copy_bytes(n, c, h, w, cw, dtype);
    return lc < 0 ? -1 : base + lc;
}

}  // extern "C"

namespace {

// Channel-shared logits of the four directions normalised once into dst
// (direction d at dst + d * wdir): fp32 triples for fp32 storage, one
// launch per direction; packed half pairs for bf16, one launch for all four.
// Points the scans p[d] at them.
hipError_t prenormalise(int64_t n, int64_t h, int64_t w, const void* const logits[4], char* dst, int64_t wdir,
                        int dtype, hipStream_t st, Timer* tm, gspn::ScanParams (&p)[4]) {
    void* wd[4];
    for (int d = 0; d < 4; ++d) wd[d] = dst + d * wdir;
    if (dtype == GSPN_F32) {
        for (int d = 0; d < 4; ++d) {
            const hipError_t e = timed(tm, GSPN_STAGE_NORMALIZE, [&] {
                return gspn::launch_normalize(d, n, 1, h, w, logits[d], wd[d], dtype, st, GSPN_F32);
            });
            if (e != hipSuccess) return e;
        }
    } else {
        const hipError_t e = timed(tm, GSPN_STAGE_NORMALIZE, [&] {
            return gspn::launch_normalize_pair4(n, h, w, logits, wd, dtype, st);
        });
        if (e != hipSuccess) return e;
    }
    for (int d = 0; d < 4; ++d) {
        p[d].wts = wd[d];
        p[d].wts_are_logits = 0;
        p[d].wdtype = dtype == GSPN_F32 ? GSPN_F32 : gspn::kPairF16;
    }
    return hipSuccess;
}

// GSPN_LAYOUT_ARRAY: copies the horizontal directions' logits and lambdas
// (array frame) into their scan frame at dst (layout_copy_bytes bytes) and
// points zl / ll at the copies (a lambda given for both horizontal
// directions is copied once).
hipError_t copy_to_scan_frame(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, const void* const logits[4],
                              const void* const lam[4], char* dst, int dtype, hipStream_t st, Timer* tm,
                              const void* (&zl)[4], const void* (&ll)[4]) {
    const int64_t es = static_cast<int64_t>(elem_size(dtype));
    const int64_t wb = n * cw * 3 * h * w * es;
    const int64_t lb = n * c * h * w * es;
    for (int d = 2; d < 4; ++d) {
        char* zt = dst + (d - 2) * wb;
        char* lt = dst + 2 * wb + (d - 2) * lb;
        hipError_t e = timed(tm, GSPN_STAGE_LAYOUT, [&] {
            return gspn::launch_transpose(logits[d], zt, n * cw * 3, static_cast<int>(h), static_cast<int>(w), dtype,
                                          st);
        });
        if (e != hipSuccess) return e;
        zl[d] = zt;
        if (d == 3 && lam[3] == lam[2]) {
            ll[d] = ll[2];
            continue;
        }
        e = timed(tm, GSPN_STAGE_LAYOUT, [&] {
            return gspn::launch_transpose(lam[d], lt, n * c, static_cast<int>(h), static_cast<int>(w), dtype, st);
        });
        if (e != hipSuccess) return e;
        ll[d] = lt;
    }
    return hipSuccess;
}

gspn_status forward4_impl(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk_len,
                          const void* x, const void* const logits_in[4], const void* const lam_in[4],
                          const float* merge, void* y, float* states, void* workspace, int64_t workspace_bytes,
                          int dtype, int layout, void* stream, Timer* tm, bool noalloc = false,
                          int64_t merge_ld = 0, int64_t states_ld = 0) {
    // noalloc: the workspace is the current device's static scratch array,
    // looked up only once every argument has passed validation.
    // merge_ld: floats between the merge weights' direction rows (0: c); more
    // than c only for the plane-sequential path's tail, a channel range of a
    // wider call, which takes the concurrent path and its transposing merge.
    // states_ld: floats between the four state maps (0: n c h w); more only
    // for that tail, whose maps are plane ranges of the wider call's.
    const int64_t mld = merge_ld > 0 ? merge_ld : c;
    const int64_t sel = states_ld > 0 ? states_ld : n * c * h * w;
    if (!valid_layout(layout)) return GSPN_ERR_BAD_LAYOUT;
    const void* const* logits = logits_in;
    const void* const* lam = lam_in;
    int64_t chunks[4];
    for (int d = 0; d < 4; ++d) {
        bool empty = false;
        const ScanCheck ck = check_scan(d, chunk_len, n, c, h, w, cw, dtype, &empty);
        if (ck.st != GSPN_OK || empty) return ck.st;
        chunks[d] = ck.chunk;
    }
    if (!x || !y || !logits || !lam) return GSPN_ERR_NULL_POINTER;
    for (int d = 0; d < 4; ++d)
        if (!logits[d] || !lam[d]) return GSPN_ERR_NULL_POINTER;
    const bool have_ws = noalloc || (workspace != nullptr && workspace_bytes > 0);
    if (layout == GSPN_LAYOUT_ARRAY && !have_ws) return GSPN_ERR_WORKSPACE;  // the copies live there
    const size_t es = elem_size(dtype);
    if (!aligned(x, es) || !aligned(y, es)) return GSPN_ERR_MISALIGNED;
    for (int d = 0; d < 4; ++d)
        if (!aligned(logits[d], es) || !aligned(lam[d], es)) return GSPN_ERR_MISALIGNED;
    const int64_t xb = n * c * h * w * static_cast<int64_t>(es);
    const int64_t wb = n * cw * 3 * h * w * static_cast<int64_t>(es);
    if (overlap(y, xb, x, xb)) return GSPN_ERR_ALIASING;
    for (int d = 0; d < 4; ++d)
        if (overlap(y, xb, logits[d], wb) || overlap(y, xb, lam[d], xb)) return GSPN_ERR_ALIASING;
    const int64_t mgb = (3 * mld + c) * 4;  // merge weights, fp32 [4][c], rows mld floats apart
    if (merge && !aligned(merge, 4)) return GSPN_ERR_MISALIGNED;
    if (merge && overlap(y, xb, merge, mgb)) return GSPN_ERR_ALIASING;
    const int64_t sb = (3 * sel + n * c * h * w) * 4;  // four fp32 state maps, sel floats apart
    if (states) {
        // the states come from the four-direction launch, which takes lines
        // of at most 2048 positions and a workspace (also for planes of at
        // most 64 x 64, whose plane-resident path keeps no states), or from
        // the plane-sequential kernel, which the same shapes allow
        if (!gspn::fused4_supported(h, w) || !fused_grid_ok(n, c, h, w, chunks)) return GSPN_ERR_UNSUPPORTED;
        if (!have_ws) return GSPN_ERR_WORKSPACE;
        if (!aligned(states, 4)) return GSPN_ERR_MISALIGNED;
        if (overlap(states, sb, y, xb) || overlap(states, sb, x, xb)) return GSPN_ERR_ALIASING;
        for (int d = 0; d < 4; ++d)
            if (overlap(states, sb, logits[d], wb) || overlap(states, sb, lam[d], xb)) return GSPN_ERR_ALIASING;
        if (merge && overlap(states, sb, merge, mgb)) return GSPN_ERR_ALIASING;
    }
    int64_t need = 0;
    if (noalloc) {
        need = gspn_forward4_workspace_bytes(n, c, h, w, cw, dtype, layout);
        if (need > GSPN_NOALLOC_SCRATCH_BYTES) return GSPN_ERR_WORKSPACE;
    } else if (have_ws) {
        need = gspn_forward4_workspace_bytes(n, c, h, w, cw, dtype, layout);
        if (workspace_bytes < need) return GSPN_ERR_WORKSPACE;
        if (!aligned(workspace, 4)) return GSPN_ERR_MISALIGNED;
        if (overlap(workspace, need, y, xb) || overlap(workspace, need, x, xb)) return GSPN_ERR_ALIASING;
        if (merge && overlap(workspace, need, merge, mgb)) return GSPN_ERR_ALIASING;
        if (states && overlap(workspace, need, states, sb)) return GSPN_ERR_ALIASING;
        for (int d = 0; d < 4; ++d)
            if (overlap(workspace, need, logits[d], wb) || overlap(workspace, need, lam[d], xb))
                return GSPN_ERR_ALIASING;
    }
    if (noalloc) {
        // the scratch is a separate device allocation: it overlaps no argument
        if (gspn::noalloc_scratch(&workspace) != hipSuccess) return GSPN_ERR_HIP;
        workspace_bytes = need;
    }
    const hipStream_t st = as_stream(stream);

    // the per-direction tensors in their scan frames
    const void* zl[4] = {logits[0], logits[1], logits[2], logits[3]};
    const void* ll[4] = {lam[0], lam[1], lam[2], lam[3]};
    if (layout == GSPN_LAYOUT_ARRAY) {
        char* dst = static_cast<char*>(workspace) + need - layout_copy_bytes(n, c, h, w, cw, dtype);
        if (copy_to_scan_frame(n, c, h, w, cw, logits, lam, dst, dtype, st, tm, zl, ll) != hipSuccess)
            return GSPN_ERR_HIP;
    }
    logits = zl;
    lam = ll;

    gspn::ScanParams p[4];
    for (int d = 0; d < 4; ++d) {
        p[d].x = x;
        p[d].wts = logits[d];
        p[d].lam = lam[d];
        p[d].out = y;
        p[d].n = n;
        p[d].c = c;
        p[d].cw = cw;
        p[d].h = h;
        p[d].w = w;
        p[d].dir = d;
        p[d].chunk = chunks[d];
        p[d].wts_are_logits = 1;
        p[d].accumulate = 0;
        p[d].dtype = dtype;
        p[d].wdtype = dtype;
        p[d].mscale = merge ? merge + d * mld : nullptr;
    }

    // Planes of at most 64 x 64: one pass over LDS-resident planes, whether
    // or not a workspace is given (unless the states are wanted).
    if (gspn::plane4_supported(h, w) && !states && (!merge || mld == c)) {
        if (tm) tm->scan_kernel = GSPN_SCAN_PLANE;
        return from_hip(timed(tm, GSPN_STAGE_SCAN, [&] {
            return gspn::launch_plane4(x, logits, lam, merge, y, n, c, cw, h, w, chunks, dtype, st);
        }));
    }

    if (!have_ws) {
        // No workspace: one direction per launch; the first writes y, the
        // others add to it; horizontal lines use per-lane row tiles.
        if (tm) tm->scan_kernel = GSPN_SCAN_PER_DIRECTION;
        for (int d = 0; d < 4; ++d) {
            p[d].accumulate = d > 0 ? 1 : 0;
            if (timed(tm, GSPN_STAGE_SCAN, [&] { return gspn::launch_scan(p[d], st); }) != hipSuccess)
                return GSPN_ERR_HIP;
        }
        return GSPN_OK;
    }

    // Workspace layout: [normalised weights of the four directions, only for
    // channel-shared weights over several channels][x transposed into the
    // horizontal scan frame][three output maps].
    char* ws = static_cast<char*>(workspace);
    const bool prenorm = cw == 1 && c > 1;
    const int64_t wdir = n * h * w * (dtype == GSPN_F32 ? 3 * 4 : 4);  // weight bytes per direction
    char* xt = ws + (prenorm ? 4 * wdir : 0);
    char* m1 = xt + xb;
    char* m2 = m1 + xb;
    char* m3 = m2 + xb;
    if (prenorm) {
        // One normalisation per position and direction, shared by all c
        // channels, so the scans run without transcendentals: fp32 triples
        // for fp32 storage; for bf16 storage packed half pairs (w_{k-1},
        // w_{k+1}) with the centre weight recovered as 1 minus their sum, a
        // third of the bytes every channel's scan reads (all four directions
        // in one launch).
        if (prenormalise(n, h, w, logits, ws, wdir, dtype, st, tm, p) != hipSuccess) return GSPN_ERR_HIP;
    }
    // Many big planes: one workgroup per plane runs the four directions in
    // turn and builds y in place; the scratch map of the horizontal
    // directions' sum takes the room of x transposed.  It also writes the
    // states (the fp32 h of every direction, unweighted), bit for bit those
    // of the four-direction launch.
    if (gspn::seq4_supported(h, w) && n * c >= gspn::kSeq4MinPlanes && (!merge || mld == c)) {
        bool vec = aligned(x, 16) && aligned(y, 16);
        for (int d = 0; d < 4; ++d) vec = vec && aligned(p[d].wts, 16) && aligned(p[d].lam, 16);
        if (vec) {
            // With one workgroup per CU, planes run in rounds of one per CU,
            // each a chain of four whole scans.  A last round at most half
            // full would cost a whole round's time for half its work, so
            // those planes (when they lie in one image) go to the concurrent
            // four-direction path instead, which spreads each plane over four
            // workgroups; its merge weights are those of the tail's channels.
            const int64_t planes = n * c;
            const int64_t cus = gspn::device_compute_units();
            const int64_t tail = cus > 0 ? planes % cus : 0;
            const bool split = planes > cus && tail > 0 && 2 * tail <= cus && mld == c &&
                               (planes - tail) / c == (planes - 1) / c;
            const int64_t run = split ? planes - tail : planes;
            const void* wts[4] = {p[0].wts, p[1].wts, p[2].wts, p[3].wts};
            if (timed(tm, GSPN_STAGE_SCAN, [&] {
                    return gspn::launch_seq4(x, wts, lam, merge, y, xt, n, c, cw, h, w, chunks, dtype, p[0].wdtype,
                                             p[0].wts_are_logits, run, states, sel, st);
                }) != hipSuccess)
                return GSPN_ERR_HIP;
            if (split) {
                // the tail: channels c0 .. c - 1 of image n0, a forward of
                // its own in the scan frame (the logits and lambdas there
                // already), in the workspace after the launch above is done
                // with it (same stream)
                const int64_t n0 = run / c, c0 = run % c;
                const int64_t plane_b = h * w * static_cast<int64_t>(es);
                const void* tz[4];
                const void* tl[4];
                for (int d = 0; d < 4; ++d) {
                    tz[d] = static_cast<const char*>(logits[d]) + (n0 * cw + (cw == 1 ? 0 : c0)) * 3 * plane_b;
                    tl[d] = static_cast<const char*>(lam[d]) + run * plane_b;
                }
                gspn_status sub = GSPN_OK;
                const hipError_t e = timed(tm, GSPN_STAGE_TAIL, [&] {
                    sub = forward4_impl(1, tail, h, w, cw == 1 ? 1 : tail, chunk_len,
                                        static_cast<const char*>(x) + run * plane_b, tz, tl,
                                        merge ? merge + c0 : nullptr, static_cast<char*>(y) + run * plane_b,
                                        states ? states + run * h * w : nullptr, workspace, workspace_bytes,
                                        dtype, GSPN_LAYOUT_SCAN, stream, nullptr, false, c, sel);
                    return sub == GSPN_OK ? hipSuccess : hipErrorLaunchFailure;
                });
                if (sub != GSPN_OK) return sub;
                if (e != hipSuccess) return GSPN_ERR_HIP;
            }
            if (tm) tm->scan_kernel = GSPN_SCAN_SEQUENTIAL;
            return GSPN_OK;
        }
    }

    // The horizontal directions become vertical-form scans in their scan
    // frame, where line k of step i is x[.., k, i]: of x transposed, or,
    // where the long-line kernel takes them (lp_xtile_supported), of x itself
    // read through LDS column tiles, so that no transposed copy is made.
    for (int d = 2; d < 4; ++d) {
        p[d].h = w;
        p[d].w = h;
        p[d].dir = d - 2;  // L2R runs like T2B, R2L like B2T, in the transposed frame
    }
    bool xtile = false;
    if (xtile_enabled() && gspn::fused4_supported(h, w) && fused_grid_ok(n, c, h, w, chunks)) {
        gspn::ScanParams q[4] = {p[0], p[1], p[2], p[3]};
        // the outputs and merge handling of the paths below
        for (int d = 0; d < 4; ++d) {
            q[d].mscale = nullptr;
            if (states) {
                q[d].out = states + d * sel;
                q[d].odtype = GSPN_F32;
            }
        }
        if (!states) {
            q[1].out = m1;
            q[2].out = m2;
            q[3].out = m3;
        }
        q[2].xtile = q[3].xtile = 1;
        xtile = gspn::lp_xtile_supported(q);
    }
    if (xtile) {
        p[2].xtile = p[3].xtile = 1;
    } else {
        if (timed(tm, GSPN_STAGE_TRANSPOSE, [&] {
                return gspn::launch_transpose(x, xt, n * c, static_cast<int>(h), static_cast<int>(w), dtype, st);
            }) != hipSuccess)
            return GSPN_ERR_HIP;
        p[2].x = p[3].x = xt;
    }

    // With the states wanted: the four directions in one launch, each into
    // its fp32 state map, then y merged from those maps.
    if (states) {
        for (int d = 0; d < 4; ++d) {
            p[d].out = states + d * sel;
            p[d].odtype = GSPN_F32;
            p[d].mscale = nullptr;  // the merge below applies the merge weights
        }
        const int nbands = state_bands(p, n, c, h, w);
        if (nbands > 0) {
            float* state = reinterpret_cast<float*>(ws + ((prenorm ? 4 * wdir : 0) + 4 * xb + 3) / 4 * 4);
            for (int b = 0; b < nbands; ++b)
                if (timed(tm, GSPN_STAGE_SCAN, [&] { return gspn::launch_scan4_band(p, state, b, st); }) !=
                    hipSuccess)
                    return GSPN_ERR_HIP;
            if (tm) tm->scan_kernel = GSPN_SCAN_BANDED;
        } else {
            int kind = GSPN_SCAN_FUSED4;
            if (timed(tm, GSPN_STAGE_SCAN, [&] { return gspn::launch_scan4v(p, st, &kind); }) != hipSuccess)
                return GSPN_ERR_HIP;
            if (tm) tm->scan_kernel = kind;
        }
        return from_hip(timed(tm, GSPN_STAGE_COMBINE, [&] {
            return gspn::launch_combine_states(y, states, states + sel, states + 2 * sel, states + 3 * sel,
                                               n * c, static_cast<int>(h), static_cast<int>(w), dtype, st, merge,
                                               c, mld);
        }));
    }

    // Concurrent path: the four directions in one launch, each into its own
    // map (lines up to 2048 positions); very few long lines instead run split
    // across workgroups, one launch per band of steps.
    if (gspn::fused4_supported(h, w) && fused_grid_ok(n, c, h, w, chunks)) {
        p[1].out = m1;
        p[2].out = m2;
        p[3].out = m3;
        for (int d = 0; d < 4; ++d) p[d].mscale = nullptr;  // the transposing merge applies the merge weights
        const int nbands = gspn::band_launches(p);
        if (nbands > 0) {
            float* state = reinterpret_cast<float*>(ws + ((prenorm ? 4 * wdir : 0) + 4 * xb + 3) / 4 * 4);
            for (int b = 0; b < nbands; ++b)
                if (timed(tm, GSPN_STAGE_SCAN, [&] { return gspn::launch_scan4_band(p, state, b, st); }) !=
                    hipSuccess)
                    return GSPN_ERR_HIP;
            if (tm) tm->scan_kernel = GSPN_SCAN_BANDED;
        } else {
            int kind = GSPN_SCAN_FUSED4;
            if (timed(tm, GSPN_STAGE_SCAN, [&] { return gspn::launch_scan4v(p, st, &kind); }) != hipSuccess)
                return GSPN_ERR_HIP;
            if (tm) tm->scan_kernel = kind;
        }
        return from_hip(timed(tm, GSPN_STAGE_COMBINE, [&] {
            return gspn::launch_combine(y, m1, m2, m3, n * c, static_cast<int>(h), static_cast<int>(w), 1, dtype,
                                        st, merge, c, mld);
        }));
    }
    // Longer lines, sequential path: T2B writes y, B2T adds to it; L2R writes
    // the transposed map, R2L adds to it; a transposing merge adds that into y.
    if (tm) tm->scan_kernel = GSPN_SCAN_PER_DIRECTION;
    p[1].accumulate = 1;
    p[2].out = m1;
    p[3].out = m1;
    p[3].accumulate = 1;
    for (int d = 0; d < 4; ++d)
        if (timed(tm, GSPN_STAGE_SCAN, [&] { return gspn::launch_scan(p[d], st); }) != hipSuccess)
            return GSPN_ERR_HIP;
    return from_hip(timed(tm, GSPN_STAGE_COMBINE, [&] {
        return gspn::launch_combine(y, nullptr, m1, nullptr, n * c, static_cast<int>(h), static_cast<int>(w), 1,
                                    dtype, st);
    }));
}

// The proxy-space state a compressive-proxy forward keeps for its backward:
// x_p, y_p (storage type) and, for planes larger than 64 x 64, the four
// directions' fp32 scans; offsets in bytes, parts rounded up to 256 bytes.
struct ProxyStates {
    int64_t xp, yp, scans, total;
    bool has_scans;
};

bool proxy_states_layout(int64_t n, int64_t c_proxy, int64_t h, int64_t w, int dtype, ProxyStates* K) {
    if (!valid_dtype(dtype) || !dims_ok({n, c_proxy, h, w}) || c_proxy < 1) return false;
    const int64_t e = checked_product({n, c_proxy, h, w});
    if (e < 0 || e > (INT64_MAX / 64)) return false;
    const int64_t pb = (e * static_cast<int64_t>(elem_size(dtype)) + 255) / 256 * 256;
    K->xp = 0;
    K->yp = pb;
    K->scans = 2 * pb;
    K->has_scans = !gspn::plane4_supported(h, w);
    K->total = K->scans + (K->has_scans ? 16 * e : 0);
    return true;
}

gspn_status proxy_impl(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw, int64_t chunk_len,
                       const void* x, const void* w_down, const void* w_up, const void* const logits[4],
                       const void* const lam[4], const float* merge, void* y, void* keep, void* workspace,
                       int64_t workspace_bytes, int dtype, int layout, void* stream, Timer* tm) {
    if (!valid_dtype(dtype)) return GSPN_ERR_BAD_DTYPE;
    if (!valid_layout(layout)) return GSPN_ERR_BAD_LAYOUT;
    if (!dims_ok({n, c, h, w}) || !dims_ok({n, c_proxy, h, w})) return GSPN_ERR_BAD_SHAPE;
    if (chunk_len < 0) return GSPN_ERR_BAD_CHUNK;
    if (!(cw == 1 || cw == c_proxy)) return GSPN_ERR_BAD_WEIGHT_CHANNELS;
    if (checked_product({n, c, h, w}) == 0) return GSPN_OK;
    if (c_proxy < 1) return GSPN_ERR_BAD_SHAPE;
    if (h > GSPN_MAX_LINE || w > GSPN_MAX_LINE) return GSPN_ERR_UNSUPPORTED;
    if (!x || !w_down || !w_up || !y || !logits || !lam || !workspace) return GSPN_ERR_NULL_POINTER;
    for (int d = 0; d < 4; ++d)
        if (!logits[d] || !lam[d]) return GSPN_ERR_NULL_POINTER;
    const size_t es = elem_size(dtype);
    if (!aligned(x, es) || !aligned(y, es) || !aligned(w_down, es) || !aligned(w_up, es))
        return GSPN_ERR_MISALIGNED;
    const int64_t need = gspn_proxy_forward4_workspace_bytes(n, c, h, w, c_proxy, cw, dtype, layout);
    if (workspace_bytes < need) return GSPN_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return GSPN_ERR_MISALIGNED;
    const int64_t xb = n * c * h * w * static_cast<int64_t>(es);
    const int64_t pb = n * c_proxy * h * w * static_cast<int64_t>(es);
    const int64_t wb = n * cw * 3 * h * w * static_cast<int64_t>(es);
    const int64_t mb = c * c_proxy * static_cast<int64_t>(es);
    if (overlap(y, xb, x, xb) || overlap(y, xb, w_down, mb) || overlap(y, xb, w_up, mb)) return GSPN_ERR_ALIASING;
    if (overlap(workspace, need, x, xb) || overlap(workspace, need, y, xb) ||
        overlap(workspace, need, w_down, mb) || overlap(workspace, need, w_up, mb))
        return GSPN_ERR_ALIASING;
    const int64_t mgb = 4 * c_proxy * 4;  // merge weights over the proxy channels, fp32 [4][c_proxy]
    if (merge && !aligned(merge, 4)) return GSPN_ERR_MISALIGNED;
    if (merge && (overlap(y, xb, merge, mgb) || overlap(workspace, need, merge, mgb))) return GSPN_ERR_ALIASING;
    for (int d = 0; d < 4; ++d) {
        if (!aligned(logits[d], es) || !aligned(lam[d], es)) return GSPN_ERR_MISALIGNED;
        if (overlap(y, xb, logits[d], wb) || overlap(y, xb, lam[d], pb) ||
            overlap(workspace, need, logits[d], wb) || overlap(workspace, need, lam[d], pb))
            return GSPN_ERR_ALIASING;
    }
    ProxyStates K;
    if (keep) {
        if (!proxy_states_layout(n, c_proxy, h, w, dtype, &K)) return GSPN_ERR_BAD_SHAPE;
        if (!aligned(keep, 256)) return GSPN_ERR_MISALIGNED;
        const int64_t kb = K.total;
        if (overlap(keep, kb, x, xb) || overlap(keep, kb, y, xb) || overlap(keep, kb, w_down, mb) ||
            overlap(keep, kb, w_up, mb) || overlap(keep, kb, workspace, need) ||
            (merge && overlap(keep, kb, merge, mgb)))
            return GSPN_ERR_ALIASING;
        for (int d = 0; d < 4; ++d)
            if (overlap(keep, kb, logits[d], wb) || overlap(keep, kb, lam[d], pb)) return GSPN_ERR_ALIASING;
    }
    char* ws = static_cast<char*>(workspace);
    // x_p and y_p in the workspace, or where the caller keeps them
    char* kp = static_cast<char*>(keep);
    void* xp = keep ? kp + K.xp : ws;
    void* yp = keep ? kp + K.yp : ws + pb;
    float* scans = keep && K.has_scans ? reinterpret_cast<float*>(kp + K.scans) : nullptr;
    char* fws = ws + 2 * pb;
    const hipStream_t st = as_stream(stream);
    if (timed(tm, GSPN_STAGE_PROJECT_DOWN,
              [&] { return gspn::launch_project(n, c, h * w, c_proxy, x, w_down, xp, dtype, st); }) != hipSuccess)
        return GSPN_ERR_HIP;
    const gspn_status s4 = forward4_impl(n, c_proxy, h, w, cw, chunk_len, xp, logits, lam, merge, yp, scans, fws,
                                         need - 2 * pb, dtype, layout, stream, tm);
    if (s4 != GSPN_OK) return s4;
    return from_hip(timed(tm, GSPN_STAGE_PROJECT_UP,
                          [&] { return gspn::launch_project(n, c_proxy, h * w, c, yp, w_up, y, dtype, st); }));
}

gspn_status backward_impl(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk_len, const void* x,
                          const void* const logits_in[4], const void* const lam_in[4], const float* merge,
                          const float* states, const void* gy, void* dx, void* const dlogits_in[4],
                          void* const dlam_in[4], float* dmerge, void* workspace, int64_t workspace_bytes, int dtype,
                          int layout, void* stream, Timer* tm) {
    if (!valid_layout(layout)) return GSPN_ERR_BAD_LAYOUT;
    const void* const* logits = logits_in;
    const void* const* lam = lam_in;
    void* const* dlogits = dlogits_in;
    void* const* dlam = dlam_in;
    int64_t chunks[4];
    for (int d = 0; d < 4; ++d) {
        bool empty = false;
        const ScanCheck ck = check_scan(d, chunk_len, n, c, h, w, cw, dtype, &empty);
        if (ck.st != GSPN_OK || empty) return ck.st;
        chunks[d] = ck.chunk;
    }
    if (!gspn::fused4_supported(h, w) || !fused_grid_ok(n, c, h, w, chunks)) return GSPN_ERR_UNSUPPORTED;
    if (!x || !gy || !dx || !logits || !lam || !dlogits || !dlam || !workspace) return GSPN_ERR_NULL_POINTER;
    for (int d = 0; d < 4; ++d)
        if (!logits[d] || !lam[d] || !dlogits[d] || !dlam[d]) return GSPN_ERR_NULL_POINTER;
    const size_t es = elem_size(dtype);
    const int64_t hb = n * c * h * w * 4;  // bytes of one fp32 state map
    // given the states, the workspace's last part (room for them) is not needed
    const int64_t need = gspn_backward4_workspace_bytes(n, c, h, w, cw, dtype, layout) - (states ? 4 * hb : 0);
    if (workspace_bytes < need) return GSPN_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return GSPN_ERR_MISALIGNED;
    if (!aligned(x, es) || !aligned(gy, es) || !aligned(dx, es)) return GSPN_ERR_MISALIGNED;
    const int64_t xb = n * c * h * w * static_cast<int64_t>(es);
    const int64_t wb = n * cw * 3 * h * w * static_cast<int64_t>(es);
    // outputs: dx, dlam[4], dlogits[4]; none may overlap an input, the
    // workspace or another output
    const void* outs[9] = {dx, dlam[0], dlam[1], dlam[2], dlam[3], dlogits[0], dlogits[1], dlogits[2], dlogits[3]};
    const int64_t ob[9] = {xb, xb, xb, xb, xb, wb, wb, wb, wb};
    for (int i = 0; i < 9; ++i) {
        if (!aligned(outs[i], es)) return GSPN_ERR_MISALIGNED;
        if (overlap(outs[i], ob[i], x, xb) || overlap(outs[i], ob[i], gy, xb) ||
            overlap(outs[i], ob[i], workspace, need))
            return GSPN_ERR_ALIASING;
        for (int d = 0; d < 4; ++d)
            if (overlap(outs[i], ob[i], logits[d], wb) || overlap(outs[i], ob[i], lam[d], xb)) return GSPN_ERR_ALIASING;
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], ob[i], outs[j], ob[j])) return GSPN_ERR_ALIASING;
    }
    for (int d = 0; d < 4; ++d) {
        if (!aligned(logits[d], es) || !aligned(lam[d], es)) return GSPN_ERR_MISALIGNED;
        if (overlap(workspace, need, logits[d], wb) || overlap(workspace, need, lam[d], xb))
            return GSPN_ERR_ALIASING;
    }
    if (overlap(workspace, need, x, xb) || overlap(workspace, need, gy, xb)) return GSPN_ERR_ALIASING;
    if (states) {
        if (!aligned(states, 4)) return GSPN_ERR_MISALIGNED;
        if (overlap(workspace, need, states, 4 * hb)) return GSPN_ERR_ALIASING;
        for (int i = 0; i < 9; ++i)
            if (overlap(outs[i], ob[i], states, 4 * hb)) return GSPN_ERR_ALIASING;
        if (dmerge && overlap(dmerge, 4 * c * 4, states, 4 * hb)) return GSPN_ERR_ALIASING;
    }
    const int64_t mgb = 4 * c * 4;  // merge weights and their gradient, fp32 [4][c]
    if ((merge && !aligned(merge, 4)) || (dmerge && !aligned(dmerge, 4))) return GSPN_ERR_MISALIGNED;
    if (merge) {
        if (overlap(workspace, need, merge, mgb)) return GSPN_ERR_ALIASING;
        for (int i = 0; i < 9; ++i)
            if (overlap(outs[i], ob[i], merge, mgb)) return GSPN_ERR_ALIASING;
    }
    if (dmerge) {
        if (overlap(dmerge, mgb, x, xb) || overlap(dmerge, mgb, gy, xb) || overlap(dmerge, mgb, workspace, need) ||
            (merge && overlap(dmerge, mgb, merge, mgb)))
            return GSPN_ERR_ALIASING;
        for (int d = 0; d < 4; ++d)
            if (overlap(dmerge, mgb, logits[d], wb) || overlap(dmerge, mgb, lam[d], xb)) return GSPN_ERR_ALIASING;
        for (int i = 0; i < 9; ++i)
            if (overlap(dmerge, mgb, outs[i], ob[i])) return GSPN_ERR_ALIASING;
    }
    const hipStream_t st = as_stream(stream);

    // Workspace: [fp32 logit-gradient sums and normalised weights of the four
    // directions (shared logits only)][x^T][gy^T][dx terms D1..D3][fp32
    // forward states H0..H3, unless the caller passes them].
    // The states stay fp32 for bf16 storage too: the logit gradient takes
    // differences of neighbouring states, which bf16 rounding would swamp.
    const bool shared = cw == 1 && c > 1;
    const int64_t zsum = 3 * n * h * w;  // floats per direction
    char* ws = static_cast<char*>(workspace);
    float* sums = reinterpret_cast<float*>(ws);
    const int64_t wdir = n * h * w * (dtype == GSPN_F32 ? 3 * 4 : 4);  // normalised weight bytes per direction
    char* wnorm = ws + 4 * zsum * 4;
    char* xt = ws + (shared ? 4 * zsum * 4 + 4 * wdir : 0);
    char* gt = xt + xb;
    char* dterm[4];
    dterm[0] = static_cast<char*>(dx);
    dterm[1] = gt + xb;
    dterm[2] = dterm[1] + xb;
    dterm[3] = dterm[2] + xb;
    // after the five storage-type maps, rounded up to 4 bytes (the sums and
    // weights before them are whole floats): for GSPN_LAYOUT_ARRAY the
    // scan-frame copies of the horizontal inputs, then room for the
    // horizontal gradients in their scan frame; last, the recomputed states
    char* hs[4];
    const int64_t loff = ((dterm[3] - ws) + xb + 3) / 4 * 4;
    const int64_t lc = layout == GSPN_LAYOUT_ARRAY ? layout_copy_bytes(n, c, h, w, cw, dtype) : 0;
    float* qband = reinterpret_cast<float*>(ws + loff + 2 * lc);  // the banded adjoint's products
    const int64_t hoff = loff + 2 * lc + adjoint_band_bytes(n, c, h, w);
    hs[0] = states ? reinterpret_cast<char*>(const_cast<float*>(states)) : ws + hoff;
    for (int d = 1; d < 4; ++d) hs[d] = hs[d - 1] + hb;
    const int H = static_cast<int>(h);
    const int W = static_cast<int>(w);

    // GSPN_LAYOUT_ARRAY: inputs copied into their scan frame; the horizontal
    // gradients are computed in the scan frame and copied out at the end
    const void* zl[4] = {logits[0], logits[1], logits[2], logits[3]};
    const void* ll[4] = {lam[0], lam[1], lam[2], lam[3]};
    void* dzl[4] = {dlogits[0], dlogits[1], dlogits[2], dlogits[3]};
    void* dll[4] = {dlam[0], dlam[1], dlam[2], dlam[3]};
    if (layout == GSPN_LAYOUT_ARRAY) {
        if (copy_to_scan_frame(n, c, h, w, cw, logits, lam, ws + loff, dtype, st, tm, zl, ll) != hipSuccess)
            return GSPN_ERR_HIP;
        char* gdst = ws + loff + lc;
        for (int d = 2; d < 4; ++d) {
            dzl[d] = gdst + (d - 2) * wb;
            dll[d] = gdst + 2 * wb + (d - 2) * xb;
        }
    }
    logits = zl;
    lam = ll;
    dlogits = dzl;
    dlam = dll;
    // copies the horizontal gradients out into the caller's array-frame buffers
    auto copy_out = [&]() -> gspn_status {
        if (layout != GSPN_LAYOUT_ARRAY) return GSPN_OK;
        for (int d = 2; d < 4; ++d) {
            if (timed(tm, GSPN_STAGE_LAYOUT, [&] {
                    return gspn::launch_transpose(dzl[d], dlogits_in[d], n * cw * 3, W, H, dtype, st);
                }) != hipSuccess ||
                timed(tm, GSPN_STAGE_LAYOUT, [&] {
                    return gspn::launch_transpose(dll[d], dlam_in[d], n * c, W, H, dtype, st);
                }) != hipSuccess)
                return GSPN_ERR_HIP;
        }
        return GSPN_OK;
    };

    // Planes of at most 64 x 64 (recomputed states only): one launch over
    // LDS-resident planes recomputes the four directions' states into the
    // workspace and runs their adjoints on them, x, gy and dx in the array
    // frame: no transposes and no per-direction dx terms.
    if (gspn::plane4_supported(h, w) && !states) {
        if (shared &&
            timed(tm, GSPN_STAGE_REDUCE, [&] { return gspn::launch_fill_zero(sums, 4 * zsum, st); }) != hipSuccess)
            return GSPN_ERR_HIP;
        if (dmerge &&
            timed(tm, GSPN_STAGE_REDUCE, [&] { return gspn::launch_fill_zero(dmerge, 4 * c, st); }) != hipSuccess)
            return GSPN_ERR_HIP;
        float* hf[4];
        for (int d = 0; d < 4; ++d) hf[d] = reinterpret_cast<float*>(hs[d]);
        if (tm) tm->scan_kernel = GSPN_SCAN_PLANE;  // the plane-resident forward, inside the adjoint launch
        gspn::AdjPlaneParams ap;
        ap.x = x;
        ap.g = gy;
        for (int d = 0; d < 4; ++d) {
            ap.z[d] = logits[d];
            ap.lam[d] = lam[d];
            ap.hs[d] = hf[d];
            ap.dlam[d] = dlam[d];
            ap.dz[d] = shared ? static_cast<void*>(sums + d * zsum) : dlogits[d];
            ap.chunk[d] = chunks[d];
        }
        ap.dx = dx;
        ap.merge = merge;
        ap.dmerge = dmerge;
        ap.n = n;
        ap.c = c;
        ap.cw = cw;
        ap.h = h;
        ap.w = w;
        ap.shared = shared ? 1 : 0;
        ap.dtype = dtype;
        if (timed(tm, GSPN_STAGE_ADJOINT, [&] { return gspn::launch_adjplane(ap, st); }) != hipSuccess)
            return GSPN_ERR_HIP;
        if (tm) tm->adjoint = {2, 1, 1, 0};  // one lane per position, one plane per workgroup
        if (shared) {
            for (int d = 0; d < 4; ++d)
                if (timed(tm, GSPN_STAGE_REDUCE, [&] {
                        return gspn::launch_finish_shared_dz(sums + d * zsum, logits[d], dlogits[d], n,
                                                             d < 2 ? h : w, d < 2 ? w : h, dtype, st);
                    }) != hipSuccess)
                    return GSPN_ERR_HIP;
        }
        return copy_out();
    }

    if (timed(tm, GSPN_STAGE_TRANSPOSE, [&] { return gspn::launch_transpose(x, xt, n * c, H, W, dtype, st); }) !=
            hipSuccess ||
        timed(tm, GSPN_STAGE_TRANSPOSE, [&] { return gspn::launch_transpose(gy, gt, n * c, H, W, dtype, st); }) !=
            hipSuccess)
        return GSPN_ERR_HIP;

    // forward states of every direction (vertical form; horizontal in the
    // transposed frame)
    gspn::ScanParams p[4];
    for (int d = 0; d < 4; ++d) {
        const bool hz = horizontal(d);
        p[d].x = hz ? static_cast<const void*>(xt) : x;
        p[d].wts = logits[d];
        p[d].lam = lam[d];
        p[d].out = hs[d];
        p[d].n = n;
        p[d].c = c;
        p[d].cw = cw;
        p[d].h = hz ? w : h;
        p[d].w = hz ? h : w;
        p[d].dir = hz ? d - 2 : d;
        p[d].chunk = chunks[d];
        p[d].wts_are_logits = 1;
        p[d].accumulate = 0;
        p[d].dtype = dtype;
        p[d].wdtype = dtype;
        p[d].odtype = GSPN_F32;
    }
    if (!states) {
        // channel-shared logits: normalised once, as in the forward
        if (shared && prenormalise(n, h, w, logits, wnorm, wdir, dtype, st, tm, p) != hipSuccess)
            return GSPN_ERR_HIP;
        // very few long lines: the banded forward, its band-border states in
        // the banded adjoint's scratch (free until the adjoint runs)
        const int nbands = state_bands(p, n, c, h, w);
        if (nbands > 0) {
            for (int b = 0; b < nbands; ++b)
                if (timed(tm, GSPN_STAGE_SCAN, [&] { return gspn::launch_scan4_band(p, qband, b, st); }) !=
                    hipSuccess)
                    return GSPN_ERR_HIP;
            if (tm) tm->scan_kernel = GSPN_SCAN_BANDED;
        } else {
            int kind = GSPN_SCAN_FUSED4;
            if (timed(tm, GSPN_STAGE_SCAN, [&] { return gspn::launch_scan4v(p, st, &kind); }) != hipSuccess)
                return GSPN_ERR_HIP;
            if (tm) tm->scan_kernel = kind;
        }
    }
    if (shared &&
        timed(tm, GSPN_STAGE_REDUCE, [&] { return gspn::launch_fill_zero(sums, 4 * zsum, st); }) != hipSuccess)
        return GSPN_ERR_HIP;
    if (dmerge &&
        timed(tm, GSPN_STAGE_REDUCE, [&] { return gspn::launch_fill_zero(dmerge, 4 * c, st); }) != hipSuccess)
        return GSPN_ERR_HIP;

    gspn::AdjointParams a[4];
    for (int d = 0; d < 4; ++d) {
        const bool hz = horizontal(d);
        a[d].x = hz ? static_cast<const void*>(xt) : x;
        a[d].g = hz ? static_cast<const void*>(gt) : gy;
        a[d].lam = lam[d];
        a[d].logits = logits[d];
        a[d].hs = hs[d];
        a[d].dlam = dlam[d];
        a[d].dz = shared ? static_cast<void*>(sums + d * zsum) : dlogits[d];
        a[d].dx = dterm[d];
        a[d].n = n;
        a[d].c = c;
        a[d].cw = cw;
        a[d].S = hz ? w : h;
        a[d].L = hz ? h : w;
        a[d].chunk = chunks[d];
        a[d].reverse = (d == GSPN_B2T || d == GSPN_R2L) ? 1 : 0;
        a[d].shared = shared ? 1 : 0;
        a[d].dtype = dtype;
        // the states above are those of the unweighted scans; the adjoint
        // applies the merge weights
        a[d].mscale = merge ? merge + d * c : nullptr;
        a[d].dmerge = dmerge ? dmerge + d * c : nullptr;
    }
    const int bands = adjoint_band_bytes(n, c, h, w) > 0 ? gspn::adjoint_band_launches(a) : 0;
    if (bands > 0) {
        for (int b = 0; b < bands; ++b)
            if (timed(tm, GSPN_STAGE_ADJOINT, [&] { return gspn::launch_adjoint4_band(a, qband, b, st); }) !=
                hipSuccess)
                return GSPN_ERR_HIP;
        const bool nt = (h * static_cast<int64_t>(es)) % 128 == 0 && (w * static_cast<int64_t>(es)) % 128 == 0;
        if (tm) tm->adjoint = {3, 2, 1, nt ? 1 : 0};
    } else {
        gspn::AdjointPlan plan{};
        if (timed(tm, GSPN_STAGE_ADJOINT, [&] { return gspn::launch_adjoint4(a, st, &plan); }) != hipSuccess)
            return GSPN_ERR_HIP;
        if (tm) tm->adjoint = {1, plan.positions, plan.group, plan.nontemporal};
    }
    // dx = ((D2^T + D3^T) + D0) + D1, D0 written into dx directly
    if (timed(tm, GSPN_STAGE_COMBINE, [&] {
            return gspn::launch_combine(dx, dterm[1], dterm[2], dterm[3], n * c, H, W, 1, dtype, st);
        }) != hipSuccess)
        return GSPN_ERR_HIP;
    if (shared) {
        for (int d = 0; d < 4; ++d)
            if (timed(tm, GSPN_STAGE_REDUCE, [&] {
                    return gspn::launch_finish_shared_dz(sums + d * zsum, logits[d], dlogits[d], n,
                                                         d < 2 ? h : w, d < 2 ? w : h, dtype, st);
                }) != hipSuccess)
                return GSPN_ERR_HIP;
    }
    return copy_out();
}

// Workspace of the proxy backward: x_p, y_p, dL/dy_p and dx_p in the storage
// type, the two weights transposed, the weight-gradient partial sums, for
// planes larger than 64 x 64 the proxy-space forward's fp32 states (kept by
// the forward, read by the backward), then the larger of the proxy-space
// forward and backward workspaces (used one after the other); every part
// starts on a 256-byte boundary.
struct ProxyBwdLayout {
    int64_t xp, yp, gp, dxp, wtu, wtd, part, states, inner, inner_bytes, total;
    bool keep;  // the states are kept
};

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

bool proxy_bwd_layout(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw, int dtype,
                      int layout, ProxyBwdLayout* L) {
    if (!valid_dtype(dtype) || !valid_layout(layout) || !dims_ok({n, c, h, w}) || !dims_ok({n, c_proxy, h, w}) ||
        c < 1 || c_proxy < 1 || !(cw == 1 || cw == c_proxy))
        return false;
    const int64_t es = static_cast<int64_t>(elem_size(dtype));
    const int64_t pb = round256(checked_product({n, c_proxy, h, w}) * es);
    const int64_t mb = round256(checked_product({c, c_proxy}) * es);
    const int64_t f4 = gspn_forward4_workspace_bytes(n, c_proxy, h, w, cw, dtype, layout);
    const int64_t b4 = gspn_backward4_workspace_bytes(n, c_proxy, h, w, cw, dtype, layout);
    if (pb < 0 || mb < 0 || f4 < 0 || b4 < 0) return false;
    L->xp = 0;
    L->yp = pb;
    L->gp = 2 * pb;
    L->dxp = 3 * pb;
    L->wtu = 4 * pb;
    L->wtd = L->wtu + mb;
    L->part = L->wtd + mb;
    L->states = L->part + round256(gspn::wgrad_slots(n, h * w) * c * c_proxy * 4);
    // planes of at most 64 x 64 recompute their states inside the adjoint
    L->keep = !gspn::plane4_supported(h, w);
    const int64_t sb = L->keep ? 16 * checked_product({n, c_proxy, h, w}) : 0;
    L->inner = L->states + round256(sb);
    const int64_t b4s = b4 - sb;  // the backward given the states
    L->inner_bytes = f4 > b4s ? f4 : b4s;
    L->total = L->inner + L->inner_bytes;
    return true;
}

gspn_status proxy_backward_impl(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw,
                                int64_t chunk_len, const void* x, const void* w_down, const void* w_up,
                                const void* const logits[4], const void* const lam[4], const float* merge,
                                const void* kept, const void* gy, void* dx, float* dw_down, float* dw_up,
                                void* const dlogits[4], void* const dlam[4], float* dmerge, void* workspace,
                                int64_t workspace_bytes, int dtype, int layout, void* stream, Timer* tm) {
    if (!valid_dtype(dtype)) return GSPN_ERR_BAD_DTYPE;
    if (!valid_layout(layout)) return GSPN_ERR_BAD_LAYOUT;
    if (!dims_ok({n, c, h, w}) || !dims_ok({n, c_proxy, h, w}) || c < 1 || c_proxy < 1) return GSPN_ERR_BAD_SHAPE;
    if (chunk_len < 0) return GSPN_ERR_BAD_CHUNK;
    if (!(cw == 1 || cw == c_proxy)) return GSPN_ERR_BAD_WEIGHT_CHANNELS;
    if (h > GSPN_MAX_LINE || w > GSPN_MAX_LINE) return GSPN_ERR_UNSUPPORTED;
    const hipStream_t st = as_stream(stream);
    if (!dw_down || !dw_up) return GSPN_ERR_NULL_POINTER;
    if (checked_product({n, h, w}) == 0) {
        // no pixels: the sums over them are zero, every other output is empty
        const int64_t gb = c * c_proxy * 4;
        if (!aligned(dw_down, 4) || !aligned(dw_up, 4) || (dmerge && !aligned(dmerge, 4)))
            return GSPN_ERR_MISALIGNED;
        if (overlap(dw_down, gb, dw_up, gb) || (dmerge && (overlap(dmerge, 4 * c_proxy * 4, dw_down, gb) ||
                                                            overlap(dmerge, 4 * c_proxy * 4, dw_up, gb))))
            return GSPN_ERR_ALIASING;
        if (timed(tm, GSPN_STAGE_REDUCE, [&] { return gspn::launch_fill_zero(dw_down, c * c_proxy, st); }) !=
                hipSuccess ||
            timed(tm, GSPN_STAGE_REDUCE, [&] { return gspn::launch_fill_zero(dw_up, c * c_proxy, st); }) !=
                hipSuccess)
            return GSPN_ERR_HIP;
        if (dmerge && timed(tm, GSPN_STAGE_REDUCE, [&] { return gspn::launch_fill_zero(dmerge, 4 * c_proxy, st); }) !=
                          hipSuccess)
            return GSPN_ERR_HIP;
        return GSPN_OK;
    }
    if (!x || !w_down || !w_up || !gy || !dx || !logits || !lam || !dlogits || !dlam || !workspace)
        return GSPN_ERR_NULL_POINTER;
    for (int d = 0; d < 4; ++d)
        if (!logits[d] || !lam[d] || !dlogits[d] || !dlam[d]) return GSPN_ERR_NULL_POINTER;
    ProxyBwdLayout L;
    if (!proxy_bwd_layout(n, c, h, w, c_proxy, cw, dtype, layout, &L)) return GSPN_ERR_BAD_SHAPE;
    if (workspace_bytes < L.total) return GSPN_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return GSPN_ERR_MISALIGNED;
    const size_t es = elem_size(dtype);
    const int64_t xb = n * c * h * w * static_cast<int64_t>(es);
    const int64_t pb = n * c_proxy * h * w * static_cast<int64_t>(es);
    const int64_t wb = n * cw * 3 * h * w * static_cast<int64_t>(es);
    const int64_t mb = c * c_proxy * static_cast<int64_t>(es);
    const int64_t gb = c * c_proxy * 4;  // a weight gradient, fp32
    const int64_t mgb = 4 * c_proxy * 4;
    const int64_t need = L.total;
    // inputs and outputs: alignment, then no output may overlap an input,
    // the workspace or another output, and the workspace no input
    const void* outs[12] = {dx, dw_down, dw_up, dlogits[0], dlogits[1], dlogits[2], dlogits[3],
                            dlam[0], dlam[1], dlam[2], dlam[3], dmerge};
    const int64_t ob[12] = {xb, gb, gb, wb, wb, wb, wb, pb, pb, pb, pb, mgb};
    const size_t oa[12] = {es, 4, 4, es, es, es, es, es, es, es, es, 4};
    const void* all_in[13] = {x, w_down, w_up, gy, logits[0], logits[1], logits[2], logits[3],
                              lam[0], lam[1], lam[2], lam[3], merge};
    const int64_t ib[13] = {xb, mb, mb, xb, wb, wb, wb, wb, pb, pb, pb, pb, mgb};
    const size_t ia[13] = {es, es, es, es, es, es, es, es, es, es, es, es, 4};
    for (int i = 0; i < 12; ++i)
        if (outs[i] && !aligned(outs[i], oa[i])) return GSPN_ERR_MISALIGNED;
    for (int j = 0; j < 13; ++j)
        if (all_in[j] && !aligned(all_in[j], ia[j])) return GSPN_ERR_MISALIGNED;
    for (int i = 0; i < 12; ++i) {
        if (!outs[i]) continue;
        if (overlap(outs[i], ob[i], workspace, need)) return GSPN_ERR_ALIASING;
        for (int j = 0; j < 13; ++j)
            if (all_in[j] && overlap(outs[i], ob[i], all_in[j], ib[j])) return GSPN_ERR_ALIASING;
        for (int j = 0; j < i; ++j)
            if (outs[j] && overlap(outs[i], ob[i], outs[j], ob[j])) return GSPN_ERR_ALIASING;
    }
    for (int j = 0; j < 13; ++j)
        if (all_in[j] && overlap(workspace, need, all_in[j], ib[j])) return GSPN_ERR_ALIASING;
    ProxyStates K;
    if (kept) {
        // read only: it may overlap inputs, but no output nor the workspace
        if (!proxy_states_layout(n, c_proxy, h, w, dtype, &K)) return GSPN_ERR_BAD_SHAPE;
        if (!aligned(kept, 256)) return GSPN_ERR_MISALIGNED;
        if (overlap(kept, K.total, workspace, need)) return GSPN_ERR_ALIASING;
        for (int i = 0; i < 12; ++i)
            if (outs[i] && overlap(kept, K.total, outs[i], ob[i])) return GSPN_ERR_ALIASING;
    }
    const int64_t hw = h * w;
    // the proxy-space backward's limits, checked before anything is queued
    int64_t chunks[4];
    for (int d = 0; d < 4; ++d) {
        bool empty = false;
        const ScanCheck ck = check_scan(d, chunk_len, n, c_proxy, h, w, cw, dtype, &empty);
        if (ck.st != GSPN_OK) return ck.st;
        chunks[d] = ck.chunk;
    }
    if (!gspn::fused4_supported(h, w) || !fused_grid_ok(n, c_proxy, h, w, chunks)) return GSPN_ERR_UNSUPPORTED;
    char* ws = static_cast<char*>(workspace);
    const char* kp = static_cast<const char*>(kept);
    void* xp = kept ? const_cast<char*>(kp + K.xp) : ws + L.xp;
    void* yp = kept ? const_cast<char*>(kp + K.yp) : ws + L.yp;
    void* gp = ws + L.gp;
    void* dxp = ws + L.dxp;
    void* wtu = ws + L.wtu;  // w_up^T [c_proxy][c]
    void* wtd = ws + L.wtd;  // w_down^T [c][c_proxy]
    float* part = reinterpret_cast<float*>(ws + L.part);
    float* states = !L.keep ? nullptr
                    : kept  ? reinterpret_cast<float*>(const_cast<char*>(kp + K.scans))
                            : reinterpret_cast<float*>(ws + L.states);
    void* inner = ws + L.inner;
    // the weights transposed, for the projections the chain rule needs
    if (timed(tm, GSPN_STAGE_REDUCE, [&] {
            return gspn::launch_transpose(w_up, wtu, 1, static_cast<int>(c), static_cast<int>(c_proxy), dtype, st);
        }) != hipSuccess ||
        timed(tm, GSPN_STAGE_REDUCE, [&] {
            return gspn::launch_transpose(w_down, wtd, 1, static_cast<int>(c_proxy), static_cast<int>(c), dtype, st);
        }) != hipSuccess)
        return GSPN_ERR_HIP;
    // the forward's proxy-space input and output (and scans), recomputed
    // unless kept
    gspn_status s = GSPN_OK;
    if (!kept) {
        if (timed(tm, GSPN_STAGE_PROJECT_DOWN,
                  [&] { return gspn::launch_project(n, c, hw, c_proxy, x, w_down, xp, dtype, st); }) != hipSuccess)
            return GSPN_ERR_HIP;
        s = forward4_impl(n, c_proxy, h, w, cw, chunk_len, xp, logits, lam, merge, yp, states, inner, L.inner_bytes,
                          dtype, layout, stream, tm);
        if (s != GSPN_OK) return s;
    }
    // dL/dy_p = w_up^T gy, and in the same pass over gy the partial sums of
    // dL/dw_up[c][k] = sum gy[c] y_p[k]
    int64_t slots = 0;
    if (timed(tm, GSPN_STAGE_WEIGHT_GRAD, [&] {
            return gspn::launch_project_wgrad(n, c, hw, c_proxy, gy, yp, wtu, gp, part, dtype, st, &slots);
        }) != hipSuccess ||
        timed(tm, GSPN_STAGE_REDUCE,
              [&] { return gspn::launch_wgrad_reduce(part, slots, c, c_proxy, dw_up, c_proxy, 1, st); }) != hipSuccess)
        return GSPN_ERR_HIP;
    // the propagation's gradients in proxy space
    s = backward_impl(n, c_proxy, h, w, cw, chunk_len, xp, logits, lam, merge, states, gp, dxp, dlogits, dlam,
                      dmerge, inner, L.inner_bytes, dtype, layout, stream, tm);
    if (s != GSPN_OK) return s;
    // dx = w_down^T dx_p; dL/dw_down[k][c] = sum dx_p[k] x[c]
    if (timed(tm, GSPN_STAGE_PROJECT_UP,
              [&] { return gspn::launch_project(n, c_proxy, hw, c, dxp, wtd, dx, dtype, st); }) != hipSuccess)
        return GSPN_ERR_HIP;
    if (timed(tm, GSPN_STAGE_WEIGHT_GRAD, [&] {
            return gspn::launch_project_wgrad(n, c, hw, c_proxy, x, dxp, nullptr, nullptr, part, dtype, st, &slots);
        }) != hipSuccess ||
        timed(tm, GSPN_STAGE_REDUCE,
              [&] { return gspn::launch_wgrad_reduce(part, slots, c, c_proxy, dw_down, 1, c, st); }) != hipSuccess)
        return GSPN_ERR_HIP;
    return GSPN_OK;
}

}  // namespace

extern "C" {

gspn_status gspn_forward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                          int64_t chunk_len, const void* x, const void* const logits[4],
                          const void* const lam[4], const float* merge, void* y, float* states, void* workspace,
                          int64_t workspace_bytes, int dtype, int layout, void* stream) {
    return forward4_impl(n, c, h, w, cw, chunk_len, x, logits, lam, merge, y, states, workspace, workspace_bytes,
                         dtype, layout, stream, nullptr);
}

gspn_status gspn_forward4_timed(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                                int64_t chunk_len, const void* x, const void* const logits[4],
                                const void* const lam[4], const float* merge, void* y, float* states,
                                void* workspace, int64_t workspace_bytes, int dtype, int layout, void* stream,
                                gspn_stage_times* times) {
    if (!times) return GSPN_ERR_NULL_POINTER;
    Timer tm;
    tm.st = as_stream(stream);
    const gspn_status s = forward4_impl(n, c, h, w, cw, chunk_len, x, logits, lam, merge, y, states, workspace,
                                        workspace_bytes, dtype, layout, stream, &tm);
    const hipError_t e = tm.finish(times);
    return s != GSPN_OK ? s : from_hip(e);
}

static_assert(GSPN_NOALLOC_SCRATCH_BYTES == gspn::kNoallocScratchBytes, "scratch size stated in gspn.h");

gspn_status gspn_forward4_noalloc(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk_len,
                                  const void* x, const void* const logits[4], const void* const lam[4],
                                  const float* merge, void* y, float* states, int dtype, int layout, void* stream) {
    return forward4_impl(n, c, h, w, cw, chunk_len, x, logits, lam, merge, y, states, nullptr, 0, dtype, layout,
                         stream, nullptr, true);
}

int64_t gspn_proxy_forward4_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy,
                                            int64_t cw, int dtype, int layout) {
    if (!valid_dtype(dtype) || !dims_ok({n, c, h, w}) || !dims_ok({n, c_proxy, h, w}) || c_proxy < 1)
        return -1;
    const int64_t f4 = gspn_forward4_workspace_bytes(n, c_proxy, h, w, cw, dtype, layout);
    if (f4 < 0) return -1;
    return 2 * checked_product({n, c_proxy, h, w}) * static_cast<int64_t>(elem_size(dtype)) + f4;
}

int64_t gspn_proxy_states_bytes(int64_t n, int64_t c_proxy, int64_t h, int64_t w, int dtype) {
    ProxyStates K;
    return proxy_states_layout(n, c_proxy, h, w, dtype, &K) ? K.total : -1;
}

gspn_status gspn_proxy_forward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw,
                                int64_t chunk_len, const void* x, const void* w_down, const void* w_up,
                                const void* const logits[4], const void* const lam[4], const float* merge,
                                void* y, void* states, void* workspace, int64_t workspace_bytes, int dtype,
                                int layout, void* stream) {
    return proxy_impl(n, c, h, w, c_proxy, cw, chunk_len, x, w_down, w_up, logits, lam, merge, y, states, workspace,
                      workspace_bytes, dtype, layout, stream, nullptr);
}

gspn_status gspn_proxy_forward4_timed(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy,
                                      int64_t cw, int64_t chunk_len, const void* x, const void* w_down,
                                      const void* w_up, const void* const logits[4],
                                      const void* const lam[4], const float* merge, void* y, void* states,
                                      void* workspace, int64_t workspace_bytes, int dtype, int layout,
                                      void* stream, gspn_stage_times* times) {
    if (!times) return GSPN_ERR_NULL_POINTER;
    Timer tm;
    tm.st = as_stream(stream);
    const gspn_status s = proxy_impl(n, c, h, w, c_proxy, cw, chunk_len, x, w_down, w_up, logits, lam, merge, y,
                                     states, workspace, workspace_bytes, dtype, layout, stream, &tm);
    const hipError_t e = tm.finish(times);
    return s != GSPN_OK ? s : from_hip(e);
}

int64_t gspn_backward4_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int dtype,
                                       int layout) {
    if (!valid_dtype(dtype) || !valid_layout(layout) || !dims_ok({n, c, h, w}) || !(cw == 1 || cw == c)) return -1;
    const int64_t elems = checked_product({n, c, h, w});
    // x^T, gy^T and three dx terms in the storage type, rounded up to 4
    // bytes; four fp32 state maps (last, so that a caller passing the states
    // may give that much less); for channel-shared logits over several
    // channels the gradient sums and the normalised weights of the recomputed
    // forward (first)
    // the banded adjoint's products at band boundaries, for launches of very
    // few long lines (before the states)
    const int64_t maps = (5 * elems * static_cast<int64_t>(elem_size(dtype)) + 3) / 4 * 4 + 4 * elems * 4 +
                         adjoint_band_bytes(n, c, h, w);
    const int64_t nhw = checked_product({n, h, w});
    const int64_t shared = (cw == 1 && c > 1) ? 4 * 3 * nhw * 4 + 4 * nhw * (dtype == GSPN_F32 ? 3 * 4 : 4) : 0;
    if (layout == GSPN_LAYOUT_SCAN) return shared + maps;
    // the scan-frame copies of the horizontal inputs and room for their
    // gradients, before the states
    const int64_t lc = layout_copy_bytes(n, c, h, w, cw, dtype);
    return lc < 0 ? -1 : shared + maps + 2 * lc;
}

gspn_status gspn_backward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk_len,
                           const void* x, const void* const logits[4], const void* const lam[4], const float* merge,
                           const float* states, const void* gy, void* dx, void* const dlogits[4],
                           void* const dlam[4], float* dmerge, void* workspace, int64_t workspace_bytes, int dtype,
                           int layout, void* stream) {
    return backward_impl(n, c, h, w, cw, chunk_len, x, logits, lam, merge, states, gy, dx, dlogits, dlam, dmerge,
                         workspace, workspace_bytes, dtype, layout, stream, nullptr);
}

gspn_status gspn_backward4_timed(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk_len,
                                 const void* x, const void* const logits[4], const void* const lam[4],
                                 const float* merge, const float* states, const void* gy, void* dx,
                                 void* const dlogits[4], void* const dlam[4], float* dmerge, void* workspace,
                                 int64_t workspace_bytes, int dtype, int layout, void* stream,
                                 gspn_stage_times* times) {
    if (!times) return GSPN_ERR_NULL_POINTER;
    Timer tm;
    tm.st = as_stream(stream);
    const gspn_status s = backward_impl(n, c, h, w, cw, chunk_len, x, logits, lam, merge, states, gy, dx, dlogits,
                                        dlam, dmerge, workspace, workspace_bytes, dtype, layout, stream, &tm);
    const hipError_t e = tm.finish(times);
    return s != GSPN_OK ? s : from_hip(e);
}

int64_t gspn_proxy_backward4_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy,
                                             int64_t cw, int dtype, int layout) {
    ProxyBwdLayout L;
    return proxy_bwd_layout(n, c, h, w, c_proxy, cw, dtype, layout, &L) ? L.total : -1;
}

gspn_status gspn_proxy_backward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw,
                                 int64_t chunk_len, const void* x, const void* w_down, const void* w_up,
                                 const void* const logits[4], const void* const lam[4], const float* merge,
                                 const void* states, const void* gy, void* dx, float* dw_down, float* dw_up,
                                 void* const dlogits[4], void* const dlam[4], float* dmerge, void* workspace,
                                 int64_t workspace_bytes, int dtype, int layout, void* stream) {
    return proxy_backward_impl(n, c, h, w, c_proxy, cw, chunk_len, x, w_down, w_up, logits, lam, merge, states, gy,
                               dx, dw_down, dw_up, dlogits, dlam, dmerge, workspace, workspace_bytes, dtype, layout,
                               stream, nullptr);
}

gspn_status gspn_proxy_backward4_timed(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw,
                                       int64_t chunk_len, const void* x, const void* w_down, const void* w_up,
                                       const void* const logits[4], const void* const lam[4], const float* merge,
                                       const void* states, const void* gy, void* dx, float* dw_down, float* dw_up,
                                       void* const dlogits[4], void* const dlam[4], float* dmerge, void* workspace,
                                       int64_t workspace_bytes, int dtype, int layout, void* stream,
                                       gspn_stage_times* times) {
    if (!times) return GSPN_ERR_NULL_POINTER;
    Timer tm;
    tm.st = as_stream(stream);
    const gspn_status s = proxy_backward_impl(n, c, h, w, c_proxy, cw, chunk_len, x, w_down, w_up, logits, lam,
                                              merge, states, gy, dx, dw_down, dw_up, dlogits, dlam, dmerge,
                                              workspace, workspace_bytes, dtype, layout, stream, &tm);
    const hipError_t e = tm.finish(times);
    return s != GSPN_OK ? s : from_hip(e);
}

}  // extern "C"
