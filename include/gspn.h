/*
 * gspn.h -- C ABI of libgspn, GSPN's 2D line-scan linear propagation on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (GSPN-2 paper notes, section "2D spatial propagation
 * recap"; GSPN summary page, section "Approach"): for x in R^{N x C x H x W}
 * a line scan runs in each of four directions,
 *
 *     h_i = w_i h_{i-1} + lambda_i (.) x_i,
 *
 * line by line along the scan axis, with h = 0 before the first line.  Each
 * w_i is tridiagonal and row-stochastic: position k of line i couples to
 * positions k-1, k, k+1 of the previous line with weights obtained from three
 * logits by a sigmoid followed by division by their sum; at a line border
 * the sum runs over the neighbours that exist (a missing neighbour has
 * weight 0).  The four direction outputs are merged by an elementwise sum,
 * or by the learnable merge of the GSPN summary page's ablation table (one
 * weight per direction and channel, see gspn_forward4).  Variants:
 * channel-shared w (GSPN-2 notes, "Optimisation 2"), independent chunks
 * along the scan axis ("Optimisation 1") and the 1x1 projections to and from
 * a C_proxy-channel space ("Optimisation 2").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All pointers are device pointers (HIP device memory) unless stated;
 *    every tensor is contiguous, row-major.  Pointers must be aligned to
 *    their element size; otherwise GSPN_ERR_MISALIGNED.
 *  - Layouts:
 *      x, y, h, out        [N][C][H][W]
 *      logits, w (dir d)   [N][Cw][3][S][L]   Cw = 1 (shared) or C
 *      lam (dir d)         [N][C][S][L]
 *    (S, L) = (H, W) for GSPN_T2B / GSPN_B2T and (W, H) for GSPN_L2R /
 *    GSPN_R2L: the per-direction tensors are stored in the direction's scan
 *    frame, so that each scan step reads one contiguous line (the coalesced
 *    layout of GSPN-2 notes, "Optimisation 3").  For a horizontal direction,
 *    element (step i, position k) is array column i, row k.  The three
 *    logits/weights of a position are ordered (k-1, k, k+1) in array order
 *    for every direction; the first line of a scan (and of each chunk) does
 *    not use its logits.
 *    The four-direction calls (gspn_forward4, gspn_proxy_forward4,
 *    gspn_backward4 and their workspace queries) take a `layout` argument:
 *    GSPN_LAYOUT_SCAN is the scan-frame layout above; GSPN_LAYOUT_ARRAY
 *    stores every direction's logits as [N][Cw][3][H][W] and lambda as
 *    [N][C][H][W] (array frame for all four directions; so are the backward's
 *    dlogits and dlam).  The library then copies the horizontal directions'
 *    tensors into their scan frame inside its workspace with an LDS-tiled
 *    transpose (and the backward's horizontal gradients back out), so this
 *    layout needs a workspace and moves those tensors' bytes twice more.
 *    Any other value is GSPN_ERR_BAD_LAYOUT.
 *  - dtype: every tensor of one call has the same storage type, GSPN_F32 or
 *    GSPN_BF16.  Arithmetic is always fp32 (bf16 values are widened exactly;
 *    bf16 results are rounded to nearest even at each store).
 *  - stream: a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call is asynchronous on that stream; the library never allocates or
 *    frees memory, keeps no mutable global state, and never synchronises
 *    (except the *_timed measurement calls, which wait for their own events).
 *  - Ownership: the caller owns every buffer and must keep it alive until the
 *    work queued on `stream` has finished.
 *  - Errors: arguments are validated on the host before anything is queued.
 *    A failed validation returns its code and queues nothing.  A failed
 *    kernel launch returns GSPN_ERR_HIP.  No C++ exception crosses the ABI.
 *    A call whose tensors are empty (a zero dimension) returns GSPN_OK and
 *    queues nothing, without looking at its pointers.
 *  - Aliasing: an output may not overlap any input, except that with
 *    accumulate = 1 the output is read and written in place.
 *  - Domain: every finite logit and +-Inf is accepted.  The fp32 sigmoid
 *    clamps its argument to [-87, 87]; a row whose every existing logit is
 *    below about -69 (where the sigmoids could underflow the row sum) is
 *    normalised as exp(z - max z) / sum, equal to the normalised sigmoids to
 *    fp32 precision there.  A row whose every existing logit is -Inf has
 *    weights 0/0 = NaN, as in exact arithmetic.  NaN inputs propagate by IEEE
 *    rules.
 *  - Limits: a line may hold at most GSPN_MAX_LINE positions (else
 *    GSPN_ERR_UNSUPPORTED); dimensions must be in [0, 2^31) and N*C*H*W < 2^58.
 */
#ifndef GSPN_H_
#define GSPN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSPN_ABI_VERSION 11
#define GSPN_MAX_LINE 4096

typedef enum {
    GSPN_OK = 0,
    GSPN_ERR_NULL_POINTER = 1,
    GSPN_ERR_BAD_SHAPE = 2,
    GSPN_ERR_BAD_DIRECTION = 3,
    GSPN_ERR_BAD_DTYPE = 4,
    GSPN_ERR_BAD_CHUNK = 5,
    GSPN_ERR_BAD_WEIGHT_CHANNELS = 6,
    GSPN_ERR_MISALIGNED = 7,
    GSPN_ERR_ALIASING = 8,
    GSPN_ERR_UNSUPPORTED = 9,
    GSPN_ERR_HIP = 10,
    GSPN_ERR_WORKSPACE = 11,
    GSPN_ERR_BAD_LAYOUT = 12
} gspn_status;

typedef enum { GSPN_T2B = 0, GSPN_B2T = 1, GSPN_L2R = 2, GSPN_R2L = 3 } gspn_dir;

typedef enum { GSPN_F32 = 0, GSPN_BF16 = 1 } gspn_dtype;

/* Where the per-direction logits and lambdas of the four-direction calls
 * live (see "Layouts" above). */
typedef enum { GSPN_LAYOUT_SCAN = 0, GSPN_LAYOUT_ARRAY = 1 } gspn_layout;

/*
 * gspn_normalize_weights -- sigmoid + row normalisation of one direction's
 * logits (GSPN summary page, "Approach"; GSPN-2 notes, "2D spatial
 * propagation recap": rows sum to 1).
 *   logits  [n][cw][3][S][L] (input), w_out same layout (output).
 *   w_out[o] = s_o / sum_{valid o'} s_{o'}, s_o = 1/(1+exp(-logit_o)), and 0
 *   for a neighbour outside the line.  (S, L) follow from dir, h, w.
 */
gspn_status gspn_normalize_weights(int dir, int64_t n, int64_t cw, int64_t h, int64_t w,
                                   const void* logits, void* w_out, int dtype, void* stream);

/*
 * gspn_scan_fwd -- one direction of the line scan (GSPN-2 notes, "2D
 * spatial propagation recap"), optionally cut into independent chunks of
 * chunk_len steps counted in scan order (GSPN-2 notes, "Optimisation 1":
 * independent (chunk, n, c) blocks).
 *   dir           GSPN_T2B / GSPN_B2T / GSPN_L2R / GSPN_R2L.
 *   chunk_len     0 or >= S: one chunk over the whole scan; K > 0: h is reset
 *                 to 0 every K steps; < 0: GSPN_ERR_BAD_CHUNK.
 *   n, c, h, w    dimensions of x and out.
 *   cw            1 (channel-shared w, "Optimisation 2") or c; else
 *                 GSPN_ERR_BAD_WEIGHT_CHANNELS.
 *   x             [n][c][h][w] input.
 *   wts           [n][cw][3][S][L]: logits if wts_are_logits = 1, else
 *                 weights already normalised (e.g. by gspn_normalize_weights).
 *   lam           [n][c][S][L] per-position scaling lambda.
 *   out           [n][c][h][w]: out = h (accumulate = 0) or out += h (1).
 */
gspn_status gspn_scan_fwd(int dir, int64_t chunk_len, int64_t n, int64_t c, int64_t h, int64_t w,
                          int64_t cw, const void* x, const void* wts, int wts_are_logits,
                          const void* lam, void* out, int accumulate, int dtype, void* stream);

/*
 * gspn_merge4 -- y = h0 + h1 + h2 + h3 elementwise over numel elements (the
 * merge of the four direction outputs by summation).  y may not overlap any
 * h_d.  Sum order: ((h0 + h1) + h2) + h3 in fp32.
 */
gspn_status gspn_merge4(const void* h0, const void* h1, const void* h2, const void* h3, void* y,
                        int64_t numel, int dtype, void* stream);

/*
 * gspn_proxy_project -- 1x1 projection between channel spaces (GSPN-2
 * notes, "Optimisation 2", compressive channel proxy): for every pixel,
 * out[n][o][p] = sum_c weight[o][c] * in[n][c][p].  No bias.
 *   in      [n][c_in][h][w], weight [c_out][c_in], out [n][c_out][h][w].
 * Accumulation is fp32 whatever the storage type.
 */
gspn_status gspn_proxy_project(int64_t n, int64_t c_in, int64_t h, int64_t w, int64_t c_out,
                               const void* in, const void* weight, void* out, int dtype,
                               void* stream);

/*
 * gspn_scan4_fwd -- the four directions' scans of one forward in a single
 * launch, each writing its own output: out[d] = scan_d(x, logits[d], lam[d])
 * for d in (T2B, B2T, L2R, R2L) (GSPN-2 notes, "2D spatial propagation
 * recap": four line scans over the same x).  The four directions run
 * concurrently.  Shapes as for gspn_forward4; out is a host array of 4
 * device pointers, each [n][c][h][w], pairwise disjoint and overlapping no
 * input.  Lines may hold at most 2048 positions, and the four directions
 * together at most 2^31 - 1 (plane, chunk) pairs (else
 * GSPN_ERR_UNSUPPORTED).
 */
gspn_status gspn_scan4_fwd(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                           int64_t chunk_len, const void* x, const void* const logits[4],
                           const void* const lam[4], void* const out[4], int dtype, void* stream);

/*
 * gspn_forward4_workspace_bytes -- bytes of the optional gspn_forward4
 * workspace: four maps of n*c*h*w elements of the storage type (x transposed
 * into the horizontal scan frame and three partial outputs); for
 * channel-shared weights over more than one channel (cw == 1 < c), the four
 * directions' normalised weights: 4 * 3 * n*h*w floats for GSPN_F32, 4 *
 * n*h*w 32-bit half pairs for GSPN_BF16 (see gspn_forward4); rounded up to a
 * multiple of 4 bytes; then 2 * 4 * n*c * max(h, w) floats of scan states at
 * band boundaries (used when very few long lines are split across
 * workgroups).  Returns -1 when the arguments are invalid (negative or
 * overflowing dimensions, cw not in {1, c}, unknown dtype).
 */
int64_t gspn_forward4_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                                      int dtype, int layout);

/*
 * gspn_forward4 -- the four-direction propagation with summed or learnable
 * merge:
 *   y[:, k] = sum over d in (T2B, B2T, L2R, R2L) of
 *             m[d][k] * scan_d(x, logits[d], lam[d])[:, k]   (channel k)
 *   logits[d]  [n][cw][3][S_d][L_d] logits of direction d (normalised inside).
 *   lam[d]     [n][c][S_d][L_d]; the same pointer may be given for all d.
 *   logits and lam are host arrays of 4 device pointers, indexed by gspn_dir.
 *   merge      NULL: m = 1, the plain sum.  Otherwise a device array of
 *              4 * c fp32 values [4][c] indexed by gspn_dir then channel,
 *              whatever the storage type: the learnable merge that the GSPN
 *              summary page's ablation table puts in place of SPN's
 *              max-pooling merge, read as one weight per direction and
 *              channel.  The scans apply it to lambda * x (each h_d is
 *              linear in it), so it costs no extra pass.  4-byte aligned;
 *              y may not overlap it.
 *   y          [n][c][h][w] output; may not overlap any input.
 *   states     NULL, or a device buffer of 4 * n*c*h*w fp32 values, 4-byte
 *              aligned, overlapping neither y, an input nor the workspace
 *              (else GSPN_ERR_MISALIGNED / GSPN_ERR_ALIASING): the four
 *              directions' unweighted scans h_d in fp32, kept for
 *              gspn_backward4, which then skips its own recompute.  Map d
 *              starts at states + d*n*c*h*w and lies in direction d's scan
 *              frame: [n][c][h][w] for T2B and B2T, [n][c][w][h] for L2R and
 *              R2L.  It needs the workspace and lines of at most 2048
 *              positions (else GSPN_ERR_WORKSPACE / GSPN_ERR_UNSUPPORTED).
 *              Planes of at most 64 x 64 then leave their one-pass path
 *              (which keeps no states) for the four-direction launch; y is
 *              then merged from these fp32 maps, so for bf16 storage it can
 *              differ from the y of a call without states in the last bf16
 *              place.  Many big planes keep the plane-sequential kernel,
 *              which writes the same maps bit for bit; its y, too, may
 *              differ from the y of a call without states in the last bf16
 *              place.
 *   workspace  optional device buffer of workspace_bytes bytes, 4-byte
 *              aligned.  NULL (or 0 bytes): the directions run one after
 *              another, the first writing y and the others adding to it, and
 *              the logits are normalised inside the scans.  Otherwise it
 *              must hold gspn_forward4_workspace_bytes() bytes (else
 *              GSPN_ERR_WORKSPACE) and overlap neither y nor any input (else
 *              GSPN_ERR_ALIASING).  The library then (a) normalises
 *              channel-shared logits once into weights that every channel's
 *              scan reads: fp32 triples for GSPN_F32; for GSPN_BF16 the two
 *              side weights w_{k-1}, w_{k+1} as IEEE half precision, the
 *              centre weight recomputed in fp32 as 1 minus their sum (rows
 *              still sum to 1; the side weights carry about 2^-11 relative
 *              rounding), (b) transposes x once so that the horizontal
 *              directions run as row-coalesced scans whose outputs a
 *              transposing merge adds into y, and (c) runs all four
 *              directions in one launch into separate maps (lines up to 2048
 *              positions and at most 2^31 - 1 (plane, chunk) pairs over the
 *              four; beyond either, one direction after another through
 *              the workspace's maps), or, when the planes are so few that the four
 *              directions make at most 64 long lines, splits each line
 *              across workgroups and runs the scan in bands of steps, one
 *              launch per band.  Its contents afterwards are unspecified.
 *              Planes of at most 64 x 64 take a one-pass path (x read once,
 *              y written once) with or without a workspace, unless states
 *              are wanted.  In all cases y
 *              is the same up to fp32 rounding order and, for bf16, rounding
 *              of the intermediates.
 */
gspn_status gspn_forward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                          int64_t chunk_len, const void* x, const void* const logits[4],
                          const void* const lam[4], const float* merge, void* y, float* states, void* workspace,
                          int64_t workspace_bytes, int dtype, int layout, void* stream);

/*
 * gspn_forward4_noalloc -- gspn_forward4 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same computation and arguments, except that
 * the workspace is not passed in.  It is taken from a static device array of
 * GSPN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on, from the moment its code is loaded on that device until the
 * process ends; the call itself allocates and frees nothing.
 *   Size limit: calls whose gspn_forward4_workspace_bytes(n, c, h, w, cw,
 *   dtype, layout) exceeds GSPN_NOALLOC_SCRATCH_BYTES return
 *   GSPN_ERR_WORKSPACE before touching the device.
 *   Device: the array of the current HIP device is used, so `stream` must
 *   belong to the current device (as for any launch).  Its address is looked
 *   up on the device's first call (a failure there is GSPN_ERR_HIP).
 *   Concurrency: every call on one GPU shares that GPU's array, which keeps
 *   whatever the last call left there (nothing in it needs clearing between
 *   calls).  Calls that overlap in time on one GPU -- on different streams or
 *   from different threads -- race on it and give undefined results; order
 *   them on one stream or with events.
 * Other arguments, validation and errors as for gspn_forward4 (the workspace
 * checks aside).
 */
#define GSPN_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)

gspn_status gspn_forward4_noalloc(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                                  int64_t chunk_len, const void* x, const void* const logits[4],
                                  const void* const lam[4], const float* merge, void* y, float* states,
                                  int dtype, int layout, void* stream);

/*
 * gspn_proxy_forward4_workspace_bytes -- bytes of the gspn_proxy_forward4
 * workspace: the projected input and the merged output in proxy space (2 *
 * n*c_proxy*h*w elements) plus gspn_forward4_workspace_bytes(n, c_proxy, h,
 * w, cw).  Returns -1 for invalid arguments.
 */
int64_t gspn_proxy_forward4_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy,
                                            int64_t cw, int dtype, int layout);

/*
 * gspn_proxy_states_bytes -- bytes of the proxy-space state that
 * gspn_proxy_forward4 can keep for gspn_proxy_backward4 (its `states`
 * argument): the projected input x_p and the merged proxy-space output y_p
 * (n*c_proxy*h*w elements of the storage type each, each part rounded up to
 * 256 bytes) and, for planes larger than 64 x 64, the four directions' fp32
 * proxy-space scans as gspn_forward4 keeps them (16 * n*c_proxy*h*w bytes).
 * Returns -1 for invalid arguments.
 */
int64_t gspn_proxy_states_bytes(int64_t n, int64_t c_proxy, int64_t h, int64_t w, int dtype);

/*
 * gspn_proxy_forward4 -- the compressive-proxy propagation (GSPN-2 notes,
 * "Optimisation 2"): project C -> C_proxy, run the four-direction
 * propagation in proxy space, project back C_proxy -> C:
 *   x_p = w_down . x,   y_p = forward4(x_p, logits, lam, merge),   y = w_up . y_p
 * (1x1 projections, no bias).
 *   x        [n][c][h][w];  y [n][c][h][w] output (may not overlap any input)
 *   w_down   [c_proxy][c];  w_up [c][c_proxy]
 *   logits[d] [n][cw][3][S_d][L_d] (cw = 1 or c_proxy), lam[d] [n][c_proxy][S_d][L_d]
 *   merge    NULL (sum) or fp32 [4][c_proxy], as in gspn_forward4
 *   workspace required: gspn_proxy_forward4_workspace_bytes() bytes, 4-byte
 *            aligned, overlapping nothing else (else GSPN_ERR_WORKSPACE /
 *            GSPN_ERR_MISALIGNED / GSPN_ERR_ALIASING; NULL is
 *            GSPN_ERR_NULL_POINTER).
 *   states   NULL, or gspn_proxy_states_bytes() bytes, 256-byte aligned, that
 *            overlap no input, y or the workspace (else GSPN_ERR_MISALIGNED /
 *            GSPN_ERR_ALIASING): the call keeps x_p, y_p and (planes larger
 *            than 64 x 64) the fp32 proxy-space scans there for
 *            gspn_proxy_backward4, which then recomputes none of them.  For
 *            planes larger than 64 x 64 y_p is then merged from those fp32
 *            scans, as gspn_forward4 does with states, so for bf16 storage y
 *            can differ from that of a call without it in the last bf16
 *            place (it is the y_p the backward's own recompute forms).
 * Intermediates are stored in the storage type (bf16 intermediates round
 * once at each store).
 */
gspn_status gspn_proxy_forward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw,
                                int64_t chunk_len, const void* x, const void* w_down, const void* w_up,
                                const void* const logits[4], const void* const lam[4], const float* merge,
                                void* y, void* states, void* workspace, int64_t workspace_bytes, int dtype,
                                int layout, void* stream);

/*
 * gspn_backward4_workspace_bytes -- bytes of the gspn_backward4 workspace:
 * for channel-shared logits over more than one channel (cw == 1 < c), 4 * 3
 * * n*h*w floats of gradient sums plus the four directions' normalised
 * weights as in gspn_forward4_workspace_bytes; five maps of n*c*h*w
 * elements of the storage type (x and dL/dy transposed into the horizontal
 * scan frame, three per-direction dx terms), rounded up to a multiple of 4
 * bytes; for at most 16 planes (n*c <= 16) with h and w both at least 512,
 * 2 * 4 * 3 * n*c * max(h, w) floats for the banded adjoint (family 3
 * below); last, the four directions' forward states in fp32 (4 * n*c*h*w
 * floats), which a call given the states does not need: it may pass 16 *
 * n*c*h*w bytes less.  Returns -1 for invalid arguments.
 */
int64_t gspn_backward4_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int dtype,
                                       int layout);

/*
 * gspn_backward4 -- gradients of the four-direction propagation of
 * gspn_forward4 (same x, logits, lam, merge, cw, chunk_len) for dL/dy = gy:
 * the exact derivative of the scan that the GSPN-2 paper notes define in "2D
 * spatial propagation recap" (the GSPN-2 summary page, "Experimental setup",
 * reports forward and backward runtimes).  Per direction, in its scan frame,
 * the adjoint a_t = g_t + M_{t+1}^T a_{t+1} runs against the scan order
 * (restarting at chunk ends), and with m_d = merge[d][k] (1 if merge is NULL)
 *   dlam[d]      = m_d a * x                  [n][c][S_d][L_d]   (written)
 *   dx           = sum_d m_d a_d * lam[d]      [n][c][h][w]       (written)
 *   dlogits[d]   = d w / d z applied to m_d a_t h_{t-1}   [n][cw][3][S_d][L_d]
 *                  (written; 0 on each chunk's first line, whose logits the
 *                  forward does not use; for cw == 1 < c the sum over
 *                  channels, accumulated in fp32 in an order that may vary
 *                  between calls)
 *   dmerge       [4][c] fp32 (written, optional: NULL skips it; computed also
 *                  when merge is NULL, as the gradient at m = 1): the sum
 *                  over images and positions of gy * h_d, evaluated as
 *                  sum_t <a_t, lam_t * x_t> (the same value for the linear
 *                  recurrence), accumulated in fp32 in an order that may vary
 *                  between calls.
 * states: NULL, or the fp32 states that gspn_forward4 wrote for the same
 * inputs (layout there), 4-byte aligned, overlapping no output and not the
 * workspace: the adjoint reads them instead of recomputing the forward.
 * Without them the forward states are recomputed inside, in fp32 and with
 * the same per-position arithmetic, so both ways give the same gradients bit
 * for bit.
 * workspace: required, gspn_backward4_workspace_bytes() bytes (16 * n*c*h*w
 * fewer with states), 4-byte aligned.  Outputs may overlap neither an input,
 * the workspace nor each other.  Lines may hold at most 2048 positions, and
 * the four directions together at most 2^31 - 1 (plane, chunk) pairs (else
 * GSPN_ERR_UNSUPPORTED).
 */
gspn_status gspn_backward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk_len,
                           const void* x, const void* const logits[4], const void* const lam[4], const float* merge,
                           const float* states, const void* gy, void* dx, void* const dlogits[4],
                           void* const dlam[4], float* dmerge, void* workspace, int64_t workspace_bytes, int dtype,
                           int layout, void* stream);

/*
 * gspn_proxy_backward4_workspace_bytes -- bytes of the gspn_proxy_backward4
 * workspace: four proxy-space maps (n*c_proxy*h*w elements of the storage
 * type each), both projection weights transposed, the weight-gradient
 * partial sums (at most 2048 * c * c_proxy floats), for planes larger than
 * 64 x 64 the proxy-space forward's fp32 states (16 * n*c_proxy*h*w bytes),
 * and the larger of gspn_forward4_workspace_bytes and
 * gspn_backward4_workspace_bytes (less the states) for (n, c_proxy, h, w,
 * cw), each part rounded up to 256 bytes.  Returns -1 for invalid arguments
 * (c < 1 or c_proxy < 1 among them).
 */
int64_t gspn_proxy_backward4_workspace_bytes(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy,
                                             int64_t cw, int dtype, int layout);

/*
 * gspn_proxy_backward4 -- gradients of gspn_proxy_forward4 (same x, w_down,
 * w_up, logits, lam, merge, cw, chunk_len, layout) for dL/dy = gy, by the
 * chain rule through its three stages (GSPN-2 notes, "Optimisation 2"):
 *   dL/dy_p   = w_up^T gy                          (a 1x1 projection C -> C_proxy)
 *   dx_p, dlogits, dlam, dmerge = gspn_backward4 in proxy space for dL/dy_p,
 *               at x_p = w_down x
 *   dx        = w_down^T dx_p                       [n][c][h][w]   (written)
 *   dw_up     [c][c_proxy] fp32   = sum over images and pixels of gy[c] y_p[k]
 *   dw_down   [c_proxy][c] fp32   = sum over images and pixels of dx_p[k] x[c]
 *   dlogits[d], dlam[d], dmerge   as gspn_backward4 gives them in proxy space
 *               (dmerge optional: NULL skips it)
 * states: NULL, or what gspn_proxy_forward4 kept for the same inputs
 * (gspn_proxy_states_bytes() bytes, 256-byte aligned, overlapping no output
 * and not the workspace).  Without it x_p and y_p = forward4(x_p) are
 * recomputed inside (stored in the storage type, as the forward stores them;
 * every intermediate rounds once at its store), and for planes larger than
 * 64 x 64 that forward keeps its fp32 states for the proxy-space backward, as
 * gspn_forward4 / gspn_backward4 do with states; both ways give the same
 * gradients (those summed with fp32 atomics up to their summation order).
 * The workspace is the same size either way.  The weight gradients are summed in fp32 over at most 2048 runs
 * of pixels, then the runs in a fixed order: they do not vary between calls.
 * With no pixels (n*h*w == 0) dw_down, dw_up and dmerge are written as
 * zeros and nothing else is touched (the other pointers may then be NULL).
 * c < 1 or c_proxy < 1 is GSPN_ERR_BAD_SHAPE.  Pointers, alignment (the storage type's size; 4 bytes
 * for the fp32 arrays and the workspace) and aliasing as in gspn_backward4:
 * outputs may overlap neither an input, the workspace nor each other.  The
 * proxy-space propagation must meet gspn_backward4's limits (else
 * GSPN_ERR_UNSUPPORTED, before anything is queued).
 */
gspn_status gspn_proxy_backward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw,
                                 int64_t chunk_len, const void* x, const void* w_down, const void* w_up,
                                 const void* const logits[4], const void* const lam[4], const float* merge,
                                 const void* states, const void* gy, void* dx, float* dw_down, float* dw_up,
                                 void* const dlogits[4], void* const dlam[4], float* dmerge, void* workspace,
                                 int64_t workspace_bytes, int dtype, int layout, void* stream);

/*
 * Stage timing of one forward call (measurement only).
 *
 * gspn_forward4_timed / gspn_proxy_forward4_timed take the arguments of
 * gspn_forward4 / gspn_proxy_forward4, validate them identically and launch
 * exactly the same kernels in the same order on the same stream, with a pair
 * of HIP timing events recorded on that stream around every launch.  Before
 * returning they wait for the last event (the only calls in the library that
 * block the host) and fill *times: per stage, the summed duration in
 * milliseconds of its launches and the number of launches.  The events are
 * created and destroyed inside the call; no device memory is allocated.
 * Stages that did not run read 0 ms / 0 launches; scan_kernel names the
 * scan kernel the call ran.  times == NULL is
 * GSPN_ERR_NULL_POINTER.  If a launch fails the call still waits for what
 * was queued, then returns GSPN_ERR_HIP.
 */
typedef enum {
    GSPN_STAGE_PROJECT_DOWN = 0, /* 1x1 projection C -> C_proxy */
    GSPN_STAGE_NORMALIZE = 1,    /* channel-shared logits -> normalised weights */
    GSPN_STAGE_TRANSPOSE = 2,    /* x into the horizontal scan frame */
    GSPN_STAGE_SCAN = 3,         /* the line-scan launches (1 fused or 4) */
    GSPN_STAGE_COMBINE = 4,      /* transposing merge of the partial maps into y */
    GSPN_STAGE_PROJECT_UP = 5,   /* 1x1 projection C_proxy -> C */
    GSPN_STAGE_ADJOINT = 6,      /* backward: the adjoint line-scan launch */
    GSPN_STAGE_REDUCE = 7,       /* backward: clearing / storing the shared-logit sums, clearing dmerge;
                                    proxy backward also: the projection weights transposed, the weight-
                                    gradient partial sums reduced */
    GSPN_STAGE_LAYOUT = 8,       /* GSPN_LAYOUT_ARRAY: horizontal logits / lambdas (and their gradients)
                                    copied between the array and scan frames */
    GSPN_STAGE_TAIL = 9,         /* GSPN_SCAN_SEQUENTIAL: the planes of a last, at most half-full round
                                    of one plane per CU, run on the concurrent four-direction path
                                    (every launch of that forward, timed as one) */
    GSPN_STAGE_WEIGHT_GRAD = 10, /* proxy backward: the two passes that sum the weight gradients' partials,
                                    over gy (with dL/dy_p = w_up^T gy folded in) and over x */
    GSPN_NUM_STAGES = 11
} gspn_stage;

/* Which scan kernel a forward call ran (gspn_stage_times.scan_kernel). */
typedef enum {
    GSPN_SCAN_NONE = 0,         /* no scan (empty input or failed validation) */
    GSPN_SCAN_PER_DIRECTION = 1,/* one launch per direction */
    GSPN_SCAN_FUSED4 = 2,       /* four directions in one launch, one workgroup per line */
    GSPN_SCAN_LONG_LINE = 3,    /* four directions in one launch, 16-byte vectors per lane */
    GSPN_SCAN_PLANE = 4,        /* one workgroup per plane, all four directions, y written once */
    GSPN_SCAN_BANDED = 5,       /* very few long lines: lines split across workgroups, one launch per band of steps */
    GSPN_SCAN_SEQUENTIAL = 6    /* many big planes: one workgroup per plane runs the four directions in turn,
                                   building y in place */
} gspn_scan_kernel;

/* The adjoint launch of a backward call (gspn_stage_times.adjoint; all 0
 * when the call ran none): the kernel family (1 = one workgroup per line and
 * direction, 2 = one workgroup per plane for planes of at most 64 x 64,
 * 3 = very few long unchunked lines, at most 16 planes with both sides at
 * least 512: each line split into segments of 256 positions, one workgroup
 * per segment with a halo of 128 positions on each side, one launch per
 * band of 128 steps, the products crossing a band's border kept in the
 * workspace), the
 * positions each lane owns, the channels one workgroup runs together (more
 * than 1 only for channel-shared logits, whose gradient it sums over them),
 * and whether the streams touched once carry the non-temporal hint. */
typedef struct {
    int32_t family;
    int32_t positions_per_lane;
    int32_t channel_group;
    int32_t nontemporal;
} gspn_adjoint_plan;

typedef struct {
    float ms[GSPN_NUM_STAGES];
    int32_t launches[GSPN_NUM_STAGES];
    int32_t scan_kernel; /* a gspn_scan_kernel value */
    gspn_adjoint_plan adjoint;
} gspn_stage_times;

gspn_status gspn_forward4_timed(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                                int64_t chunk_len, const void* x, const void* const logits[4],
                                const void* const lam[4], const float* merge, void* y, float* states,
                                void* workspace, int64_t workspace_bytes, int dtype, int layout, void* stream,
                                gspn_stage_times* times);

gspn_status gspn_proxy_forward4_timed(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy,
                                      int64_t cw, int64_t chunk_len, const void* x, const void* w_down,
                                      const void* w_up, const void* const logits[4],
                                      const void* const lam[4], const float* merge, void* y, void* states,
                                      void* workspace, int64_t workspace_bytes, int dtype, int layout,
                                      void* stream, gspn_stage_times* times);

/* gspn_backward4 with stage timing (same contract as gspn_forward4_timed);
 * the forward recompute is reported as GSPN_STAGE_SCAN, except for planes of
 * at most 64 x 64, whose adjoint launch (GSPN_STAGE_ADJOINT) recomputes the
 * states itself (scan_kernel GSPN_SCAN_PLANE, no scan launches). */
gspn_status gspn_backward4_timed(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk_len,
                                 const void* x, const void* const logits[4], const void* const lam[4],
                                 const float* merge, const float* states, const void* gy, void* dx,
                                 void* const dlogits[4], void* const dlam[4], float* dmerge, void* workspace,
                                 int64_t workspace_bytes, int dtype, int layout, void* stream,
                                 gspn_stage_times* times);

/* gspn_proxy_backward4 with stage timing (same contract as gspn_forward4_timed);
 * the stages of the proxy-space forward and backward it runs are reported as
 * theirs, x's projection as GSPN_STAGE_PROJECT_DOWN, dx's as
 * GSPN_STAGE_PROJECT_UP, the passes over gy and x that sum the weight
 * gradients' partials as GSPN_STAGE_WEIGHT_GRAD. */
gspn_status gspn_proxy_backward4_timed(int64_t n, int64_t c, int64_t h, int64_t w, int64_t c_proxy, int64_t cw,
                                       int64_t chunk_len, const void* x, const void* w_down, const void* w_up,
                                       const void* const logits[4], const void* const lam[4], const float* merge,
                                       const void* states, const void* gy, void* dx, float* dw_down, float* dw_up,
                                       void* const dlogits[4], void* const dlam[4], float* dmerge, void* workspace,
                                       int64_t workspace_bytes, int dtype, int layout, void* stream,
                                       gspn_stage_times* times);

/* Human-readable name of a status code (static storage, never NULL). */
const char* gspn_status_string(int status);

/* GSPN_ABI_VERSION of the built library. */
int gspn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GSPN_H_ */
