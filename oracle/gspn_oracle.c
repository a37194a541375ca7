/*
 * gspn_oracle.c -- plain, slow, fp64 CPU oracle for GSPN's 2D line-scan
 * linear propagation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
 * and its Python binding) may include, link, load or call this file.  Only
 * the tests, the smoke check and the bench's CPU-baseline leg use it.  It
 * shares no code, header, table or helper with the GPU path.
 *
 * What it computes (sources are the GSPN pages):
 *  - "GSPN-2: Efficient Parallel Sequence Modeling" paper notes (zhaoyang97
 *    Paper-Notes page), section "2D spatial propagation recap": for an input
 *    x the propagation runs line by line, h_i = w_i h_{i-1} + lambda_i (.) x_i,
 *    where w_i is a W x W tridiagonal, row-stochastic matrix (rows sum to 1)
 *    and lambda_i a per-position scaling; four directions (top->bottom,
 *    bottom->top, left->right, right->left) each run one scan.
 *  - "Parallel Sequence Modeling via Generalized Spatial Propagation
 *    Network" summary page (atlas.scime.ai), section "Approach": the
 *    weights are made row-stochastic by a sigmoid followed by row
 *    normalisation over the three tridiagonal neighbours.
 *  - GSPN-2 notes, section "Optimisation 2: compact channel propagation":
 *    channel-shared w_i (lambda stays per channel) and the 1x1 projection
 *    to a C_proxy-channel space and back.
 *  - GSPN-2 notes, section "Optimisation 1": independent (chunk, n, c)
 *    blocks, i.e. the scan axis may be cut into independent chunks.
 *
 * Readings taken where the pages are silent (each also listed in the
 * design notes of the repository):
 *  - h is zero before the first line of a scan and before each chunk.
 *  - At a line border the sigmoid values are renormalised over the valid
 *    neighbours only; a missing neighbour gets weight exactly 0.  A line of
 *    length 1 therefore has w = [1].
 *  - The three logits of line i, position k, sit at (i, k) and weight
 *    h_{prev}[k-1], h_{prev}[k], h_{prev}[k+1] (array order, offsets -1,0,+1,
 *    not mirrored for the reversed directions).  The logits of the first
 *    line of a scan / chunk are unused.
 *  - Chunks start at scan step 0 in scan order; the last chunk may be short.
 *
 * Layouts (all contiguous, row-major):
 *  - x, h, y:      [N][C][H][W]                (array frame)
 *  - logits / w:   [N][Cw][3][S][L]           (scan frame of the direction)
 *  - lambda:       [N][C][S][L]                (scan frame of the direction)
 *  For the vertical directions (T2B, B2T) S = H, L = W and the scan frame is
 *  the array frame.  For the horizontal ones (L2R, R2L) S = W, L = H: step i
 *  is array column i and line position k is array row k.
 *
 * Everything is evaluated in double precision with straightforward loops.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

enum { DIR_T2B = 0, DIR_B2T = 1, DIR_L2R = 2, DIR_R2L = 3 };

static int dir_is_horizontal(int dir) { return dir == DIR_L2R || dir == DIR_R2L; }
static int dir_is_reversed(int dir) { return dir == DIR_B2T || dir == DIR_R2L; }

/* Logistic sigmoid, 1 / (1 + e^{-z}). */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/*
 * Row normalisation of one tridiagonal row (Approach section of the GSPN
 * summary; "rows sum to 1" in the GSPN-2 notes): s_o = sigmoid(z_o) for the
 * neighbours k-1, k, k+1 that exist on a line of length L, then each s_o is
 * divided by their sum.  Missing neighbours get 0.
 */
static void normalise_row(const double z[3], int64_t k, int64_t L, double w[3]) {
    double s[3];
    double sum = 0.0;
    for (int o = 0; o < 3; ++o) {
        int64_t nb = k + (o - 1);
        if (nb >= 0 && nb < L) {
            s[o] = sigmoid(z[o]);
        } else {
            s[o] = 0.0;
        }
        sum += s[o];
    }
    for (int o = 0; o < 3; ++o) {
        int64_t nb = k + (o - 1);
        w[o] = (nb >= 0 && nb < L) ? s[o] / sum : 0.0;
    }
}

static void frame_sizes(int dir, int64_t h, int64_t w, int64_t* S, int64_t* L) {
    if (dir_is_horizontal(dir)) {
        *S = w;
        *L = h;
    } else {
        *S = h;
        *L = w;
    }
}

/*
 * oracle_normalize: logits [n][cw][3][S][L] -> w (same layout).
 */
int oracle_normalize(int dir, int64_t n, int64_t cw, int64_t h, int64_t w,
                     const double* logits, double* w_out) {
    if (dir < 0 || dir > 3 || n < 0 || cw < 0 || h < 0 || w < 0 || !logits || !w_out)
        return ORACLE_BAD_ARG;
    int64_t S, L;
    frame_sizes(dir, h, w, &S, &L);
    const int64_t plane = S * L;
    const int64_t nplanes = n * cw;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < nplanes; ++p) {
        const double* zp = logits + p * 3 * plane;
        double* wp = w_out + p * 3 * plane;
        for (int64_t i = 0; i < S; ++i) {
            for (int64_t k = 0; k < L; ++k) {
                double z[3], ww[3];
                for (int o = 0; o < 3; ++o) z[o] = zp[o * plane + i * L + k];
                normalise_row(z, k, L, ww);
                for (int o = 0; o < 3; ++o) wp[o * plane + i * L + k] = ww[o];
            }
        }
    }
    return ORACLE_OK;
}

/*
 * oracle_scan: one direction of the line scan (GSPN-2 notes, "2D spatial
 * propagation recap"):
 *
 *   for scan step t = 0 .. S-1, line i = t (forward) or S-1-t (reversed):
 *     if t is the first step of a chunk: h_prev = 0
 *     h_i[k] = sum_{o in {-1,0,+1}, 0 <= k+o < L} w_i[k,o] * h_prev[k+o]
 *              + lambda_i[k] * x_i[k]
 *     h_prev = h_i
 *
 * chunk: 0 (or >= S) = one chunk over the whole line; K > 0 = a new chunk
 * every K steps counted in scan order.  cw: 1 (channel-shared w) or c
 * (per-channel w).  wts_are_logits: 1 = wts holds logits that are
 * normalised here, 0 = wts already holds the normalised w.
 * accumulate: 0 = out = h, 1 = out += h.  out is [n][c][h][w].
 */
int oracle_scan(int dir, int64_t chunk, int64_t n, int64_t c, int64_t h, int64_t w,
                int64_t cw, const double* x, const double* wts, int wts_are_logits,
                const double* lam, double* out, int accumulate) {
    if (dir < 0 || dir > 3 || chunk < 0 || n < 0 || c < 0 || h < 0 || w < 0) return ORACLE_BAD_ARG;
    if (!(cw == 1 || cw == c)) return ORACLE_BAD_ARG;
    if (!x || !wts || !lam || !out) return ORACLE_BAD_ARG;
    int64_t S, L;
    frame_sizes(dir, h, w, &S, &L);
    const int64_t plane = S * L;
    const int horizontal = dir_is_horizontal(dir);
    const int reversed = dir_is_reversed(dir);
    const int64_t K = (chunk == 0 || chunk >= S) ? S : chunk;
    const int64_t nplanes = n * c;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < nplanes; ++p) {
        const int64_t ni = p / (c > 0 ? c : 1);
        const int64_t ci = p % (c > 0 ? c : 1);
        const int64_t wplane = ni * cw + (cw == 1 ? 0 : ci);
        const double* xp = x + p * plane;            /* array frame [h][w] */
        const double* zp = wts + wplane * 3 * plane; /* scan frame [3][S][L] */
        const double* lp = lam + p * plane;          /* scan frame [S][L] */
        double* op = out + p * plane;                /* array frame [h][w] */

        /* Two line buffers: previous and current hidden state. */
        double* hprev = (double*)__builtin_alloca((size_t)(L > 0 ? L : 1) * sizeof(double));
        double* hcur = (double*)__builtin_alloca((size_t)(L > 0 ? L : 1) * sizeof(double));

        for (int64_t t = 0; t < S; ++t) {
            const int64_t i = reversed ? (S - 1 - t) : t;
            const int chunk_start = (t % K) == 0;
            for (int64_t k = 0; k < L; ++k) {
                /* array coordinates of (line i, position k) */
                const int64_t ah = horizontal ? k : i;
                const int64_t aw = horizontal ? i : k;
                const int64_t aidx = ah * w + aw;
                double acc = 0.0;
                if (!chunk_start) {
                    double ww[3];
                    if (wts_are_logits) {
                        double z[3];
                        for (int o = 0; o < 3; ++o) z[o] = zp[o * plane + i * L + k];
                        normalise_row(z, k, L, ww);
                    } else {
                        for (int o = 0; o < 3; ++o) ww[o] = zp[o * plane + i * L + k];
                    }
                    for (int o = 0; o < 3; ++o) {
                        const int64_t nb = k + (o - 1);
                        if (nb >= 0 && nb < L) acc += ww[o] * hprev[nb];
                    }
                }
                acc += lp[i * L + k] * xp[aidx];
                hcur[k] = acc;
                if (accumulate) {
                    op[aidx] += acc;
                } else {
                    op[aidx] = acc;
                }
            }
            double* tmp = hprev;
            hprev = hcur;
            hcur = tmp;
        }
    }
    return ORACLE_OK;
}

/*
 * oracle_forward4: the four directions T2B, B2T, L2R, R2L on the same x,
 * merged by an elementwise sum, y = sum_d h_d.  logits[d] / lam[d] are the
 * per-direction tensors in that direction's scan frame.
 */
int oracle_forward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk,
                    const double* x, const double* const* logits, const double* const* lam,
                    double* y) {
    if (!logits || !lam || !y) return ORACLE_BAD_ARG;
    const int64_t total = n * c * h * w;
    for (int64_t e = 0; e < total; ++e) y[e] = 0.0;
    for (int d = 0; d < 4; ++d) {
        int rc = oracle_scan(d, chunk, n, c, h, w, cw, x, logits[d], 1, lam[d], y, 1);
        if (rc != ORACLE_OK) return rc;
    }
    return ORACLE_OK;
}

/*
 * Backward pass: the exact gradient of the scan above.  The pages define only
 * the forward propagation (GSPN-2 notes, "2D spatial propagation recap") and
 * list forward/backward runtime among the measured quantities (GSPN-2
 * summary page, "Experimental setup"); the gradient is the derivative of
 * that definition, written out step by step:
 *
 *   forward, in scan order t (line i = t or S-1-t):
 *     h_t = M_t h_{t-1} + u_t,   u_t[k] = lambda_t[k] x_t[k],
 *     (M_t v)[k] = sum_o w_t[k,o] v[k+o],   M_t = 0 at the first step of a chunk
 *   with g_t = dL/dh_t coming from y (y = sum of the four h), the adjoint runs
 *   backwards in t:
 *     a_t = g_t + M_{t+1}^T a_{t+1}   (no M_{t+1} term past the chunk's end),
 *     (M^T v)[k] = sum_o w[k-o, o] v[k-o]
 *   and
 *     d lambda_t[k] = a_t[k] x_t[k],      dx_t[k] += a_t[k] lambda_t[k],
 *     dw_t[k,o]     = a_t[k] h_{t-1}[k+o] (existing neighbours, not at a chunk start),
 *     dz_t[k,q]     = sum_o dw_t[k,o] d w_t[k,o] / d z_t[k,q]
 *                   = w_q (1 - s_q) (dw_q - sum_o dw_o w_o)   for existing q, else 0,
 *   with s_q = sigmoid(z_q) and w_q = s_q / sum_existing s (the derivative of
 *   the row normalisation).  Channel-shared logits receive the sum over
 *   channels.
 *
 * oracle_scan_backward: one direction.  gy [n][c][h][w] (array frame) is
 * dL/dy; dx (array frame) is accumulated (+=); dlam [n][c][S][L] is written;
 * dlogits [n][cw][3][S][L] is accumulated (+=).  Planes run in parallel only
 * for per-channel logits (shared logits are summed over channels in order).
 */
int oracle_scan_backward(int dir, int64_t chunk, int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw,
                         const double* x, const double* logits, const double* lam, const double* gy,
                         double* dx, double* dlam, double* dlogits) {
    if (dir < 0 || dir > 3 || chunk < 0 || n < 0 || c < 0 || h < 0 || w < 0) return ORACLE_BAD_ARG;
    if (!(cw == 1 || cw == c)) return ORACLE_BAD_ARG;
    if (!x || !logits || !lam || !gy || !dx || !dlam || !dlogits) return ORACLE_BAD_ARG;
    int64_t S, L;
    frame_sizes(dir, h, w, &S, &L);
    const int64_t plane = S * L;
    const int horizontal = dir_is_horizontal(dir);
    const int reversed = dir_is_reversed(dir);
    const int64_t K = (chunk == 0 || chunk >= S) ? S : chunk;
    const int64_t nplanes = n * c;
    const int shared = (cw == 1 && c > 1);

#pragma omp parallel for schedule(dynamic, 1) if (!shared)
    for (int64_t p = 0; p < nplanes; ++p) {
        const int64_t ni = p / (c > 0 ? c : 1);
        const int64_t ci = p % (c > 0 ? c : 1);
        const int64_t wplane = ni * cw + (cw == 1 ? 0 : ci);
        const double* xp = x + p * plane;
        const double* zp = logits + wplane * 3 * plane;
        const double* lp = lam + p * plane;
        const double* gp = gy + p * plane;
        double* dxp = dx + p * plane;
        double* dlp = dlam + p * plane;
        double* dzp = dlogits + wplane * 3 * plane;

        /* forward states of every step, h[t][k], and the weights w[t][k][o] */
        double* hs = (double*)calloc((size_t)(plane > 0 ? plane : 1), sizeof(double));
        double* ws = (double*)calloc((size_t)(3 * plane > 0 ? 3 * plane : 1), sizeof(double));
        double* ss = (double*)calloc((size_t)(3 * plane > 0 ? 3 * plane : 1), sizeof(double));
        double* anext = (double*)calloc((size_t)(L > 0 ? L : 1), sizeof(double));
        double* acur = (double*)calloc((size_t)(L > 0 ? L : 1), sizeof(double));
        for (int64_t t = 0; t < S; ++t) {
            const int64_t i = reversed ? (S - 1 - t) : t;
            for (int64_t k = 0; k < L; ++k) {
                double z[3], ww[3];
                for (int o = 0; o < 3; ++o) z[o] = zp[o * plane + i * L + k];
                normalise_row(z, k, L, ww);
                for (int o = 0; o < 3; ++o) {
                    const int64_t nb = k + (o - 1);
                    ws[(t * L + k) * 3 + o] = ww[o];
                    ss[(t * L + k) * 3 + o] = (nb >= 0 && nb < L) ? sigmoid(z[o]) : 0.0;
                }
            }
        }
        for (int64_t t = 0; t < S; ++t) {
            const int64_t i = reversed ? (S - 1 - t) : t;
            const int chunk_start = (t % K) == 0;
            for (int64_t k = 0; k < L; ++k) {
                const int64_t aidx = horizontal ? (k * w + i) : (i * w + k);
                double acc = lp[i * L + k] * xp[aidx];
                if (!chunk_start) {
                    for (int o = 0; o < 3; ++o) {
                        const int64_t nb = k + (o - 1);
                        if (nb >= 0 && nb < L) acc += ws[(t * L + k) * 3 + o] * hs[(t - 1) * L + nb];
                    }
                }
                hs[t * L + k] = acc;
            }
        }

        /* adjoint, t = S-1 down to 0 */
        for (int64_t k = 0; k < L; ++k) anext[k] = 0.0;
        for (int64_t t = S - 1; t >= 0; --t) {
            const int64_t i = reversed ? (S - 1 - t) : t;
            const int next_in_chunk = (t + 1 < S) && ((t + 1) % K) != 0;
            for (int64_t k = 0; k < L; ++k) {
                const int64_t aidx = horizontal ? (k * w + i) : (i * w + k);
                double a = gp[aidx];
                if (next_in_chunk) {
                    for (int o = 0; o < 3; ++o) {
                        const int64_t m = k - (o - 1); /* row m of M_{t+1} reads position k with offset o */
                        if (m >= 0 && m < L) a += ws[((t + 1) * L + m) * 3 + o] * anext[m];
                    }
                }
                acur[k] = a;
            }
            const int chunk_start = (t % K) == 0;
            for (int64_t k = 0; k < L; ++k) {
                const int64_t aidx = horizontal ? (k * w + i) : (i * w + k);
                const double a = acur[k];
                dlp[i * L + k] = a * xp[aidx];
                dxp[aidx] += a * lp[i * L + k];
                if (!chunk_start) {
                    double dw[3] = {0.0, 0.0, 0.0};
                    double dot = 0.0;
                    for (int o = 0; o < 3; ++o) {
                        const int64_t nb = k + (o - 1);
                        if (nb >= 0 && nb < L) dw[o] = a * hs[(t - 1) * L + nb];
                        dot += dw[o] * ws[(t * L + k) * 3 + o];
                    }
                    for (int q = 0; q < 3; ++q) {
                        const int64_t nb = k + (q - 1);
                        if (nb < 0 || nb >= L) continue;
                        const double wq = ws[(t * L + k) * 3 + q];
                        const double sq = ss[(t * L + k) * 3 + q];
                        dzp[q * plane + i * L + k] += wq * (1.0 - sq) * (dw[q] - dot);
                    }
                }
            }
            double* tmp = anext;
            anext = acur;
            acur = tmp;
        }
        free(hs);
        free(ws);
        free(ss);
        free(anext);
        free(acur);
    }
    return ORACLE_OK;
}

/*
 * oracle_backward4: gradient of y = sum_d scan_d(x, logits[d], lam[d]) for
 * dL/dy = gy: dx (written), dlam[d] (written), dlogits[d] (written).
 */
int oracle_backward4(int64_t n, int64_t c, int64_t h, int64_t w, int64_t cw, int64_t chunk,
                     const double* x, const double* const* logits, const double* const* lam, const double* gy,
                     double* dx, double* const* dlam, double* const* dlogits) {
    if (!logits || !lam || !gy || !dx || !dlam || !dlogits) return ORACLE_BAD_ARG;
    const int64_t total = n * c * h * w;
    const int64_t ztotal = n * cw * 3 * h * w;
    for (int64_t e = 0; e < total; ++e) dx[e] = 0.0;
    for (int d = 0; d < 4; ++d) {
        for (int64_t e = 0; e < ztotal; ++e) dlogits[d][e] = 0.0;
        int rc = oracle_scan_backward(d, chunk, n, c, h, w, cw, x, logits[d], lam[d], gy, dx, dlam[d], dlogits[d]);
        if (rc != ORACLE_OK) return rc;
    }
    return ORACLE_OK;
}

/*
 * oracle_project: the 1x1 projection between channel spaces (GSPN-2 notes,
 * "Optimisation 2", compressive proxy): out[n][o][p] = sum_c W[o][c] in[n][c][p]
 * for every pixel p.  No bias.
 */
int oracle_project(int64_t n, int64_t c_in, int64_t hw, int64_t c_out, const double* in,
                   const double* weight, double* out) {
    if (n < 0 || c_in < 0 || hw < 0 || c_out < 0 || !in || !weight || !out) return ORACLE_BAD_ARG;
    /* Pixels are taken in blocks only so that the channel planes are walked
     * contiguously; every output is still the sum over c in order 0..c_in-1. */
    const int64_t blk = 1024;
    const int64_t nblk = (hw + blk - 1) / blk;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t ni = 0; ni < n; ++ni) {
        for (int64_t b = 0; b < nblk; ++b) {
            const int64_t p0 = b * blk;
            const int64_t p1 = (p0 + blk < hw) ? p0 + blk : hw;
            for (int64_t o = 0; o < c_out; ++o) {
                double* op = out + (ni * c_out + o) * hw;
                for (int64_t pix = p0; pix < p1; ++pix) op[pix] = 0.0;
                for (int64_t ci = 0; ci < c_in; ++ci) {
                    const double wv = weight[o * c_in + ci];
                    const double* ip = in + (ni * c_in + ci) * hw;
                    for (int64_t pix = p0; pix < p1; ++pix) op[pix] += wv * ip[pix];
                }
            }
        }
    }
    return ORACLE_OK;
}

int oracle_abi_version(void) { return 1; }

/* Threads an OpenMP parallel region of this library may use. */
int oracle_max_threads(void) { return omp_get_max_threads(); }
