/*
 * gspn_oracle.c -- plain fp64 CPU oracle for the GSPN 4-direction line scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header or constant with the HIP library; the product path never
 * calls it.
 *
 * What it computes (written from the method's definition, not from any
 * listing):
 *
 *  - "Parallel Sequence Modeling via Generalized Spatial Propagation
 *    Network" (CVPR 2025 paper notes), section "Key design 1: stability-
 *    context condition": the 2D linear propagation h_i = w_i h_{i-1} +
 *    lambda_i (.) x_i over the lines of the grid; each w_i is made
 *    row-stochastic by applying a sigmoid to the non-zero entries of each of
 *    its rows and dividing by the row sum.
 *  - same notes, section "Key design 2: tridiagonal matrix + 4-direction line
 *    scan": each pixel connects to the 3 adjacent pixels of the previous line
 *    (for the top-to-bottom scan: top-left, top, top-right), so w_i is
 *    tridiagonal; the scan runs in 4 directions and the results are merged.
 *  - same notes, section "Key design 3: global/local variants": the local
 *    variant splits one spatial dimension into g non-overlapping groups that
 *    propagate independently.
 *
 * Readings taken where the pages are silent (each one is a convention the
 * HIP library documents identically):
 *  - the previous state before the first line of a group is zero, so the
 *    first line of every group is h = lambda * x (its raw taps are unused);
 *  - the weights of line i are stored at the destination pixel of line i;
 *  - tap t = 0, 1, 2 couples position p to position p-1, p, p+1 of the
 *    previous line, in absolute grid coordinates for all four directions;
 *  - at a line border the missing tap is dropped and the remaining sigmoids
 *    are renormalised (a line of length 1 has the single weight 1);
 *  - the local groups split each direction's scan axis into g equal
 *    segments; the state restarts at each segment's first line;
 *  - the merge is y = u * sum over the enabled directions of h_dir, with
 *    lambda and u shared by all directions and the raw taps per direction;
 *  - channel c uses weight set c / cpw (compact multi-channel mode).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { DIR_TB = 0, DIR_BT = 1, DIR_LR = 2, DIR_RL = 3 };

/* Grid coordinates (r, q) of position p on line i of direction d. */
static void pixel_of(int d, int64_t H, int64_t W, int64_t i, int64_t p, int64_t *r, int64_t *q)
{
    switch (d) {
    case DIR_TB: *r = i;         *q = p;         break;
    case DIR_BT: *r = H - 1 - i; *q = p;         break;
    case DIR_LR: *r = p;         *q = i;         break;
    default:     *r = p;         *q = W - 1 - i; break;
    }
}

static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/*
 * One (b, c) slice.
 *   x, lam, u : [H][W]
 *   w         : [popcount(dirs)][3][H][W], raw taps of this slice's weight
 *               set, one slab per enabled direction in ascending bit order
 *   y         : [H][W] output
 *   work      : 3 * max(H, W) + H * W doubles of scratch
 * Returns 0, or -1 on a bad argument.
 */
static int slice_fwd(const double *x, const double *w, const double *lam, const double *u,
                     double *y, int64_t H, int64_t W, uint32_t dirs, int32_t groups, double *work)
{
    const int64_t HW = H * W;
    const int64_t mmax = H > W ? H : W;
    double *h = work;
    double *hn = work + mmax;
    double *acc = work + 2 * mmax;
    memset(acc, 0, sizeof(double) * (size_t)HW);

    int slab = 0;
    for (int d = 0; d < 4; ++d) {
        if (!((dirs >> d) & 1u))
            continue;
        const double *wd = w + (int64_t)slab * 3 * HW;
        ++slab;
        const int64_t n = (d == DIR_TB || d == DIR_BT) ? H : W; /* lines */
        const int64_t m = (d == DIR_TB || d == DIR_BT) ? W : H; /* positions per line */
        if (n % groups)
            return -1;
        const int64_t L = n / groups; /* lines per group */

        for (int64_t i = 0; i < n; ++i) {
            for (int64_t p = 0; p < m; ++p) {
                int64_t r, q;
                pixel_of(d, H, W, i, p, &r, &q);
                const double xl = lam[r * W + q] * x[r * W + q];
                if (i % L == 0) {
                    hn[p] = xl; /* zero state before a group's first line */
                    continue;
                }
                /* sigmoid of the taps that exist, then divide by their sum */
                double s[3] = {0.0, 0.0, 0.0};
                double ssum = 0.0;
                for (int t = 0; t < 3; ++t) {
                    const int64_t pp = p + t - 1;
                    if (pp < 0 || pp >= m)
                        continue;
                    s[t] = sigmoid(wd[(int64_t)t * HW + r * W + q]);
                    ssum += s[t];
                }
                double v = xl;
                for (int t = 0; t < 3; ++t) {
                    const int64_t pp = p + t - 1;
                    if (pp < 0 || pp >= m)
                        continue;
                    v += (s[t] / ssum) * h[pp];
                }
                hn[p] = v;
            }
            for (int64_t p = 0; p < m; ++p) {
                int64_t r, q;
                pixel_of(d, H, W, i, p, &r, &q);
                acc[r * W + q] += hn[p];
                h[p] = hn[p];
            }
        }
    }
    for (int64_t j = 0; j < HW; ++j)
        y[j] = u[j] * acc[j];
    return 0;
}

static int ndirs_of(uint32_t dirs)
{
    int k = 0;
    for (int d = 0; d < 4; ++d)
        k += (int)((dirs >> d) & 1u);
    return k;
}

static int check_args(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs,
                      int32_t groups, int32_t cpw)
{
    if (B <= 0 || C <= 0 || H <= 0 || W <= 0)
        return -2;
    if (dirs == 0 || (dirs & ~15u))
        return -3;
    if (groups < 1)
        return -4;
    if (((dirs & 3u) && H % groups) || ((dirs & 12u) && W % groups))
        return -4;
    if (cpw < 1 || C % cpw)
        return -5;
    return 0;
}

/*
 * Whole tensors.
 *   x, lam, u, y : [B][C][H][W]
 *   w            : [popcount(dirs)][B][C/cpw][3][H][W]
 * nthreads <= 0 uses the OpenMP default.  Returns 0 or a negative code.
 */
int gspn_oracle_fwd_f64(const double *x, const double *w, const double *lam, const double *u,
                        double *y, int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs,
                        int32_t groups, int32_t cpw, int nthreads)
{
    int rc = check_args(B, C, H, W, dirs, groups, cpw);
    if (rc)
        return rc;
    if (!x || !w || !lam || !u || !y)
        return -1;
    const int64_t HW = H * W;
    const int64_t Cw = C / cpw;
    const int nd = ndirs_of(dirs);
    const int64_t mmax = H > W ? H : W;
    const int64_t nslices = B * C;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(2 * mmax + HW));
        /* per-slice gather of this slice's weight slabs */
        double *wsl = (double *)malloc(sizeof(double) * (size_t)(nd * 3 * HW));
        if (!work || !wsl) {
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t s = 0; s < nslices; ++s) {
                const int64_t b = s / C, c = s % C, k = c / cpw;
                for (int j = 0; j < nd; ++j)
                    memcpy(wsl + (int64_t)j * 3 * HW,
                           w + (((int64_t)j * B + b) * Cw + k) * 3 * HW,
                           sizeof(double) * (size_t)(3 * HW));
                const int64_t off = s * HW;
                if (slice_fwd(x + off, wsl, lam + off, u + off, y + off, H, W, dirs, groups, work))
                    bad = 1;
            }
        }
        free(work);
        free(wsl);
    }
    return bad ? -2 : 0;
}

/*
 * One slice from its own inputs (for sampled checks on large tensors).
 *   x, lam, u, y : [H][W];  w : [popcount(dirs)][3][H][W]
 */
int gspn_oracle_slice_f64(const double *x, const double *w, const double *lam, const double *u,
                          double *y, int64_t H, int64_t W, uint32_t dirs, int32_t groups)
{
    int rc = check_args(1, 1, H, W, dirs, groups, 1);
    if (rc)
        return rc;
    if (!x || !w || !lam || !u || !y)
        return -1;
    const int64_t mmax = H > W ? H : W;
    double *work = (double *)malloc(sizeof(double) * (size_t)(2 * mmax + H * W));
    if (!work)
        return -2;
    rc = slice_fwd(x, w, lam, u, y, H, W, dirs, groups, work);
    free(work);
    return rc;
}

int gspn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Backward: the exact vector-Jacobian product of the forward above.
 *
 * The pages state only that a backward pass exists and gains about as much
 * as the forward ("GSPN-2: Efficient Parallel Sequence Modeling", author
 * response, paragraph "Backward Benchmark"); the gradients
 * below are the chain rule applied to the forward's definition, written out
 * step by step:
 *
 *   y = u * S,  S = sum_d h_d          =>  gu = gy * S,  gh = gy * u
 *   h_i = w_i h_{i-1} + lam_i * x_i    =>  adjoint state, run from the last
 *       line of a group back to its first:
 *         g_i = gh_i + w_{i+1}^T g_{i+1}     (second term only when line i+1
 *                                             is in the same group)
 *       and, per direction, G = sum over that direction's g at each pixel:
 *         gx  += lam * g,  glam += x * g
 *         dL/dw_t[i][p] = g_i[p] * h_{i-1}[p+t-1]   (valid taps, i not a
 *                                                    group's first line)
 *   w_t = s_t / sum_v s_v, s = sigmoid(a)  =>
 *         ga_t = s_t (1 - s_t) / sum_v s_v * (dw_t - sum_v dw_v w_v)
 *       for valid taps; unused taps (missing neighbours, first lines of
 *       groups) get 0.  dw is summed over the cpw channels sharing the set
 *       before this step (the step is linear in dw).
 * ---------------------------------------------------------------------- */

/* Normalised weights and sigmoids of pixel p of line i (direction d), valid
 * taps only; invalid taps get w = s = 0.  Returns the sigmoid sum. */
static double line_taps(const double *wd, int d, int64_t H, int64_t W, int64_t i, int64_t p,
                        int64_t m, double wt[3], double st[3])
{
    const int64_t HW = H * W;
    int64_t r, q;
    pixel_of(d, H, W, i, p, &r, &q);
    double ssum = 0.0;
    for (int t = 0; t < 3; ++t) {
        const int64_t pp = p + t - 1;
        st[t] = 0.0;
        if (pp < 0 || pp >= m)
            continue;
        st[t] = sigmoid(wd[(int64_t)t * HW + r * W + q]);
        ssum += st[t];
    }
    for (int t = 0; t < 3; ++t)
        wt[t] = st[t] / ssum;
    return ssum;
}

/*
 * One weight set (b, k) and its cpw channels, one direction at a time.
 *   x, lam, u, gy, gx, glam, gu : [cpw][H][W] (this set's channels)
 *   w, gw : [popcount(dirs)][3][H][W] (this set's slabs; gw written fully)
 *   work  : H*W (forward states) + 2*max(H,W) + 2*H*W doubles
 */
static int set_bwd(const double *x, const double *w, const double *lam, const double *u,
                   const double *gy, double *gx, double *gw, double *glam, double *gu,
                   int64_t H, int64_t W, uint32_t dirs, int32_t groups, int32_t cpw, double *work)
{
    const int64_t HW = H * W;
    const int64_t mmax = H > W ? H : W;
    double *hist = work;              /* [n][m] forward states of one direction */
    double *g = work + HW;            /* adjoint of line i */
    double *gn = g + mmax;            /* adjoint of line i + 1 */
    double *G = gn + mmax;            /* [H][W] sum over directions of the adjoint */
    double *S = G + HW;               /* [H][W] sum over directions of h */
    const int nd = ndirs_of(dirs);
    memset(gw, 0, sizeof(double) * (size_t)(nd * 3 * HW));

    for (int32_t c = 0; c < cpw; ++c) {
        const double *xc = x + c * HW, *lc = lam + c * HW, *uc = u + c * HW, *gyc = gy + c * HW;
        memset(G, 0, sizeof(double) * (size_t)HW);
        memset(S, 0, sizeof(double) * (size_t)HW);
        int slab = 0;
        for (int d = 0; d < 4; ++d) {
            if (!((dirs >> d) & 1u))
                continue;
            const double *wd = w + (int64_t)slab * 3 * HW;
            double *gwd = gw + (int64_t)slab * 3 * HW;
            ++slab;
            const int64_t n = (d == DIR_TB || d == DIR_BT) ? H : W;
            const int64_t m = (d == DIR_TB || d == DIR_BT) ? W : H;
            if (n % groups)
                return -1;
            const int64_t L = n / groups;
            double wt[3], st[3];

            /* forward, keeping every line's state */
            for (int64_t i = 0; i < n; ++i) {
                for (int64_t p = 0; p < m; ++p) {
                    int64_t r, q;
                    pixel_of(d, H, W, i, p, &r, &q);
                    double v = lc[r * W + q] * xc[r * W + q];
                    if (i % L != 0) {
                        line_taps(wd, d, H, W, i, p, m, wt, st);
                        for (int t = 0; t < 3; ++t) {
                            const int64_t pp = p + t - 1;
                            if (pp >= 0 && pp < m)
                                v += wt[t] * hist[(i - 1) * m + pp];
                        }
                    }
                    hist[i * m + p] = v;
                    S[r * W + q] += v;
                }
            }

            /* adjoint, last line first */
            for (int64_t i = n - 1; i >= 0; --i) {
                for (int64_t p = 0; p < m; ++p) {
                    int64_t r, q;
                    pixel_of(d, H, W, i, p, &r, &q);
                    g[p] = gyc[r * W + q] * uc[r * W + q];
                }
                if (i + 1 < n && (i + 1) % L != 0) {
                    /* + w_{i+1}^T g_{i+1}: pixel p' of line i+1 reads p'+t-1 */
                    for (int64_t pq = 0; pq < m; ++pq) {
                        line_taps(wd, d, H, W, i + 1, pq, m, wt, st);
                        for (int t = 0; t < 3; ++t) {
                            const int64_t pp = pq + t - 1;
                            if (pp >= 0 && pp < m)
                                g[pp] += wt[t] * gn[pq];
                        }
                    }
                }
                for (int64_t p = 0; p < m; ++p) {
                    int64_t r, q;
                    pixel_of(d, H, W, i, p, &r, &q);
                    G[r * W + q] += g[p];
                    if (i % L != 0) {
                        for (int t = 0; t < 3; ++t) {
                            const int64_t pp = p + t - 1;
                            if (pp < 0 || pp >= m)
                                continue;
                            gwd[(int64_t)t * HW + r * W + q] += g[p] * hist[(i - 1) * m + pp];
                        }
                    }
                }
                memcpy(gn, g, sizeof(double) * (size_t)m);
            }
        }
        for (int64_t j = 0; j < HW; ++j) {
            gx[c * HW + j] = lc[j] * G[j];
            glam[c * HW + j] = xc[j] * G[j];
            gu[c * HW + j] = gyc[j] * S[j];
        }
    }

    /* through sigmoid-then-normalise: dL/dw -> dL/da, in place */
    int slab = 0;
    for (int d = 0; d < 4; ++d) {
        if (!((dirs >> d) & 1u))
            continue;
        const double *wd = w + (int64_t)slab * 3 * HW;
        double *gwd = gw + (int64_t)slab * 3 * HW;
        ++slab;
        const int64_t n = (d == DIR_TB || d == DIR_BT) ? H : W;
        const int64_t m = (d == DIR_TB || d == DIR_BT) ? W : H;
        const int64_t L = n / groups;
        for (int64_t i = 0; i < n; ++i) {
            for (int64_t p = 0; p < m; ++p) {
                int64_t r, q;
                pixel_of(d, H, W, i, p, &r, &q);
                double *gp[3];
                for (int t = 0; t < 3; ++t)
                    gp[t] = gwd + (int64_t)t * HW + r * W + q;
                if (i % L == 0) {
                    for (int t = 0; t < 3; ++t)
                        *gp[t] = 0.0;
                    continue;
                }
                double wt[3], st[3];
                const double ssum = line_taps(wd, d, H, W, i, p, m, wt, st);
                double dot = 0.0;
                for (int t = 0; t < 3; ++t)
                    dot += *gp[t] * wt[t];
                for (int t = 0; t < 3; ++t)
                    *gp[t] = st[t] * (1.0 - st[t]) / ssum * (*gp[t] - dot);
            }
        }
    }
    return 0;
}

/*
 * Whole tensors, same layouts as gspn_oracle_fwd_f64; gy is dL/dy.
 * Outputs gx, glam, gu : [B][C][H][W] and gw : [popcount(dirs)][B][C/cpw][3][H][W]
 * (dL/d raw taps), all fully written.  OpenMP over weight sets (b, k).
 */
int gspn_oracle_bwd_f64(const double *x, const double *w, const double *lam, const double *u,
                        const double *gy, double *gx, double *gw, double *glam, double *gu,
                        int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs,
                        int32_t groups, int32_t cpw, int nthreads)
{
    int rc = check_args(B, C, H, W, dirs, groups, cpw);
    if (rc)
        return rc;
    if (!x || !w || !lam || !u || !gy || !gx || !gw || !glam || !gu)
        return -1;
    const int64_t HW = H * W;
    const int64_t Cw = C / cpw;
    const int nd = ndirs_of(dirs);
    const int64_t mmax = H > W ? H : W;
    const int64_t nsets = B * Cw;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(3 * HW + 2 * mmax));
        double *wsl = (double *)malloc(sizeof(double) * (size_t)(2 * nd * 3 * HW));
        if (!work || !wsl) {
            bad = 1;
        } else {
            double *gsl = wsl + (int64_t)nd * 3 * HW;
#pragma omp for schedule(dynamic, 1)
            for (int64_t s = 0; s < nsets; ++s) {
                const int64_t b = s / Cw, k = s % Cw;
                for (int j = 0; j < nd; ++j)
                    memcpy(wsl + (int64_t)j * 3 * HW,
                           w + (((int64_t)j * B + b) * Cw + k) * 3 * HW,
                           sizeof(double) * (size_t)(3 * HW));
                const int64_t off = (b * C + k * cpw) * HW;
                if (set_bwd(x + off, wsl, lam + off, u + off, gy + off, gx + off, gsl,
                            glam + off, gu + off, H, W, dirs, groups, cpw, work))
                    bad = 1;
                for (int j = 0; j < nd; ++j)
                    memcpy(gw + (((int64_t)j * B + b) * Cw + k) * 3 * HW,
                           gsl + (int64_t)j * 3 * HW, sizeof(double) * (size_t)(3 * HW));
            }
        }
        free(work);
        free(wsl);
    }
    return bad ? -2 : 0;
}
