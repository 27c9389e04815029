/*
 * gs_oracle.c -- CPU float64 oracle for tile-based Gaussian-splat rasterization.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the test oracle, not the product: it is
 * built and called by the tests, by the package's smoke check and by the
 * benchmark's CPU-baseline leg, never by the library itself. It shares no code
 * with the HIP kernels.
 *
 * What it computes (a plain definition, written out per pixel):
 *
 *   The backward pass named on page "Phase 5 step 30b — kernel-by-kernel
 *   timing" (section ホットスポット ranking, item 1: nine per-splat gradient
 *   fields -- 2D mean, conic, RGB, opacity -- summed over all pixels) and on
 *   the Spirula Studio page (从 8.6 KB 到 4.2 KB, section 机制拆解: the 2D
 *   screen-space path rasterize_bwd_2d, with an optional accumulated-weight
 *   output). Neither page prints the compositing formula; the reading used is
 *   the standard tile-based 3D Gaussian splatting rule:
 *
 *     pixel centre p = (x + 0.5, y + 0.5), d = p - mean
 *     sigma = -1/2 (a dx^2 + c dy^2) - b dx dy        (conic = (a, b, c))
 *     G = exp(sigma),  alpha = min(0.99, opacity * G)
 *     walk the tile's depth-sorted list front to back:
 *       skip the splat if alpha < 1/255
 *       stop (without compositing it) if T (1 - alpha) < 1e-4
 *       else  C += colour alpha T,  T *= (1 - alpha)
 *     image = C + T bg,  final_T = T,  n_contrib = list position of the last
 *     composited splat + 1 (0 if none)
 *
 *   Backward: L = sum_p <g_p, image_p> with g = dL/dImage; the exact partial
 *   derivatives of L with respect to each stored per-splat scalar, with the
 *   discrete decisions (skip set, stop point, clamp state) held fixed:
 *     dL/dcolour_i  = sum_p alpha_i T_i g_p
 *     dL/dalpha_i   = sum_p <g_p, colour_i T_i - S_i / (1 - alpha_i)>,
 *                     S_i = sum_{j>i} colour_j alpha_j T_j + T_final bg
 *     if not clamped: dL/dsigma = alpha dL/dalpha, dL/dopacity = G dL/dalpha,
 *       dL/da = -dx^2/2 dL/dsigma, dL/db = -dx dy dL/dsigma,
 *       dL/dc = -dy^2/2 dL/dsigma,
 *       dL/dmean = (a dx + b dy, b dx + c dy) dL/dsigma
 *     accum_weight_i = sum_p alpha_i T_i over composited pairs
 *
 *   Max weight (the "max wt" line of the Spirula Studio page's raster_bench,
 *   section 亲手验证, which names it without a formula; read as the largest
 *   compositing weight a splat receives):
 *     max_weight_i = max_p alpha_i T_i over composited pairs (0 if none)
 *
 *   Depth terms (gso_forward_depth / gso_backward_depth, below): the
 *   distortion and median-depth options of rasterize_bwd_2d that the Spirula
 *   Studio page names (section 机制拆解) without formulas; read as the squared
 *   distortion over a pixel's composited pairs and the depth where its
 *   transmittance falls to 1/2.
 *
 *   Unlike the kernels this evaluates T forwards (products) and S as a suffix
 *   sum, in float64, with no division recurrence.
 *
 * Ambiguity flags: the kernels decide the three thresholds in float32. For
 * each decision this file also computes a bound on how far a float32
 * evaluation can be from the float64 value; a pixel is flagged when any of its
 * decisions lies inside that band (several results are then correct).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TILE 16
#define ALPHA_MAX 0.99
#define ALPHA_MIN (1.0 / 255.0)
#define T_MIN 1e-4

/* unit roundoff of float32, and the guard-band scale factors */
static const double U32 = 5.9604644775390625e-08; /* 2^-24 */
static const double K_ALPHA = 4.0;
static const double K_T = 2.0;

typedef struct {
    const double* means;   /* [n][2] */
    const double* conics;  /* [n][3] */
    const double* colors;  /* [n][3] */
    const double* opac;    /* [n]    */
    double bg[3];
} splats_t;

/* One walked entry of a pixel: enough to form its gradient afterwards. */
typedef struct {
    int32_t k;       /* position in the tile list */
    double alpha, T, G, dx, dy;
    int clamped;
    double errT;     /* float32 error bound of T (relative), before this entry */
} contrib_t;

/* Relative error bound of a float32 evaluation of alpha at this pair. */
static double alpha_rel_bound(double a, double b, double c, double dx, double dy, double sigma)
{
    double m = fabs(a) * dx * dx + fabs(c) * dy * dy + 2.0 * fabs(b * dx * dy);
    return K_ALPHA * U32 * (4.0 + m + fabs(sigma));
}

/* The three decision bands: 1 when a float32 evaluation (alpha within relative
 * error ea, T(1 - alpha) within relative error et) may take the decision the
 * other way. */
static int in_skip_band(double alpha, double ea)
{
    return fabs(alpha - ALPHA_MIN) <= ea * alpha + 2.0 * U32 * ALPHA_MIN;
}

static int in_clamp_band(double ah, double ea)
{
    return fabs(ah - ALPHA_MAX) <= ea * ah + 2.0 * U32;
}

static int in_stop_band(double test, double et)
{
    return fabs(test - T_MIN) <= K_T * et * T_MIN + 1e-6 * T_MIN;
}

/* Splat i at pixel centre (px, py): offset, sigma, G, unclamped and clamped
 * alpha, and the float32 error bound of alpha. */
typedef struct {
    double dx, dy, sigma, G, ah, alpha, ea;
} pair_t;

static pair_t eval_pair(const splats_t* s, int32_t i, double px, double py)
{
    pair_t q;
    double a = s->conics[3 * i], b = s->conics[3 * i + 1], c = s->conics[3 * i + 2];
    q.dx = px - s->means[2 * i];
    q.dy = py - s->means[2 * i + 1];
    q.sigma = -0.5 * (a * q.dx * q.dx + c * q.dy * q.dy) - b * q.dx * q.dy;
    q.G = exp(q.sigma);
    q.ah = s->opac[i] * q.G;
    q.alpha = q.ah < ALPHA_MAX ? q.ah : ALPHA_MAX;
    q.ea = alpha_rel_bound(a, b, c, q.dx, q.dy, q.sigma);
    return q;
}

/*
 * Walk one pixel's list front to back. Fills `out` (capacity `cap`) with the
 * composited entries, returns how many; writes T_final, n_contrib, colour sum
 * and the ambiguity flag.
 */
static int walk_pixel(const splats_t* s, const int32_t* ids, int32_t start, int32_t end,
                      double px, double py, contrib_t* out, int cap,
                      double* T_out, int32_t* nc_out, double C[3], int* amb_out, int32_t* kamb_out)
{
    double T = 1.0, errT = 0.0;
    int cnt = 0, amb = 0;
    int32_t last = 0, kamb = end;
    C[0] = C[1] = C[2] = 0.0;
    for (int32_t k = start; k < end; ++k) {
        int32_t i = ids[k];
        const pair_t q = eval_pair(s, i, px, py);
        double ah = q.ah, alpha = q.alpha, ea = q.ea;
        if (in_skip_band(alpha, ea)) amb = 1;
        if (amb && kamb == end) kamb = k;
        if (alpha < ALPHA_MIN) continue;
        if (in_clamp_band(ah, ea)) amb = 1;
        double test = T * (1.0 - alpha);
        double et = errT + ea * alpha / (1.0 - alpha) + 4.0 * U32;
        if (in_stop_band(test, et)) amb = 1;
        if (amb && kamb == end) kamb = k;
        if (test < T_MIN) break;
        const double* col = s->colors + 3 * i;
        C[0] += col[0] * alpha * T;
        C[1] += col[1] * alpha * T;
        C[2] += col[2] * alpha * T;
        if (out && cnt < cap) {
            contrib_t* e = &out[cnt];
            e->k = k; e->alpha = alpha; e->T = T; e->G = q.G; e->dx = q.dx; e->dy = q.dy;
            e->clamped = !(ah < ALPHA_MAX);
            e->errT = errT;
        }
        ++cnt;
        T = test;
        errT += ea * alpha / (1.0 - alpha) + 2.0 * U32;
        last = k - start + 1;
    }
    *T_out = T;
    *nc_out = last;
    *amb_out = amb;
    if (kamb_out) *kamb_out = kamb;
    return cnt;
}

static int threads_used(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int gso_threads(void) { return threads_used(); }

/* Threads of the parallel loops from now on (n >= 1). */
void gso_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Forward over the tiles listed in `tiles` (or all tiles if tiles == NULL).
 * image [H][W][3], final_T [H][W], n_contrib [H][W], amb [H][W]: only pixels
 * of processed tiles are written.
 */
int gso_forward(int W, int H, const int32_t* ranges, const int32_t* ids,
                const double* means, const double* conics, const double* colors, const double* opac,
                const double* bg, const int32_t* tiles, int ntiles,
                double* image, double* final_T, int32_t* n_contrib, uint8_t* amb)
{
    splats_t s = {means, conics, colors, opac, {bg[0], bg[1], bg[2]}};
    int GX = (W + TILE - 1) / TILE, GY = (H + TILE - 1) / TILE;
    int nt = tiles ? ntiles : GX * GY;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ti = 0; ti < nt; ++ti) {
        int t = tiles ? tiles[ti] : ti;
        int tx = t % GX, ty = t / GX;
        int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
        for (int ly = 0; ly < TILE; ++ly) {
            int y = ty * TILE + ly;
            if (y >= H) break;
            for (int lx = 0; lx < TILE; ++lx) {
                int x = tx * TILE + lx;
                if (x >= W) break;
                double T, C[3];
                int32_t nc;
                int a;
                walk_pixel(&s, ids, start, end, x + 0.5, y + 0.5, NULL, 0, &T, &nc, C, &a, NULL);
                size_t p = (size_t)y * W + x;
                image[3 * p + 0] = C[0] + T * s.bg[0];
                image[3 * p + 1] = C[1] + T * s.bg[1];
                image[3 * p + 2] = C[2] + T * s.bg[2];
                final_T[p] = T;
                n_contrib[p] = nc;
                amb[p] = (uint8_t)a;
            }
        }
    }
    return threads_used();
}

/*
 * Backward over the listed tiles. grads [n][9] = (dmean x, dmean y, da, db, dc,
 * dr, dg, db_colour, dopacity), accum_w [n]; both are ADDED to (caller zeroes).
 * dimg [H][W][3] is the upstream gradient g.
 */
/* dL/dalpha of one walked entry carried on to the mean (o[0..1]), the conic
 * (o[2..4]) and the opacity (o[8]); a clamped alpha passes nothing on. */
static void add_alpha_grad(double* o, const contrib_t* q, const double* conic, double dal)
{
    if (q->clamped) return;
    double a_ = conic[0], b_ = conic[1], c_ = conic[2];
    double ds = q->alpha * dal;  /* dL/dsigma */
    o[0] += (a_ * q->dx + b_ * q->dy) * ds;
    o[1] += (b_ * q->dx + c_ * q->dy) * ds;
    o[2] += -0.5 * q->dx * q->dx * ds;
    o[3] += -q->dx * q->dy * ds;
    o[4] += -0.5 * q->dy * q->dy * ds;
    o[8] += q->G * dal;
}

int gso_backward(int W, int H, int n, const int32_t* ranges, const int32_t* ids,
                 const double* means, const double* conics, const double* colors, const double* opac,
                 const double* bg, const double* dimg, const int32_t* tiles, int ntiles,
                 double* grads, double* accum_w)
{
    (void)n;
    splats_t s = {means, conics, colors, opac, {bg[0], bg[1], bg[2]}};
    int GX = (W + TILE - 1) / TILE, GY = (H + TILE - 1) / TILE;
    int nt = tiles ? ntiles : GX * GY;
#pragma omp parallel
    {
        int cap = 0;
        contrib_t* buf = NULL;
        double* part = NULL;  /* per tile-list entry: 9 grads + accum weight */
        int part_cap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int ti = 0; ti < nt; ++ti) {
            int t = tiles ? tiles[ti] : ti;
            int tx = t % GX, ty = t / GX;
            int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
            int L = end - start;
            if (L <= 0) continue;
            if (L > cap) { free(buf); cap = L; buf = (contrib_t*)malloc(sizeof(contrib_t) * cap); }
            if (L > part_cap) { free(part); part_cap = L; part = (double*)malloc(sizeof(double) * 10 * part_cap); }
            memset(part, 0, sizeof(double) * 10 * L);
            for (int ly = 0; ly < TILE; ++ly) {
                int y = ty * TILE + ly;
                if (y >= H) break;
                for (int lx = 0; lx < TILE; ++lx) {
                    int x = tx * TILE + lx;
                    if (x >= W) break;
                    double T, C[3];
                    int32_t nc;
                    int a;
                    int cnt = walk_pixel(&s, ids, start, end, x + 0.5, y + 0.5, buf, cap, &T, &nc, C, &a, NULL);
                    size_t p = (size_t)y * W + x;
                    double g[3] = {dimg[3 * p], dimg[3 * p + 1], dimg[3 * p + 2]};
                    /* S = sum over composited splats behind + T_final bg */
                    double S[3] = {T * s.bg[0], T * s.bg[1], T * s.bg[2]};
                    for (int e = cnt - 1; e >= 0; --e) {
                        const contrib_t* q = &buf[e];
                        int32_t i = ids[q->k];
                        const double* col = s.colors + 3 * i;
                        double al = q->alpha, Ti = q->T;
                        double dal = 0.0;
                        for (int ch = 0; ch < 3; ++ch)
                            dal += g[ch] * (col[ch] * Ti - S[ch] / (1.0 - al));
                        double* o = part + 10 * (q->k - start);
                        double w = al * Ti;
                        o[5] += w * g[0];
                        o[6] += w * g[1];
                        o[7] += w * g[2];
                        add_alpha_grad(o, q, s.conics + 3 * i, dal);
                        o[9] += w;
                        S[0] += col[0] * w;
                        S[1] += col[1] * w;
                        S[2] += col[2] * w;
                    }
                }
            }
#pragma omp critical(gso_merge)
            {
                for (int k = 0; k < L; ++k) {
                    const double* o = part + 10 * k;
                    int32_t i = ids[start + k];
                    for (int f = 0; f < 9; ++f) grads[9 * (size_t)i + f] += o[f];
                    accum_w[i] += o[9];
                }
            }
        }
        free(buf);
        free(part);
    }
    return threads_used();
}

/*
 * Admissible outcomes of one pixel. Where a decision lies inside its band,
 * a float32 walk may take it either way, and both results are correct. This
 * walks the pixel's list front to back like walk_pixel and, at every skip or
 * stop decision inside its band, follows both outcomes (each branch then
 * continues with its own T and its own later decisions and bands). Every leaf is one admissible
 * (image, final_T, n_contrib); at most `cap` are kept, and *overflow is set if
 * there were more.
 */
typedef struct {
    const splats_t* s;
    const int32_t* ids;
    int32_t start, end;
    double px, py;
    double* img;      /* [cap][3] */
    double* T;        /* [cap] */
    int32_t* nc;      /* [cap] */
    int cap, count, overflow;
} explore_t;

/* Walk from list position k0 with the state (T, errT, C, last) reached
 * before it; fs / fc / ft force the skip / clamp / stop decision of entry k0
 * (-1: the float64 decision, with its band followed). */
static void explore(explore_t* e, int32_t k0, int fs, int fc, int ft, double T, double errT, const double C0[3],
                    int32_t last)
{
    const splats_t* s = e->s;
    double C[3] = {C0[0], C0[1], C0[2]};
    for (int32_t k = k0; k < e->end; ++k) {
        if (e->count >= e->cap) { e->overflow = 1; return; }
        int32_t i = e->ids[k];
        const pair_t q = eval_pair(s, i, e->px, e->py);
        double ah = q.ah, alpha = q.alpha, ea = q.ea;
        int first = k == k0;
        int skip = alpha < ALPHA_MIN;
        if (first && fs >= 0) skip = fs;
        else if (in_skip_band(alpha, ea)) explore(e, k, !skip, -1, -1, T, errT, C, last);
        if (skip) continue;
        /* a clamp decided the other way moves alpha by no more than its band
         * (a few ulp), far below the image tolerance, and its effect on the
         * stop decision lies inside the stop band: it is not branched on */
        int clamp = !(ah < ALPHA_MAX);
        if (first && fc >= 0) clamp = fc;
        double al = clamp ? ALPHA_MAX : ah;
        double test = T * (1.0 - al);
        double et = errT + ea * al / (1.0 - al) + 4.0 * U32;
        int stop = test < T_MIN;
        if (first && ft >= 0) stop = ft;
        else if (in_stop_band(test, et)) explore(e, k, 0, clamp, !stop, T, errT, C, last);
        if (stop) break;
        const double* col = s->colors + 3 * i;
        C[0] += col[0] * al * T;
        C[1] += col[1] * al * T;
        C[2] += col[2] * al * T;
        T = test;
        errT += ea * al / (1.0 - al) + 2.0 * U32;
        last = k - e->start + 1;
    }
    if (e->count >= e->cap) { e->overflow = 1; return; }
    double* im = e->img + 3 * (size_t)e->count;
    im[0] = C[0] + T * s->bg[0];
    im[1] = C[1] + T * s->bg[1];
    im[2] = C[2] + T * s->bg[2];
    e->T[e->count] = T;
    e->nc[e->count] = last;
    e->count++;
}

/*
 * Admissible outcomes of the listed pixels (xs[p], ys[p]): img [np][cap][3],
 * T [np][cap], nc [np][cap], count [np] (-1: more than cap outcomes).
 */
int gso_pixel_outcomes(int W, int H, const int32_t* ranges, const int32_t* ids,
                       const double* means, const double* conics, const double* colors, const double* opac,
                       const double* bg, int npix, const int32_t* xs, const int32_t* ys, int cap,
                       double* img, double* T, int32_t* nc, int32_t* count)
{
    splats_t s = {means, conics, colors, opac, {bg[0], bg[1], bg[2]}};
    int GX = (W + TILE - 1) / TILE;
    (void)H;
#pragma omp parallel for schedule(dynamic, 16)
    for (int p = 0; p < npix; ++p) {
        int t = (ys[p] / TILE) * GX + xs[p] / TILE;
        explore_t e = {&s, ids, ranges[2 * t], ranges[2 * t + 1], xs[p] + 0.5, ys[p] + 0.5,
                       img + 3 * (size_t)cap * p, T + (size_t)cap * p, nc + (size_t)cap * p, cap, 0, 0};
        double C[3] = {0.0, 0.0, 0.0};
        explore(&e, e.start, -1, -1, -1, 1.0, 0.0, C, 0);
        count[p] = e.overflow ? -1 : e.count;
    }
    return threads_used();
}

/*
 * Max weight over the listed tiles: max_w [n] = max over composited pairs of
 * alpha T (MAXED into; caller zeroes). max_w_amb [n] (MAXED into) bounds what
 * a float32 walk may give a splat at pixels with an ambiguous decision: up to
 * such a pixel's first ambiguous decision the float32 walk takes the same
 * decisions; from there on, every splat of its list whose alpha reaches the
 * skip threshold (within the error band) may be composited with a weight of
 * at most 1.01 alpha T, T being this walk's transmittance before it, the walk
 * continued past its stop (each flipped skip changes T by a factor within
 * (1 - 1/255)^-1; a flipped clamp changes alpha by a few ulp). A splat whose
 * max_w_amb stays below its max_w less the comparison tolerance has the same
 * maximum in any correct float32 walk. max_w_cert [n] (MAXED into; may be
 * NULL) is the maximum over the pairs composited before their pixel's first
 * ambiguous decision, which every correct float32 walk composites too: a
 * lower bound of any admissible maximum, as max(max_w, max_w_amb) is an upper
 * bound.
 */
int gso_max_weight(int W, int H, int n, const int32_t* ranges, const int32_t* ids,
                   const double* means, const double* conics, const double* colors, const double* opac,
                   const double* bg, const int32_t* tiles, int ntiles, double* max_w, double* max_w_amb,
                   double* max_w_cert)
{
    (void)n;
    splats_t s = {means, conics, colors, opac, {bg[0], bg[1], bg[2]}};
    int GX = (W + TILE - 1) / TILE, GY = (H + TILE - 1) / TILE;
    int nt = tiles ? ntiles : GX * GY;
#pragma omp parallel
    {
        int cap = 0;
        contrib_t* buf = NULL;
        double* part = NULL;   /* per tile-list entry: max weight */
        double* pamb = NULL;   /* per tile-list entry: bound at ambiguous pixels */
        double* pcert = NULL;  /* per tile-list entry: max over pairs before their pixel's first ambiguity */
        int part_cap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int ti = 0; ti < nt; ++ti) {
            int t = tiles ? tiles[ti] : ti;
            int tx = t % GX, ty = t / GX;
            int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
            int L = end - start;
            if (L <= 0) continue;
            if (L > cap) { free(buf); cap = L; buf = (contrib_t*)malloc(sizeof(contrib_t) * cap); }
            if (L > part_cap) {
                free(part); free(pamb); free(pcert); part_cap = L;
                part = (double*)malloc(sizeof(double) * part_cap);
                pamb = (double*)malloc(sizeof(double) * part_cap);
                pcert = (double*)malloc(sizeof(double) * part_cap);
            }
            memset(part, 0, sizeof(double) * L);
            memset(pamb, 0, sizeof(double) * L);
            memset(pcert, 0, sizeof(double) * L);
            for (int ly = 0; ly < TILE; ++ly) {
                int y = ty * TILE + ly;
                if (y >= H) break;
                for (int lx = 0; lx < TILE; ++lx) {
                    int x = tx * TILE + lx;
                    if (x >= W) break;
                    double T, C[3];
                    int32_t nc, kamb;
                    int a;
                    double px = x + 0.5, py = y + 0.5;
                    int cnt = walk_pixel(&s, ids, start, end, px, py, buf, cap, &T, &nc, C, &a, &kamb);
                    for (int e = 0; e < cnt; ++e) {
                        double w = buf[e].alpha * buf[e].T;
                        double* o = part + (buf[e].k - start);
                        if (w > *o) *o = w;
                        double* oc = pcert + (buf[e].k - start);
                        if (buf[e].k < kamb && w > *oc) *oc = w;
                    }
                    if (!a) continue;
                    double Tw = 1.0;  /* this walk's T, continued past its stop */
                    for (int32_t k = start; k < end; ++k) {
                        const pair_t q = eval_pair(&s, ids[k], px, py);
                        double ah = q.ah, alpha = q.alpha, ea = q.ea;
                        if (k >= kamb && ah >= ALPHA_MIN * (1.0 - ea) - 2.0 * U32 * ALPHA_MIN) {
                            double wb = 1.01 * alpha * Tw;
                            double* o = pamb + (k - start);
                            if (wb > *o) *o = wb;
                        }
                        if (alpha >= ALPHA_MIN) Tw *= 1.0 - alpha;
                    }
                }
            }
#pragma omp critical(gso_merge_max)
            {
                for (int k = 0; k < L; ++k) {
                    int32_t i = ids[start + k];
                    if (part[k] > max_w[i]) max_w[i] = part[k];
                    if (pamb[k] > max_w_amb[i]) max_w_amb[i] = pamb[k];
                    if (max_w_cert && pcert[k] > max_w_cert[i]) max_w_cert[i] = pcert[k];
                }
            }
        }
        free(buf);
        free(part);
        free(pamb);
        free(pcert);
    }
    return threads_used();
}

/*
 * Depth terms (the distortion and median-depth options that the Spirula Studio
 * page names in section 机制拆解 -- a per-pixel float4 of "distortion totals"
 * and a median-depth output -- without defining them). Read as:
 *
 *   distortion  D(p) = sum over composited pairs i < j of w_i w_j (z_i - z_j)^2,
 *               w = alpha T, z = the splat's view depth (the squared form of the
 *               mip-NeRF 360 distortion loss over the pixel's composited splats)
 *   median      the depth z_m of the last composited splat m whose transmittance
 *               before it is still > 1/2 (0 when the pixel composites nothing);
 *               m + 1 is reported as the median's list position (0: none)
 *
 * Because D does not change when every depth is shifted, the totals the
 * backward needs are taken about the median depth:
 *   totals = (A, B, C, D),  A = sum w,  B = sum w (z - z_m),  C = sum w (z - z_m)^2
 *
 * median_amb marks a pixel whose median decision (T > 1/2) lies inside the
 * float32 error band of T.
 */
/* The median entry of a walked pixel: the last composited entry whose
 * transmittance before it is > 1/2 (-1 if none). *amb (if given) is set when
 * some entry's T lies inside the float32 error band of 1/2. */
static int median_entry(const contrib_t* buf, int cnt, int* amb)
{
    int m = -1;
    for (int e = 0; e < cnt; ++e) {
        const contrib_t* q = &buf[e];
        if (amb && fabs(q->T - 0.5) <= K_T * (q->errT + 4.0 * U32) * 0.5 + 1e-6 * 0.5) *amb = 1;
        if (q->T > 0.5) m = e;
    }
    return m;
}

/* Totals of a walked pixel about the reference depth zm: A = sum w,
 * B = sum w u, C = sum w u^2 (u = z - zm), and the distortion in list order,
 * D = sum_j w_j (sum_{i<j} w_i (z_i - z_j)^2), the inner sum expanded about zm. */
static void depth_totals(const contrib_t* buf, int cnt, const int32_t* ids, const double* depths, double zm,
                         double* A_, double* B_, double* C_, double* D_)
{
    double A = 0.0, B = 0.0, Cs = 0.0, D = 0.0;
    for (int e = 0; e < cnt; ++e) {
        const contrib_t* q = &buf[e];
        double w = q->alpha * q->T, u = depths[ids[q->k]] - zm;
        D += w * (u * u * A - 2.0 * u * B + Cs);
        A += w;
        B += w * u;
        Cs += w * u * u;
    }
    *A_ = A;
    *B_ = B;
    *C_ = Cs;
    *D_ = D;
}

int gso_forward_depth(int W, int H, const int32_t* ranges, const int32_t* ids,
                      const double* means, const double* conics, const double* colors, const double* opac,
                      const double* bg, const double* depths, const int32_t* tiles, int ntiles,
                      double* totals, double* median, int32_t* median_pos, uint8_t* median_amb)
{
    splats_t s = {means, conics, colors, opac, {bg[0], bg[1], bg[2]}};
    int GX = (W + TILE - 1) / TILE, GY = (H + TILE - 1) / TILE;
    int nt = tiles ? ntiles : GX * GY;
#pragma omp parallel
    {
        int cap = 0;
        contrib_t* buf = NULL;
#pragma omp for schedule(dynamic, 1)
        for (int ti = 0; ti < nt; ++ti) {
            int t = tiles ? tiles[ti] : ti;
            int tx = t % GX, ty = t / GX;
            int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
            int L = end - start;
            if (L > cap) { free(buf); cap = L; buf = (contrib_t*)malloc(sizeof(contrib_t) * cap); }
            for (int ly = 0; ly < TILE; ++ly) {
                int y = ty * TILE + ly;
                if (y >= H) break;
                for (int lx = 0; lx < TILE; ++lx) {
                    int x = tx * TILE + lx;
                    if (x >= W) break;
                    double T, C[3];
                    int32_t nc;
                    int a;
                    int cnt = L > 0 ? walk_pixel(&s, ids, start, end, x + 0.5, y + 0.5, buf, cap, &T, &nc, C, &a, NULL)
                                    : 0;
                    size_t p = (size_t)y * W + x;
                    int amb = 0;
                    int m = median_entry(buf, cnt, &amb);
                    double zm = m >= 0 ? depths[ids[buf[m].k]] : 0.0;
                    double A, B, Cs, D;
                    depth_totals(buf, cnt, ids, depths, zm, &A, &B, &Cs, &D);
                    totals[4 * p + 0] = A;
                    totals[4 * p + 1] = B;
                    totals[4 * p + 2] = Cs;
                    totals[4 * p + 3] = D;
                    median[p] = zm;
                    median_pos[p] = m >= 0 ? buf[m].k - start + 1 : 0;
                    median_amb[p] = (uint8_t)amb;
                }
            }
        }
        free(buf);
    }
    return threads_used();
}

/*
 * Gradients of L_depth = sum_p gD_p D_p + gM_p median_p (upstream g_dist [H][W],
 * g_median [H][W]), every discrete decision held fixed, ADDED into grads [n][9]
 * (the same fields as gso_backward) and ddepth [n]:
 *   dD/dw_k     = sum_i w_i (z_i - z_k)^2 = u_k^2 A - 2 u_k B + C   (u = z - z_m)
 *   dD/dalpha_k = T_k dD/dw_k - (sum_{j>k} w_j dD/dw_j) / (1 - alpha_k)
 *   dD/dz_k     = 2 w_k (u_k A - B)
 *   dmedian/dz_m = 1
 * and dL/dalpha continues to opacity, conic and mean as in gso_backward (no
 * alpha path for a clamped alpha).
 */
int gso_backward_depth(int W, int H, int n, const int32_t* ranges, const int32_t* ids,
                       const double* means, const double* conics, const double* colors, const double* opac,
                       const double* bg, const double* depths, const double* g_dist, const double* g_median,
                       const int32_t* tiles, int ntiles, double* grads, double* ddepth)
{
    (void)n;
    splats_t s = {means, conics, colors, opac, {bg[0], bg[1], bg[2]}};
    int GX = (W + TILE - 1) / TILE, GY = (H + TILE - 1) / TILE;
    int nt = tiles ? ntiles : GX * GY;
#pragma omp parallel
    {
        int cap = 0;
        contrib_t* buf = NULL;
        double* part = NULL;  /* per tile-list entry: 9 grads + ddepth */
        int part_cap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int ti = 0; ti < nt; ++ti) {
            int t = tiles ? tiles[ti] : ti;
            int tx = t % GX, ty = t / GX;
            int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
            int L = end - start;
            if (L <= 0) continue;
            if (L > cap) { free(buf); cap = L; buf = (contrib_t*)malloc(sizeof(contrib_t) * cap); }
            if (L > part_cap) { free(part); part_cap = L; part = (double*)malloc(sizeof(double) * 10 * part_cap); }
            memset(part, 0, sizeof(double) * 10 * L);
            for (int ly = 0; ly < TILE; ++ly) {
                int y = ty * TILE + ly;
                if (y >= H) break;
                for (int lx = 0; lx < TILE; ++lx) {
                    int x = tx * TILE + lx;
                    if (x >= W) break;
                    double T, C[3];
                    int32_t nc;
                    int a;
                    int cnt = walk_pixel(&s, ids, start, end, x + 0.5, y + 0.5, buf, cap, &T, &nc, C, &a, NULL);
                    size_t p = (size_t)y * W + x;
                    double gD = g_dist ? g_dist[p] : 0.0, gM = g_median ? g_median[p] : 0.0;
                    int m = median_entry(buf, cnt, NULL);
                    double zm = m >= 0 ? depths[ids[buf[m].k]] : 0.0;
                    double A, B, Cs, D;
                    depth_totals(buf, cnt, ids, depths, zm, &A, &B, &Cs, &D);
                    double S = 0.0;  /* sum over the composited entries behind: w_j dD/dw_j */
                    for (int e = cnt - 1; e >= 0; --e) {
                        const contrib_t* q = &buf[e];
                        int32_t i = ids[q->k];
                        double al = q->alpha, Ti = q->T, w = al * Ti, u = depths[i] - zm;
                        double dw = u * u * A - 2.0 * u * B + Cs;
                        double dal = gD * (Ti * dw - S / (1.0 - al));
                        double* o = part + 10 * (q->k - start);
                        o[9] += gD * 2.0 * w * (u * A - B) + (e == m ? gM : 0.0);
                        add_alpha_grad(o, q, s.conics + 3 * i, dal);
                        S += w * dw;
                    }
                }
            }
#pragma omp critical(gso_merge_depth)
            {
                for (int k = 0; k < L; ++k) {
                    const double* o = part + 10 * k;
                    int32_t i = ids[start + k];
                    for (int f = 0; f < 9; ++f) grads[9 * (size_t)i + f] += o[f];
                    ddepth[i] += o[9];
                }
            }
        }
        free(buf);
        free(part);
    }
    return threads_used();
}
