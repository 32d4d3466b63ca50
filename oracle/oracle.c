/*
 * Reference oracle for the 2-D convolution forward (Conv and ConvTranspose).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * call or execute this file; only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant generator with the HIP library: every formula below is written
 * out again from the pages' statement of the problem.
 *
 * Everything is computed in IEEE double with no blocking, fusion or
 * reordering beyond what the definition states.  Inputs arrive as double
 * arrays that hold the values the GPU sees (already rounded once to the
 * layer's element type by the caller).
 *
 * Sources (the pages):
 *  - "Convolutions" (ml-interview-book, part 4, ch. 2), section 1
 *    "Intuition first" (worked 4x4 * 3x3 example, im2col), section 2.1
 *    (boxed output-size equation), 2.3 (MACs and params), 2.4 (convolution
 *    as a matrix multiply; col2im is the adjoint scatter-add), 2.6
 *    (Winograd's minimal filtering: F(2x2, 3x3) with 16 multiplies), 2.5
 *    (transposed convolution), section 6 (output_padding), exercise 3
 *    (checkerboard counts).
 *  - "Convolution, pooling and resize" (OneGpu docs), section "Layout and
 *    operands" (NCHW / OIHW, ConvTranspose weight [Cin, Cout/groups, KH, KW],
 *    explicit pads, dilation, groups, fused epilogue order: sum, bias,
 *    residual, activation; the nine fused activations), section
 *    "ConvInteger" (asymmetric padding is part of the problem geometry) and
 *    section "ConvInteger" (the integer convolution with zero points, int32
 *    with wrap-around, padding as the zero point), and
 *    section "Pooling and resize" (MaxPool / AveragePool with padding,
 *    dilation, ceil_mode and count_include_pad; the NaN and empty-window
 *    rules; global pools over a plane).
 *
 * Readings where the pages are silent:
 *  - padding is zero padding (ONNX Conv semantics), begin and end pads are
 *    separate;
 *  - auto_pad follows the ONNX operator definitions (parity unpinned beyond
 *    the invariants the tests check);
 *  - activation formulas follow the ONNX operator definitions;
 *  - groups are contiguous channel blocks for both Conv and ConvTranspose.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Activation codes (the order the OneGpu page lists the fused activations). */
enum {
    OR_ACT_IDENTITY = 0,
    OR_ACT_RELU = 1,
    OR_ACT_TANH = 2,
    OR_ACT_SIGMOID = 3,
    OR_ACT_SILU = 4,
    OR_ACT_HARD_SIGMOID = 5,
    OR_ACT_HARD_SWISH = 6,
    OR_ACT_CLIP = 7,
    OR_ACT_LEAKY_RELU = 8
};

/* Geometry of one problem, explicit pads (t, l, b, r). */
typedef struct {
    int64_t n, c_in, h, w, c_out, kh, kw, groups;
    int64_t sh, sw, dh, dw;
    int64_t pt, pl, pb, pr;
    int64_t oph, opw;  /* ConvTranspose output_padding */
    int32_t act;
    int32_t pad_;
    double alpha, beta; /* activation parameters */
} oracle_geom;

/* ---------------------------------------------------------------------- */
/* Output sizes                                                           */
/* ---------------------------------------------------------------------- */

/* Boxed output-size equation of section 2.1, with the begin and end pads
 * written separately:  out = floor((in + pb + pe - d(k-1) - 1) / s) + 1.
 * Returns 0 and writes *out, or -1 when no window fits. */
int oracle_conv_extent(int64_t in, int64_t k, int64_t s, int64_t d,
                       int64_t pb, int64_t pe, int64_t* out)
{
    if (in < 1 || k < 1 || s < 1 || d < 1 || pb < 0 || pe < 0) return -1;
    int64_t span = in + pb + pe - d * (k - 1) - 1;
    if (span < 0) return -1;
    *out = span / s + 1; /* span >= 0, so C division is the floor */
    return 0;
}

/* Transposed size (section 2.1's inversion plus output_padding, with
 * dilation):  out = s(in - 1) + op + d(k - 1) + 1 - pb - pe. */
int oracle_convt_extent(int64_t in, int64_t k, int64_t s, int64_t d,
                        int64_t pb, int64_t pe, int64_t op, int64_t* out)
{
    if (in < 1 || k < 1 || s < 1 || d < 1 || pb < 0 || pe < 0) return -1;
    if (op < 0 || op >= s) return -1; /* op only picks among the s preimages */
    int64_t o = s * (in - 1) + op + d * (k - 1) + 1 - pb - pe;
    if (o < 1) return -1;
    *out = o;
    return 0;
}

/* auto_pad modes (ONNX names): 0 NOTSET, 1 SAME_UPPER, 2 SAME_LOWER, 3 VALID.
 * Conv: SAME_* targets out = ceil(in / s); the total pad is what that needs,
 * UPPER puts the odd unit at the end, LOWER at the begin.
 * ConvTranspose: the total pad is s(in-1)+op+d(k-1)+1-out for the requested
 * out (default s*in under SAME_*); UPPER puts the odd unit at the end.
 * NOTSET leaves *pb and *pe as given.  Returns 0 or -1. */
int oracle_auto_pad(int transpose, int mode, int64_t in, int64_t k, int64_t s,
                    int64_t d, int64_t op, int64_t out_req,
                    int64_t* pb, int64_t* pe)
{
    if (in < 1 || k < 1 || s < 1 || d < 1) return -1;
    int64_t keff = d * (k - 1) + 1;
    if (!transpose) {
        if (mode == 0) return 0;
        if (mode == 3) { *pb = 0; *pe = 0; return 0; }
        if (mode != 1 && mode != 2) return -1;
        int64_t out = (in + s - 1) / s;
        int64_t total = (out - 1) * s + keff - in;
        if (total < 0) total = 0;
        int64_t small = total / 2, big = total - total / 2;
        if (mode == 1) { *pb = small; *pe = big; }
        else { *pb = big; *pe = small; }
        return 0;
    }
    if (mode == 3) { *pb = 0; *pe = 0; return 0; }
    if (mode == 0 && out_req < 0) return 0;
    int64_t out = out_req;
    if (out < 0) out = s * in; /* SAME_* without an explicit output shape */
    int64_t total = s * (in - 1) + op + keff - out;
    if (total < 0) return -1;
    int64_t small = total / 2, big = total - total / 2;
    if (mode == 1) { *pb = small; *pe = big; }
    else { *pb = big; *pe = small; }
    return 0;
}

/* MACs of a convolution, section 2.3: Ho*Wo*Co*(Ci/g)*k^2 per image. */
int64_t oracle_conv_macs(const oracle_geom* g, int64_t ho, int64_t wo)
{
    return g->n * ho * wo * g->c_out * (g->c_in / g->groups) * g->kh * g->kw;
}

/* ---------------------------------------------------------------------- */
/* Activations (ONNX operator definitions), in double                     */
/* ---------------------------------------------------------------------- */
double oracle_activation(int act, double v, double alpha, double beta)
{
    switch (act) {
    case OR_ACT_IDENTITY: return v;
    case OR_ACT_RELU: return v > 0.0 ? v : 0.0;
    case OR_ACT_TANH: return tanh(v);
    case OR_ACT_SIGMOID: return 1.0 / (1.0 + exp(-v));
    case OR_ACT_SILU: return v / (1.0 + exp(-v));
    case OR_ACT_HARD_SIGMOID: {
        double t = alpha * v + beta;
        return t < 0.0 ? 0.0 : (t > 1.0 ? 1.0 : t);
    }
    case OR_ACT_HARD_SWISH: {
        double t = v / 6.0 + 0.5;
        t = t < 0.0 ? 0.0 : (t > 1.0 ? 1.0 : t);
        return v * t;
    }
    case OR_ACT_CLIP: return v < alpha ? alpha : (v > beta ? beta : v);
    case OR_ACT_LEAKY_RELU: return v >= 0.0 ? v : alpha * v;
    default: return NAN;
    }
}

static int geom_ok(const oracle_geom* g)
{
    if (g->n < 1 || g->c_in < 1 || g->h < 1 || g->w < 1 || g->c_out < 1) return 0;
    if (g->kh < 1 || g->kw < 1 || g->groups < 1) return 0;
    if (g->c_in % g->groups || g->c_out % g->groups) return 0;
    return 1;
}

static void set_threads(int threads)
{
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
}

/* ---------------------------------------------------------------------- */
/* Conv, direct definition                                                 */
/* ---------------------------------------------------------------------- */

/* y[n,co,oh,ow] = act( sum_{ci',kh,kw} x[n, g*Cg+ci', ih, iw] * w[co,ci',kh,kw]
 *                      + b[co] + r[n,co,oh,ow] ),
 * ih = oh*sh - pt + kh*dh, iw = ow*sw - pl + kw*dw, taps outside the input
 * are zero (skipped).  Cross-correlation: no kernel flip.  s[...] receives
 * sum |x*w| over the same taps.  b, r, s may be NULL. */
int oracle_conv2d(const oracle_geom* g, const double* x, const double* w,
                  const double* b, const double* r, double* y, double* s,
                  int threads)
{
    int64_t ho, wo;
    if (!geom_ok(g)) return -1;
    if (oracle_conv_extent(g->h, g->kh, g->sh, g->dh, g->pt, g->pb, &ho)) return -1;
    if (oracle_conv_extent(g->w, g->kw, g->sw, g->dw, g->pl, g->pr, &wo)) return -1;
    const int64_t cig = g->c_in / g->groups, cog = g->c_out / g->groups;
    set_threads(threads);
    int64_t planes = g->n * g->c_out;
#pragma omp parallel for schedule(dynamic)
    for (int64_t pc = 0; pc < planes; ++pc) {
        int64_t n = pc / g->c_out, co = pc % g->c_out;
        int64_t grp = co / cog;
        for (int64_t oh = 0; oh < ho; ++oh) {
            for (int64_t ow = 0; ow < wo; ++ow) {
                double acc = 0.0, sc = 0.0;
                for (int64_t ci = 0; ci < cig; ++ci) {
                    const double* xp = x + ((n * g->c_in + grp * cig + ci) * g->h) * g->w;
                    const double* wp = w + ((co * cig + ci) * g->kh) * g->kw;
                    for (int64_t kh = 0; kh < g->kh; ++kh) {
                        int64_t ih = oh * g->sh - g->pt + kh * g->dh;
                        if (ih < 0 || ih >= g->h) continue;
                        for (int64_t kw = 0; kw < g->kw; ++kw) {
                            int64_t iw = ow * g->sw - g->pl + kw * g->dw;
                            if (iw < 0 || iw >= g->w) continue;
                            double t = xp[ih * g->w + iw] * wp[kh * g->kw + kw];
                            acc += t;
                            sc += fabs(t);
                        }
                    }
                }
                int64_t oi = ((n * g->c_out + co) * ho + oh) * wo + ow;
                double v = acc;
                if (b) v += b[co];
                if (r) v += r[oi];
                y[oi] = oracle_activation(g->act, v, g->alpha, g->beta);
                if (s) s[oi] = sc;
            }
        }
    }
    return 0;
}

/* The same definition evaluated only at the given flat NCHW output indices
 * (for sampled checks of large layers). */
int oracle_conv2d_points(const oracle_geom* g, const double* x, const double* w,
                         const double* b, const double* r, const int64_t* idx,
                         int64_t count, double* y, double* s, int threads)
{
    int64_t ho, wo;
    if (!geom_ok(g)) return -1;
    if (oracle_conv_extent(g->h, g->kh, g->sh, g->dh, g->pt, g->pb, &ho)) return -1;
    if (oracle_conv_extent(g->w, g->kw, g->sw, g->dw, g->pl, g->pr, &wo)) return -1;
    const int64_t cig = g->c_in / g->groups, cog = g->c_out / g->groups;
    const int64_t total = g->n * g->c_out * ho * wo;
    set_threads(threads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int64_t q = 0; q < count; ++q) {
        int64_t oi = idx[q];
        if (oi < 0 || oi >= total) { bad |= 1; continue; }
        int64_t ow = oi % wo, t1 = oi / wo;
        int64_t oh = t1 % ho, t2 = t1 / ho;
        int64_t co = t2 % g->c_out, n = t2 / g->c_out;
        int64_t grp = co / cog;
        double acc = 0.0, sc = 0.0;
        for (int64_t ci = 0; ci < cig; ++ci) {
            for (int64_t kh = 0; kh < g->kh; ++kh) {
                int64_t ih = oh * g->sh - g->pt + kh * g->dh;
                if (ih < 0 || ih >= g->h) continue;
                for (int64_t kw = 0; kw < g->kw; ++kw) {
                    int64_t iw = ow * g->sw - g->pl + kw * g->dw;
                    if (iw < 0 || iw >= g->w) continue;
                    double t = x[((n * g->c_in + grp * cig + ci) * g->h + ih) * g->w + iw]
                             * w[((co * cig + ci) * g->kh + kh) * g->kw + kw];
                    acc += t;
                    sc += fabs(t);
                }
            }
        }
        double v = acc;
        if (b) v += b[co];
        if (r) v += r[oi];
        y[q] = oracle_activation(g->act, v, g->alpha, g->beta);
        if (s) s[q] = sc;
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------- */
/* Conv as unfold + matrix product (section 2.4 / section 1 im2col)        */
/* ---------------------------------------------------------------------- */

/* For each image and group: cols[(ci',kh,kw), (oh,ow)] holds the input
 * value under that tap (zero in padding), then Y_g = W_g * cols with W_g the
 * group's weights flattened to (Cout/g) x (Cin/g*KH*KW), then bias,
 * residual, activation.  A second formulation used to cross-check the
 * direct loops. */
int oracle_conv2d_im2col(const oracle_geom* g, const double* x, const double* w,
                         const double* b, const double* r, double* y, int threads)
{
    int64_t ho, wo;
    if (!geom_ok(g)) return -1;
    if (oracle_conv_extent(g->h, g->kh, g->sh, g->dh, g->pt, g->pb, &ho)) return -1;
    if (oracle_conv_extent(g->w, g->kw, g->sw, g->dw, g->pl, g->pr, &wo)) return -1;
    const int64_t cig = g->c_in / g->groups, cog = g->c_out / g->groups;
    const int64_t kk = cig * g->kh * g->kw, p = ho * wo;
    set_threads(threads);
    int64_t jobs = g->n * g->groups;
    int fail = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : fail)
    for (int64_t job = 0; job < jobs; ++job) {
        int64_t n = job / g->groups, grp = job % g->groups;
        double* cols = (double*)malloc(sizeof(double) * (size_t)(kk * p));
        if (!cols) { fail |= 1; continue; }
        /* unfold: row (ci',kh,kw) in the order of w's flattening */
        for (int64_t ci = 0; ci < cig; ++ci)
            for (int64_t kh = 0; kh < g->kh; ++kh)
                for (int64_t kw = 0; kw < g->kw; ++kw) {
                    int64_t row = (ci * g->kh + kh) * g->kw + kw;
                    for (int64_t oh = 0; oh < ho; ++oh)
                        for (int64_t ow = 0; ow < wo; ++ow) {
                            int64_t ih = oh * g->sh - g->pt + kh * g->dh;
                            int64_t iw = ow * g->sw - g->pl + kw * g->dw;
                            double v = 0.0;
                            if (ih >= 0 && ih < g->h && iw >= 0 && iw < g->w)
                                v = x[((n * g->c_in + grp * cig + ci) * g->h + ih) * g->w + iw];
                            cols[row * p + oh * wo + ow] = v;
                        }
                }
        /* matrix product, then bias / residual / activation */
        for (int64_t j = 0; j < cog; ++j) {
            int64_t co = grp * cog + j;
            const double* wr = w + co * kk;
            for (int64_t q = 0; q < p; ++q) {
                double acc = 0.0;
                for (int64_t k = 0; k < kk; ++k) acc += wr[k] * cols[k * p + q];
                int64_t oi = (n * g->c_out + co) * p + q;
                double v = acc;
                if (b) v += b[co];
                if (r) v += r[oi];
                y[oi] = oracle_activation(g->act, v, g->alpha, g->beta);
            }
        }
        free(cols);
    }
    return fail ? -1 : 0;
}

/* ---------------------------------------------------------------------- */
/* ConvTranspose                                                           */
/* ---------------------------------------------------------------------- */

/* Scatter definition (section 2.5: each input value places a scaled copy of
 * the kernel at stride s and overlaps add).  Weight layout [Cin, Cout/g, KH,
 * KW]; input channel ci is in group ci / (Cin/g) and writes output channel
 * g*(Cout/g) + j.  oh = ih*sh - pt + kh*dh, ow = iw*sw - pl + kw*dw; contributions
 * that land outside [0,Ho) x [0,Wo) are dropped.  Then bias, residual,
 * activation. */
int oracle_conv_transpose2d(const oracle_geom* g, const double* x, const double* w,
                            const double* b, const double* r, double* y, double* s,
                            int threads)
{
    int64_t ho, wo;
    if (!geom_ok(g)) return -1;
    if (oracle_convt_extent(g->h, g->kh, g->sh, g->dh, g->pt, g->pb, g->oph, &ho)) return -1;
    if (oracle_convt_extent(g->w, g->kw, g->sw, g->dw, g->pl, g->pr, g->opw, &wo)) return -1;
    const int64_t cig = g->c_in / g->groups, cog = g->c_out / g->groups;
    const int64_t osz = g->c_out * ho * wo;
    set_threads(threads);
#pragma omp parallel for schedule(dynamic)
    for (int64_t n = 0; n < g->n; ++n) {
        double* acc = y + n * osz;
        double* sc = s ? s + n * osz : NULL;
        for (int64_t i = 0; i < osz; ++i) { acc[i] = 0.0; if (sc) sc[i] = 0.0; }
        for (int64_t ci = 0; ci < g->c_in; ++ci) {
            int64_t grp = ci / cig;
            for (int64_t ih = 0; ih < g->h; ++ih)
                for (int64_t iw = 0; iw < g->w; ++iw) {
                    double xv = x[((n * g->c_in + ci) * g->h + ih) * g->w + iw];
                    for (int64_t j = 0; j < cog; ++j) {
                        int64_t co = grp * cog + j;
                        for (int64_t kh = 0; kh < g->kh; ++kh) {
                            int64_t oh = ih * g->sh - g->pt + kh * g->dh;
                            if (oh < 0 || oh >= ho) continue;
                            for (int64_t kw = 0; kw < g->kw; ++kw) {
                                int64_t ow = iw * g->sw - g->pl + kw * g->dw;
                                if (ow < 0 || ow >= wo) continue;
                                double t = xv * w[((ci * cog + j) * g->kh + kh) * g->kw + kw];
                                int64_t oi = (co * ho + oh) * wo + ow;
                                acc[oi] += t;
                                if (sc) sc[oi] += fabs(t);
                            }
                        }
                    }
                }
        }
        for (int64_t co = 0; co < g->c_out; ++co)
            for (int64_t q = 0; q < ho * wo; ++q) {
                int64_t oi = co * ho * wo + q;
                double v = acc[oi];
                if (b) v += b[co];
                if (r) v += r[n * osz + oi];
                acc[oi] = oracle_activation(g->act, v, g->alpha, g->beta);
            }
    }
    return 0;
}

/* Gather form of the same operator: for each output, visit the taps whose
 * source position (oh + pt - kh*dh)/sh, (ow + pl - kw*dw)/sw is integral and
 * inside the input.  An independent cross-check of the scatter form. */
int oracle_conv_transpose2d_gather(const oracle_geom* g, const double* x,
                                   const double* w, const double* b, const double* r,
                                   double* y, int threads)
{
    int64_t ho, wo;
    if (!geom_ok(g)) return -1;
    if (oracle_convt_extent(g->h, g->kh, g->sh, g->dh, g->pt, g->pb, g->oph, &ho)) return -1;
    if (oracle_convt_extent(g->w, g->kw, g->sw, g->dw, g->pl, g->pr, g->opw, &wo)) return -1;
    const int64_t cig = g->c_in / g->groups, cog = g->c_out / g->groups;
    set_threads(threads);
    int64_t planes = g->n * g->c_out;
#pragma omp parallel for schedule(dynamic)
    for (int64_t pc = 0; pc < planes; ++pc) {
        int64_t n = pc / g->c_out, co = pc % g->c_out;
        int64_t grp = co / cog, j = co % cog;
        for (int64_t oh = 0; oh < ho; ++oh)
            for (int64_t ow = 0; ow < wo; ++ow) {
                double acc = 0.0;
                for (int64_t c = 0; c < cig; ++c) {
                    int64_t ci = grp * cig + c;
                    for (int64_t kh = 0; kh < g->kh; ++kh) {
                        int64_t th = oh + g->pt - kh * g->dh;
                        if (th < 0 || th % g->sh) continue;
                        int64_t ih = th / g->sh;
                        if (ih >= g->h) continue;
                        for (int64_t kw = 0; kw < g->kw; ++kw) {
                            int64_t tw = ow + g->pl - kw * g->dw;
                            if (tw < 0 || tw % g->sw) continue;
                            int64_t iw = tw / g->sw;
                            if (iw >= g->w) continue;
                            acc += x[((n * g->c_in + ci) * g->h + ih) * g->w + iw]
                                 * w[((ci * cog + j) * g->kh + kh) * g->kw + kw];
                        }
                    }
                }
                int64_t oi = ((n * g->c_out + co) * ho + oh) * wo + ow;
                double v = acc;
                if (b) v += b[co];
                if (r) v += r[oi];
                y[oi] = oracle_activation(g->act, v, g->alpha, g->beta);
            }
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would use. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* Pooling ("Convolution, pooling and resize", section "Pooling and        */
/* resize"; ONNX MaxPool / AveragePool / GlobalMaxPool /                   */
/* GlobalAveragePool)                                                      */
/* ---------------------------------------------------------------------- */

typedef struct {
    int64_t n, c, h, w, kh, kw, sh, sw, dh, dw, pt, pl, pb, pr;
    int32_t kind;              /* 0 max, 1 average */
    int32_t ceil_mode;         /* 1: the output size rounds up */
    int32_t count_include_pad; /* average: padding taps count in the divisor */
    int32_t pad_;
} oracle_pool_geom;

/* Output size along one axis.  Floor mode is the convolution's equation.
 * Ceil mode rounds the division up, and then drops a last window that starts
 * inside the end padding (its first tap at or beyond the input's end).
 * Returns 0 and writes *out, or -1 when no window fits. */
int oracle_pool_extent(int64_t in, int64_t k, int64_t s, int64_t d, int64_t pb,
                       int64_t pe, int ceil_mode, int64_t* out)
{
    if (in < 1 || k < 1 || s < 1 || d < 1 || pb < 0 || pe < 0) return -1;
    int64_t span = in + pb + pe - d * (k - 1) - 1;
    if (span < 0) return -1;
    int64_t o = ceil_mode ? (span + s - 1) / s + 1 : span / s + 1;
    if (ceil_mode && (o - 1) * s - pb >= in) o -= 1;
    if (o < 1) return -1;
    *out = o;
    return 0;
}

/* Windowed pooling over each (n, c) plane.  The window of output (oh, ow)
 * holds the taps ih = oh*sh - pt + kh*dh, iw = ow*sw - pl + kw*dw.  A tap is
 * real when it lies inside the input, padding when it lies inside the pads,
 * and beyond the padding otherwise (only in ceil mode).
 *  - max: the largest real tap.  NaN taps are skipped unless every real tap is
 *    NaN (then NaN); +0 counts as larger than -0; a window with no real tap
 *    gives `lowest` (the lowest finite value of the element type).
 *  - average: the sum of the real taps over the divisor, which counts the
 *    real taps, plus the padding taps when count_include_pad is set (taps
 *    beyond the padding never count); 0/0 is NaN.  scale (may be NULL)
 *    receives sum |x| over the same divisor, the magnitude the tolerance
 *    scales with.
 * y is [n, c, ho, wo]. */
int oracle_pool2d(const oracle_pool_geom* g, const double* x, double lowest, double* y,
                  double* scale)
{
    int64_t ho, wo;
    if (g->n < 1 || g->c < 1) return -1;
    if (oracle_pool_extent(g->h, g->kh, g->sh, g->dh, g->pt, g->pb, g->ceil_mode, &ho) ||
        oracle_pool_extent(g->w, g->kw, g->sw, g->dw, g->pl, g->pr, g->ceil_mode, &wo))
        return -1;
    if (g->kind != 0 && g->kind != 1) return -1;
    for (int64_t p = 0; p < g->n * g->c; ++p) {
        const double* xp = x + p * g->h * g->w;
        for (int64_t oh = 0; oh < ho; ++oh)
            for (int64_t ow = 0; ow < wo; ++ow) {
                double best = 0.0, sum = 0.0, mag = 0.0;
                int64_t real = 0, counted = 0, finite_seen = 0, nan_seen = 0;
                for (int64_t kh = 0; kh < g->kh; ++kh)
                    for (int64_t kw = 0; kw < g->kw; ++kw) {
                        int64_t ih = oh * g->sh - g->pt + kh * g->dh;
                        int64_t iw = ow * g->sw - g->pl + kw * g->dw;
                        int in_h = ih >= 0 && ih < g->h, in_w = iw >= 0 && iw < g->w;
                        int pad_h = ih >= -g->pt && ih < g->h + g->pb;
                        int pad_w = iw >= -g->pl && iw < g->w + g->pr;
                        if (in_h && in_w) {
                            double v = xp[ih * g->w + iw];
                            ++real;
                            ++counted;
                            sum += v;
                            mag += fabs(v);
                            if (isnan(v)) {
                                nan_seen = 1;
                            } else if (!finite_seen || v > best ||
                                       (v == best && signbit(best) && !signbit(v))) {
                                best = v;
                                finite_seen = 1;
                            }
                        } else if (pad_h && pad_w) {
                            ++counted; /* a padding tap */
                        }
                    }
                int64_t oi = (p * ho + oh) * wo + ow;
                if (g->kind == 0) {
                    y[oi] = finite_seen ? best : (nan_seen ? NAN : lowest);
                    if (scale) scale[oi] = 0.0;
                } else {
                    int64_t div = g->count_include_pad ? counted : real;
                    y[oi] = sum / (double)div;
                    if (scale) scale[oi] = mag / (double)div;
                }
            }
    }
    return 0;
}

/* Global pooling: one value per (n, c) plane of hw elements.  kind 0: the
 * largest element under the same rules as oracle_pool2d's max (the plane is
 * never empty); kind 1: the mean.  scale receives the mean of |x|. */
int oracle_global_pool(int kind, int64_t planes, int64_t hw, const double* x, double* y,
                       double* scale)
{
    if (planes < 1 || hw < 1 || (kind != 0 && kind != 1)) return -1;
    for (int64_t p = 0; p < planes; ++p) {
        const double* xp = x + p * hw;
        double best = 0.0, sum = 0.0, mag = 0.0;
        int finite_seen = 0, nan_seen = 0;
        for (int64_t i = 0; i < hw; ++i) {
            double v = xp[i];
            sum += v;
            mag += fabs(v);
            if (isnan(v)) nan_seen = 1;
            else if (!finite_seen || v > best || (v == best && signbit(best) && !signbit(v))) {
                best = v;
                finite_seen = 1;
            }
        }
        y[p] = kind == 0 ? (finite_seen ? best : (nan_seen ? NAN : 0.0)) : sum / (double)hw;
        if (scale) scale[p] = kind == 0 ? 0.0 : mag / (double)hw;
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* ConvInteger ("Convolution, pooling and resize", section "ConvInteger";  */
/* ONNX ConvInteger)                                                        */
/* ---------------------------------------------------------------------- */

/* y[n,co,oh,ow] = sum over the real taps of (x - x_zero) * (w[co,...] - w_zero[co]),
 * exactly in 64-bit integers, then reduced to int32 with wrap-around (the value
 * modulo 2^32 in two's complement).  x and w hold the integer values of their
 * uint8 or int8 elements; w_zero has c_out entries (a per-tensor zero point is
 * passed repeated).  A padded tap is the real value zero, i.e. the quantized
 * value x_zero, so it adds nothing: it is skipped.  Geometry as oracle_conv2d
 * (the activation, bias and residual fields are not used). */
int oracle_conv_integer(const oracle_geom* g, const int32_t* x, const int32_t* w,
                        int32_t x_zero, const int32_t* w_zero, int32_t* y, int threads)
{
    int64_t ho, wo;
    if (!geom_ok(g)) return -1;
    if (oracle_conv_extent(g->h, g->kh, g->sh, g->dh, g->pt, g->pb, &ho) ||
        oracle_conv_extent(g->w, g->kw, g->sw, g->dw, g->pl, g->pr, &wo))
        return -1;
    const int64_t cig = g->c_in / g->groups, cog = g->c_out / g->groups;
    set_threads(threads);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < g->n; ++n)
        for (int64_t co = 0; co < g->c_out; ++co) {
            const int64_t grp = co / cog;
            for (int64_t oh = 0; oh < ho; ++oh)
                for (int64_t ow = 0; ow < wo; ++ow) {
                    int64_t acc = 0;
                    for (int64_t ci = 0; ci < cig; ++ci)
                        for (int64_t kh = 0; kh < g->kh; ++kh)
                            for (int64_t kw = 0; kw < g->kw; ++kw) {
                                int64_t ih = oh * g->sh - g->pt + kh * g->dh;
                                int64_t iw = ow * g->sw - g->pl + kw * g->dw;
                                if (ih < 0 || ih >= g->h || iw < 0 || iw >= g->w) continue;
                                int64_t xv = x[((n * g->c_in + grp * cig + ci) * g->h + ih) * g->w + iw];
                                int64_t wv = w[((co * cig + ci) * g->kh + kh) * g->kw + kw];
                                acc += (xv - x_zero) * (wv - w_zero[co]);
                            }
                    uint32_t low = (uint32_t)(uint64_t)acc;
                    y[((n * g->c_out + co) * ho + oh) * wo + ow] =
                        (int32_t)(low >= 0x80000000u ? (int64_t)low - 0x100000000LL : (int64_t)low);
                }
        }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Winograd F(2x2, 3x3) ("Convolutions", section 2.6: F(m, r) computes m   */
/* outputs of an r-tap filter with m + r - 1 multiplies, 16 against 36 in  */
/* 2-D, at the cost of transforms of the input tiles and the weights;      */
/* "Convolution, pooling and resize", "Not built, with the numbers":       */
/* sixteen batched products between the transforms)                       */
/* ---------------------------------------------------------------------- */

/* The minimal filtering algorithm of Lavin and Gray (2016) for a 3x3
 * cross-correlation with stride 1 and dilation 1, in double:
 *   U = G g G^T    (4x4, per output channel and input channel)
 *   V = B^T d B    (4x4, per input channel and 4x4 input tile d, the tiles
 *                   taken every 2 outputs; taps outside the input are 0)
 *   M = sum over input channels of U (.) V  (the sixteen products)
 *   Y = A^T M A    (the 2x2 outputs of the tile)
 * with B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1],
 *      G   = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2 1/2; 0 0 1],
 *      A^T = [1 1 1 0; 0 1 -1 -1],
 * then bias, residual and activation as oracle_conv2d.  Groups are contiguous
 * channel blocks.  Outputs of a tile beyond Ho or Wo are dropped.  Returns -1
 * unless the kernel is 3x3 with stride 1 and dilation 1. */
int oracle_conv2d_winograd(const oracle_geom* g, const double* x, const double* w,
                           const double* b, const double* r, double* y, int threads)
{
    static const double BT[4][4] = {{1, 0, -1, 0}, {0, 1, 1, 0}, {0, -1, 1, 0}, {0, 1, 0, -1}};
    static const double GM[4][3] = {{1, 0, 0}, {0.5, 0.5, 0.5}, {0.5, -0.5, 0.5}, {0, 0, 1}};
    static const double AT[2][4] = {{1, 1, 1, 0}, {0, 1, -1, -1}};
    int64_t ho, wo;
    if (!geom_ok(g)) return -1;
    if (g->kh != 3 || g->kw != 3 || g->sh != 1 || g->sw != 1 || g->dh != 1 || g->dw != 1) return -1;
    if (oracle_conv_extent(g->h, 3, 1, 1, g->pt, g->pb, &ho) ||
        oracle_conv_extent(g->w, 3, 1, 1, g->pl, g->pr, &wo))
        return -1;
    const int64_t cig = g->c_in / g->groups, cog = g->c_out / g->groups;
    const int64_t th_n = (ho + 1) / 2, tw_n = (wo + 1) / 2;
    set_threads(threads);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < g->n; ++n)
        for (int64_t co = 0; co < g->c_out; ++co) {
            const int64_t grp = co / cog;
            for (int64_t th = 0; th < th_n; ++th)
                for (int64_t tw = 0; tw < tw_n; ++tw) {
                    double m[4][4] = {{0}};
                    for (int64_t ci = 0; ci < cig; ++ci) {
                        const double* gw = w + (co * cig + ci) * 9;
                        double gg[4][3], u[4][4], d[4][4], bd[4][4], v[4][4];
                        for (int i = 0; i < 4; ++i)      /* G g */
                            for (int j = 0; j < 3; ++j)
                                gg[i][j] = GM[i][0] * gw[j] + GM[i][1] * gw[3 + j] + GM[i][2] * gw[6 + j];
                        for (int i = 0; i < 4; ++i)      /* (G g) G^T */
                            for (int j = 0; j < 4; ++j)
                                u[i][j] = gg[i][0] * GM[j][0] + gg[i][1] * GM[j][1] + gg[i][2] * GM[j][2];
                        for (int i = 0; i < 4; ++i)      /* the input tile */
                            for (int j = 0; j < 4; ++j) {
                                int64_t ih = 2 * th - g->pt + i, iw = 2 * tw - g->pl + j;
                                d[i][j] = (ih >= 0 && ih < g->h && iw >= 0 && iw < g->w)
                                              ? x[((n * g->c_in + grp * cig + ci) * g->h + ih) * g->w + iw]
                                              : 0.0;
                            }
                        for (int i = 0; i < 4; ++i)      /* B^T d */
                            for (int j = 0; j < 4; ++j)
                                bd[i][j] = BT[i][0] * d[0][j] + BT[i][1] * d[1][j] + BT[i][2] * d[2][j] + BT[i][3] * d[3][j];
                        for (int i = 0; i < 4; ++i)      /* (B^T d) B */
                            for (int j = 0; j < 4; ++j)
                                v[i][j] = bd[i][0] * BT[j][0] + bd[i][1] * BT[j][1] + bd[i][2] * BT[j][2] + bd[i][3] * BT[j][3];
                        for (int i = 0; i < 4; ++i)
                            for (int j = 0; j < 4; ++j) m[i][j] += u[i][j] * v[i][j];
                    }
                    double am[2][4];
                    for (int i = 0; i < 2; ++i)          /* A^T M */
                        for (int j = 0; j < 4; ++j)
                            am[i][j] = AT[i][0] * m[0][j] + AT[i][1] * m[1][j] + AT[i][2] * m[2][j] + AT[i][3] * m[3][j];
                    for (int i = 0; i < 2; ++i)          /* (A^T M) A, then the epilogue */
                        for (int j = 0; j < 2; ++j) {
                            int64_t oh = 2 * th + i, ow = 2 * tw + j;
                            if (oh >= ho || ow >= wo) continue;
                            double acc = am[i][0] * AT[j][0] + am[i][1] * AT[j][1] + am[i][2] * AT[j][2] + am[i][3] * AT[j][3];
                            int64_t oi = ((n * g->c_out + co) * ho + oh) * wo + ow;
                            if (b) acc += b[co];
                            if (r) acc += r[oi];
                            y[oi] = oracle_activation(g->act, acc, g->alpha, g->beta);
                        }
                }
        }
    return 0;
}
