/*
 * convt_oracle.c -- CPU oracle for the transposed-convolution forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  The product path (the HIP
 * library) never calls, links or includes it, and it includes nothing of the
 * product path.
 *
 * What it computes: the direct scatter definition of a transposed convolution,
 * accumulated in fp64, with no blocking, no phase tables and no gather.
 *
 *   Every input element x[n, ci, i] (i a position per axis) is multiplied by
 *   every kernel tap w[ci, co_l, k] of its group and added to the output at
 *   o = i*s - p + k*d on each axis.  Contributions that land outside
 *   [0, L_out) are dropped.  The bias of the output channel is added once to
 *   every output element.  With groups G, input channel ci belongs to group
 *   g = ci / (C_in/G) and writes output channels g*(C_out/G) + co_l.
 *
 *   Source: "Kimi-K2.6 l1_p79" transcript (ConvTranspose1d, dilation 2), the
 *   scatter-then-crop derivation and its worked example with two inputs; the
 *   "Kimi-K2.6 l1_p72" transcript (ConvTranspose3d, groups 4), the
 *   per-group reference loop with bias and its remark that writes falling
 *   outside the output are ignored.
 *
 *   Output size per axis (closed form on all three pages):
 *     L_out = (L_in - 1)*s - 2p + d*(K - 1) + out_pad + 1
 *
 *   Fused epilogue ("Kimi-K2.6 l2_p26" transcript, ConvTranspose3d + add +
 *   HardSwish, its statement of the forward and of hardswish):
 *     t = conv_transpose(x) + bias + add_input
 *     y = t * hardswish(t),  hardswish(t) = t * min(max(t + 3, 0), 6) / 6
 *   The selectable epilogue takes the parts of that forward singly or
 *   together: the add of add_input or not, then y = t, hardswish(t) or
 *   t * hardswish(t) (act 0, 1, 2).
 *
 *   Layouts: channels first (layout 0: x (N, C_in, L_in...), y and add_input
 *   (N, C_out, L_out...)) or channels last (layout 1: x (N, L_in..., C_in),
 *   y and add_input (N, L_out..., C_out)); the weight is (C_in, C_out/G, K...)
 *   in both.  The layout changes where each element sits, nothing of the
 *   arithmetic.
 *
 * Readings taken where the pages leave a point open: output_padding only
 * lengthens the output at the high end and those positions receive whatever
 * the scatter lands there (plus bias); any out_pad >= 0 is accepted; dilation
 * applies per axis in 3D the same way as in 1D; the weight is used as stored,
 * never flipped.
 *
 * Inputs are float32 (the values the GPU sees); every product and sum is
 * formed in double; results are returned as double.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_MAX_AXES 3

/* One problem, every axis padded to 3 (missing leading axes are unit axes:
 * L_in=1, K=1, s=1, p=0, out_pad=0, d=1, which give L_out=1). */
typedef struct {
    int64_t N, C_in, C_out, G;
    int64_t L_in[ORACLE_MAX_AXES], K[ORACLE_MAX_AXES], s[ORACLE_MAX_AXES];
    int64_t p[ORACLE_MAX_AXES], op[ORACLE_MAX_AXES], d[ORACLE_MAX_AXES];
    int64_t L_out[ORACLE_MAX_AXES];
} problem;

/* The closed form for one axis. */
static int64_t closed_form(int64_t L_in, int64_t K, int64_t s, int64_t p, int64_t op, int64_t d)
{
    return (L_in - 1) * s - 2 * p + d * (K - 1) + op + 1;
}

int oracle_output_size(int ndim, const int64_t *in_size, const int64_t *K, const int64_t *s,
                       const int64_t *p, const int64_t *op, const int64_t *d, int64_t *out_size)
{
    if (ndim < 1 || ndim > ORACLE_MAX_AXES) return 1;
    for (int a = 0; a < ndim; ++a)
        out_size[a] = closed_form(in_size[a], K[a], s[a], p[a], op[a], d[a]);
    return 0;
}

static int set_problem(problem *P, int ndim, int64_t N, int64_t C_in, int64_t C_out, int64_t G,
                       const int64_t *in_size, const int64_t *K, const int64_t *s,
                       const int64_t *p, const int64_t *op, const int64_t *d)
{
    if (ndim < 1 || ndim > ORACLE_MAX_AXES || N < 0 || C_in < 1 || C_out < 1 || G < 1) return 1;
    if (C_in % G != 0 || C_out % G != 0) return 1;
    P->N = N; P->C_in = C_in; P->C_out = C_out; P->G = G;
    int lead = ORACLE_MAX_AXES - ndim;
    for (int a = 0; a < ORACLE_MAX_AXES; ++a) {
        if (a < lead) {
            P->L_in[a] = 1; P->K[a] = 1; P->s[a] = 1; P->p[a] = 0; P->op[a] = 0; P->d[a] = 1;
        } else {
            int b = a - lead;
            P->L_in[a] = in_size[b]; P->K[a] = K[b]; P->s[a] = s[b];
            P->p[a] = p[b]; P->op[a] = op[b]; P->d[a] = d[b];
        }
        if (P->L_in[a] < 1 || P->K[a] < 1 || P->s[a] < 1 || P->d[a] < 1 || P->p[a] < 0 ||
            P->op[a] < 0)
            return 1;
        P->L_out[a] = closed_form(P->L_in[a], P->K[a], P->s[a], P->p[a], P->op[a], P->d[a]);
        if (P->L_out[a] < 1) return 1;
    }
    return 0;
}

/* hardswish(t) = t * clamp(t + 3, 0, 6) / 6. */
static double hardswish(double t)
{
    double r = t + 3.0;
    if (r < 0.0) r = 0.0;
    if (r > 6.0) r = 6.0;
    return t * r / 6.0;
}

/* The fused forward's epilogue: t * hardswish(t). */
static double times_hardswish(double t)
{
    return t * hardswish(t);
}

/* Activation act: 0 none, 1 hardswish, 2 t * hardswish(t). */
static double activate(double t, int act)
{
    if (act == 1) return hardswish(t);
    if (act == 2) return times_hardswish(t);
    return t;
}

/* Flat index of element (n, c, e) (e the flat spatial position, sp of them
 * per channel, C channels) in layout 0 (channels first) or 1 (channels last). */
static int64_t at(int layout, int64_t n, int64_t c, int64_t e, int64_t C, int64_t sp)
{
    return layout ? (n * sp + e) * C + c : (n * C + c) * sp + e;
}

typedef struct {
    const problem *P;
    const float *x, *w, *bias, *add;
    int act, layout;
    double *y;
    int64_t next_slab, n_slabs;
    pthread_mutex_t lock;
} scatter_job;

/* One (n, g) slab: the scatter loop over every input element and every tap. */
static void scatter_slab(const scatter_job *J, int64_t n, int64_t g)
{
    const problem *P = J->P;
    const int64_t Cig = P->C_in / P->G, Cog = P->C_out / P->G;
    const int64_t ID = P->L_in[0], IH = P->L_in[1], IW = P->L_in[2];
    const int64_t OD = P->L_out[0], OH = P->L_out[1], OW = P->L_out[2];
    const int64_t KD = P->K[0], KH = P->K[1], KW = P->K[2];
    const int64_t in_sp = ID * IH * IW, out_sp = OD * OH * OW, k_sp = KD * KH * KW;

    /* slab[co_l][od][oh][ow], starting from the bias: in y itself for
     * channels first, else in a scratch slab written out at the end */
    double *own = NULL;
    if (J->layout) {
        own = (double *)malloc(sizeof(double) * (size_t)(Cog * out_sp));
        if (!own) abort();
    }
    double *slab = J->layout ? own : J->y + (n * P->C_out + g * Cog) * out_sp;
    for (int64_t co_l = 0; co_l < Cog; ++co_l) {
        double b = J->bias ? (double)J->bias[g * Cog + co_l] : 0.0;
        for (int64_t e = 0; e < out_sp; ++e) slab[co_l * out_sp + e] = b;
    }

    for (int64_t ci_l = 0; ci_l < Cig; ++ci_l) {
        const int64_t ci = g * Cig + ci_l;
        const float *xc = J->x + at(J->layout, n, ci, 0, P->C_in, in_sp);
        const int64_t xs = J->layout ? P->C_in : 1; /* step between positions */
        const float *wc = J->w + ci * Cog * k_sp;
        for (int64_t id = 0; id < ID; ++id)
        for (int64_t ih = 0; ih < IH; ++ih)
        for (int64_t iw = 0; iw < IW; ++iw) {
            const double xv = (double)xc[((id * IH + ih) * IW + iw) * xs];
            for (int64_t co_l = 0; co_l < Cog; ++co_l)
            for (int64_t kd = 0; kd < KD; ++kd) {
                const int64_t od = id * P->s[0] - P->p[0] + kd * P->d[0];
                if (od < 0 || od >= OD) continue;
                for (int64_t kh = 0; kh < KH; ++kh) {
                    const int64_t oh = ih * P->s[1] - P->p[1] + kh * P->d[1];
                    if (oh < 0 || oh >= OH) continue;
                    for (int64_t kw = 0; kw < KW; ++kw) {
                        const int64_t ow = iw * P->s[2] - P->p[2] + kw * P->d[2];
                        if (ow < 0 || ow >= OW) continue;
                        const double wv = (double)wc[co_l * k_sp + (kd * KH + kh) * KW + kw];
                        slab[co_l * out_sp + (od * OH + oh) * OW + ow] += xv * wv;
                    }
                }
            }
        }
    }

    /* epilogue: t = slab (+ add_input), then the activation, stored at the
     * element's place in the layout */
    for (int64_t co_l = 0; co_l < Cog; ++co_l)
        for (int64_t e = 0; e < out_sp; ++e) {
            const int64_t yi = at(J->layout, n, g * Cog + co_l, e, P->C_out, out_sp);
            double t = slab[co_l * out_sp + e];
            if (J->add) t += (double)J->add[yi];
            J->y[yi] = activate(t, J->act);
        }
    free(own);
}

static void *scatter_worker(void *arg)
{
    scatter_job *J = (scatter_job *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t t = J->next_slab++;
        pthread_mutex_unlock(&J->lock);
        if (t >= J->n_slabs) break;
        scatter_slab(J, t / J->P->G, t % J->P->G);
    }
    return NULL;
}

static int resolve_threads(int nthreads)
{
    if (nthreads > 0) return nthreads;
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c > 0 ? (int)c : 1;
}

/* Full forward with the selectable epilogue and layout.  y has
 * N*C_out*prod(L_out) doubles.  bias and add may be NULL.  act is 0, 1 or 2,
 * layout 0 or 1.  Returns 0, or 1 on bad arguments. */
int oracle_convt_forward_ex(int ndim, int64_t N, int64_t C_in, int64_t C_out, int64_t G,
                            const int64_t *in_size, const int64_t *K, const int64_t *s,
                            const int64_t *p, const int64_t *op, const int64_t *d,
                            const float *x, const float *w, const float *bias, const float *add,
                            int act, int layout, double *y, int nthreads)
{
    problem P;
    if (set_problem(&P, ndim, N, C_in, C_out, G, in_size, K, s, p, op, d)) return 1;
    if (act < 0 || act > 2 || layout < 0 || layout > 1) return 1;
    scatter_job J;
    J.P = &P; J.x = x; J.w = w; J.bias = bias; J.add = add; J.y = y;
    J.act = act; J.layout = layout;
    J.next_slab = 0; J.n_slabs = N * G;
    pthread_mutex_init(&J.lock, NULL);
    int nt = resolve_threads(nthreads);
    if (nt > J.n_slabs) nt = (int)(J.n_slabs > 0 ? J.n_slabs : 1);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) return 1;
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, scatter_worker, &J);
    for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

/* Full forward, channels first: the plain forward, or with add != NULL the
 * fused one (t * hardswish(t) of conv + bias + add). */
int oracle_convt_forward(int ndim, int64_t N, int64_t C_in, int64_t C_out, int64_t G,
                         const int64_t *in_size, const int64_t *K, const int64_t *s,
                         const int64_t *p, const int64_t *op, const int64_t *d,
                         const float *x, const float *w, const float *bias, const float *add,
                         double *y, int nthreads)
{
    return oracle_convt_forward_ex(ndim, N, C_in, C_out, G, in_size, K, s, p, op, d, x, w, bias, add,
                                   add ? 2 : 0, 0, y, nthreads);
}

/* The (i, k) pairs of one axis whose scatter lands on output position o:
 * every i in [0, L_in) and k in [0, K) is tried.  Returns the count. */
static int64_t pairs_hitting(int64_t o, int64_t L_in, int64_t K, int64_t s, int64_t p, int64_t d,
                             int64_t *pi, int64_t *pk)
{
    int64_t n = 0;
    for (int64_t i = 0; i < L_in; ++i)
        for (int64_t k = 0; k < K; ++k)
            if (i * s - p + k * d == o) { pi[n] = i; pk[n] = k; ++n; }
    return n;
}

/* Per-position pair counts for one axis, by scattering every (i, k):
 * counts[o] = #{(i, k) : i*s - p + k*d == o}, o in [0, L_out). */
int oracle_axis_pair_counts(int64_t L_in, int64_t K, int64_t s, int64_t p, int64_t op, int64_t d,
                            int64_t *counts)
{
    if (L_in < 1 || K < 1 || s < 1 || d < 1 || p < 0 || op < 0) return 1;
    int64_t L_out = closed_form(L_in, K, s, p, op, d);
    if (L_out < 1) return 1;
    memset(counts, 0, sizeof(int64_t) * (size_t)L_out);
    for (int64_t i = 0; i < L_in; ++i)
        for (int64_t k = 0; k < K; ++k) {
            int64_t o = i * s - p + k * d;
            if (o >= 0 && o < L_out) counts[o] += 1;
        }
    return 0;
}

/* Selected outputs, one by one: idx holds flat indices into y (N, C_out,
 * L_out...) in the given layout.  Each value is the sum of the scatter
 * contributions that land on that element (per axis, every (i, k) pair is
 * tried), plus bias, plus add_input if add != NULL, then the activation act.
 * Returns 0, or 1 on bad arguments. */
int oracle_convt_points_ex(int ndim, int64_t N, int64_t C_in, int64_t C_out, int64_t G,
                           const int64_t *in_size, const int64_t *K, const int64_t *s,
                           const int64_t *p, const int64_t *op, const int64_t *d,
                           const float *x, const float *w, const float *bias, const float *add,
                           int act, int layout, const int64_t *idx, int64_t npts, double *out)
{
    problem P;
    if (set_problem(&P, ndim, N, C_in, C_out, G, in_size, K, s, p, op, d)) return 1;
    if (act < 0 || act > 2 || layout < 0 || layout > 1) return 1;
    const int64_t Cig = C_in / G, Cog = C_out / G;
    const int64_t in_sp = P.L_in[0] * P.L_in[1] * P.L_in[2];
    const int64_t out_sp = P.L_out[0] * P.L_out[1] * P.L_out[2];
    const int64_t k_sp = P.K[0] * P.K[1] * P.K[2];
    int64_t cap[ORACLE_MAX_AXES];
    int64_t *pi[ORACLE_MAX_AXES], *pk[ORACLE_MAX_AXES];
    for (int a = 0; a < ORACLE_MAX_AXES; ++a) {
        cap[a] = P.L_in[a] * P.K[a];
        pi[a] = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap[a]);
        pk[a] = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap[a]);
    }
    int rc = 0;
    for (int64_t t = 0; t < npts; ++t) {
        int64_t e = idx[t];
        if (e < 0 || e >= N * C_out * out_sp) { rc = 1; break; }
        int64_t o[ORACLE_MAX_AXES], co;
        if (layout) { co = e % C_out; e /= C_out; }
        o[2] = e % P.L_out[2]; e /= P.L_out[2];
        o[1] = e % P.L_out[1]; e /= P.L_out[1];
        o[0] = e % P.L_out[0]; e /= P.L_out[0];
        if (!layout) { co = e % C_out; e /= C_out; }
        const int64_t n = e;
        const int64_t g = co / Cog, co_l = co % Cog;
        int64_t np[ORACLE_MAX_AXES];
        for (int a = 0; a < ORACLE_MAX_AXES; ++a)
            np[a] = pairs_hitting(o[a], P.L_in[a], P.K[a], P.s[a], P.p[a], P.d[a], pi[a], pk[a]);
        double acc = bias ? (double)bias[co] : 0.0;
        for (int64_t ci_l = 0; ci_l < Cig; ++ci_l) {
            const int64_t ci = g * Cig + ci_l;
            const float *wc = w + (ci * Cog + co_l) * k_sp;
            for (int64_t a0 = 0; a0 < np[0]; ++a0)
            for (int64_t a1 = 0; a1 < np[1]; ++a1)
            for (int64_t a2 = 0; a2 < np[2]; ++a2) {
                const int64_t ie = (pi[0][a0] * P.L_in[1] + pi[1][a1]) * P.L_in[2] + pi[2][a2];
                double xv = (double)x[at(layout, n, ci, ie, C_in, in_sp)];
                double wv = (double)wc[(pk[0][a0] * P.K[1] + pk[1][a1]) * P.K[2] + pk[2][a2]];
                acc += xv * wv;
            }
        }
        if (add) acc += (double)add[idx[t]];
        out[t] = activate(acc, act);
    }
    for (int a = 0; a < ORACLE_MAX_AXES; ++a) { free(pi[a]); free(pk[a]); }
    return rc;
}

/* Channels-first points, plain or (add != NULL) fused. */
int oracle_convt_points(int ndim, int64_t N, int64_t C_in, int64_t C_out, int64_t G,
                        const int64_t *in_size, const int64_t *K, const int64_t *s,
                        const int64_t *p, const int64_t *op, const int64_t *d,
                        const float *x, const float *w, const float *bias, const float *add,
                        const int64_t *idx, int64_t npts, double *out)
{
    return oracle_convt_points_ex(ndim, N, C_in, C_out, G, in_size, K, s, p, op, d, x, w, bias, add,
                                  add ? 2 : 0, 0, idx, npts, out);
}

/* The fused epilogue alone, elementwise: out[e] = t * hardswish(t), t = in[e]. */
void oracle_times_hardswish(const double *in, double *out, int64_t n)
{
    for (int64_t e = 0; e < n; ++e) out[e] = times_hardswish(in[e]);
}

/* An activation alone, elementwise: out[e] = activation act of in[e]. */
void oracle_activate(const double *in, double *out, int64_t n, int act)
{
    for (int64_t e = 0; e < n; ++e) out[e] = activate(in[e], act);
}

/* ---------------------------------------------------------------------------
 * Input gradient: the adjoint of the forward's linear part (no bias, no
 * epilogue).  The forward scatter adds x[n, ci, i] * w[ci, co_l, k] to
 * y[n, g*Cog + co_l, o] with o = i*s - p + k*d; its transpose therefore sends
 * dy[n, g*Cog + co_l, o] * w[ci, co_l, k] back to dx[n, ci, i], over the same
 * (i, k) pairs, dropping those whose o leaves [0, L_out) on some axis.
 * "Kimi-K2.6 l1_p79" transcript: the adjoint derivation that defines the
 * transposed convolution as the transpose of the strided convolution; "Kimi-K2.6
 * l2_p26" transcript: the convolution matrix C and its transpose C^T.
 */
typedef struct {
    const problem *P;
    const float *dy, *w;
    double *dx;
    int64_t next_slab, n_slabs;
    pthread_mutex_t lock;
} adjoint_job;

/* One (n, g) slab: the scatter loop of the forward, read backwards. */
static void adjoint_slab(const adjoint_job *J, int64_t n, int64_t g)
{
    const problem *P = J->P;
    const int64_t Cig = P->C_in / P->G, Cog = P->C_out / P->G;
    const int64_t ID = P->L_in[0], IH = P->L_in[1], IW = P->L_in[2];
    const int64_t OD = P->L_out[0], OH = P->L_out[1], OW = P->L_out[2];
    const int64_t KD = P->K[0], KH = P->K[1], KW = P->K[2];
    const int64_t in_sp = ID * IH * IW, out_sp = OD * OH * OW, k_sp = KD * KH * KW;

    for (int64_t ci_l = 0; ci_l < Cig; ++ci_l) {
        const int64_t ci = g * Cig + ci_l;
        double *dxc = J->dx + (n * P->C_in + ci) * in_sp;
        const float *wci = J->w + ci * Cog * k_sp;      /* w[ci][co_l][kd][kh][kw] */
        for (int64_t id = 0; id < ID; ++id)
        for (int64_t ih = 0; ih < IH; ++ih)
        for (int64_t iw = 0; iw < IW; ++iw) {
            double acc = 0.0;
            for (int64_t co_l = 0; co_l < Cog; ++co_l) {
                const float *dyc = J->dy + (n * P->C_out + g * Cog + co_l) * out_sp;
                for (int64_t kd = 0; kd < KD; ++kd) {
                    const int64_t zd = id * P->s[0] + kd * P->d[0] - P->p[0];
                    if (zd < 0 || zd >= OD) continue;
                    for (int64_t kh = 0; kh < KH; ++kh) {
                        const int64_t zh = ih * P->s[1] + kh * P->d[1] - P->p[1];
                        if (zh < 0 || zh >= OH) continue;
                        for (int64_t kw = 0; kw < KW; ++kw) {
                            const int64_t zw = iw * P->s[2] + kw * P->d[2] - P->p[2];
                            if (zw < 0 || zw >= OW) continue;
                            acc += (double)dyc[(zd * OH + zh) * OW + zw] *
                                   (double)wci[((co_l * KD + kd) * KH + kh) * KW + kw];
                        }
                    }
                }
            }
            dxc[(id * IH + ih) * IW + iw] = acc;
        }
    }
}

static void *adjoint_worker(void *arg)
{
    adjoint_job *J = (adjoint_job *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t t = J->next_slab++;
        pthread_mutex_unlock(&J->lock);
        if (t >= J->n_slabs) break;
        adjoint_slab(J, t / J->P->G, t % J->P->G);
    }
    return NULL;
}

/* dx (N*C_in*prod(L_in) doubles) from dy (N*C_out*prod(L_out) floats).
 * Returns 0, or 1 on bad arguments. */
int oracle_convt_backward_data(int ndim, int64_t N, int64_t C_in, int64_t C_out, int64_t G,
                               const int64_t *in_size, const int64_t *K, const int64_t *s,
                               const int64_t *p, const int64_t *op, const int64_t *d,
                               const float *dy, const float *w, double *dx, int nthreads)
{
    problem P;
    if (set_problem(&P, ndim, N, C_in, C_out, G, in_size, K, s, p, op, d)) return 1;
    adjoint_job J;
    J.P = &P; J.dy = dy; J.w = w; J.dx = dx;
    J.next_slab = 0; J.n_slabs = N * G;
    pthread_mutex_init(&J.lock, NULL);
    int nt = resolve_threads(nthreads);
    if (nt > J.n_slabs) nt = (int)(J.n_slabs > 0 ? J.n_slabs : 1);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) return 1;
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, adjoint_worker, &J);
    for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Weight and bias gradients.  The forward is linear in w: y depends on
 * w[ci, co_l, k] through the terms x[n, ci, i] * w[ci, co_l, k] landing on
 * y[n, g*Cog + co_l, o], o = i*s - p + k*d.  So for an output gradient dy
 *   dw[ci, co_l, k] = sum over n and the inputs i whose o lies in [0, L_out)
 *                     of x[n, ci, i] * dy[n, g*Cog + co_l, o]
 *   db[co]          = sum over n and every output position of dy[n, co, o]
 * (the bias is added once to every output element).  Same sources as the
 * forward; one thread per input channel, the sums in fp64.
 */
typedef struct {
    const problem *P;
    const float *x, *dy;
    double *dw;
    int64_t next, total;
    pthread_mutex_t lock;
} wgrad_job;

static void wgrad_channel(const wgrad_job *J, int64_t ci)
{
    const problem *P = J->P;
    const int64_t Cig = P->C_in / P->G, Cog = P->C_out / P->G, g = ci / Cig;
    const int64_t ID = P->L_in[0], IH = P->L_in[1], IW = P->L_in[2];
    const int64_t OD = P->L_out[0], OH = P->L_out[1], OW = P->L_out[2];
    const int64_t KD = P->K[0], KH = P->K[1], KW = P->K[2];
    const int64_t in_sp = ID * IH * IW, out_sp = OD * OH * OW;
    double *dwc = J->dw + ci * Cog * KD * KH * KW;   /* dw[ci][co_l][kd][kh][kw] */
    for (int64_t co_l = 0; co_l < Cog; ++co_l)
    for (int64_t kd = 0; kd < KD; ++kd)
    for (int64_t kh = 0; kh < KH; ++kh)
    for (int64_t kw = 0; kw < KW; ++kw) {
        double sum = 0.0;
        for (int64_t n = 0; n < P->N; ++n) {
            const float *xc = J->x + (n * P->C_in + ci) * in_sp;
            const float *dyc = J->dy + (n * P->C_out + (g * Cog + co_l)) * out_sp;
            for (int64_t id = 0; id < ID; ++id) {
                const int64_t vd = kd * P->d[0] + id * P->s[0] - P->p[0];
                if (vd < 0 || vd >= OD) continue;
                for (int64_t ih = 0; ih < IH; ++ih) {
                    const int64_t vh = kh * P->d[1] + ih * P->s[1] - P->p[1];
                    if (vh < 0 || vh >= OH) continue;
                    for (int64_t iw = 0; iw < IW; ++iw) {
                        const int64_t vw = kw * P->d[2] + iw * P->s[2] - P->p[2];
                        if (vw < 0 || vw >= OW) continue;
                        sum += (double)xc[(id * IH + ih) * IW + iw] * (double)dyc[(vd * OH + vh) * OW + vw];
                    }
                }
            }
        }
        dwc[((co_l * KD + kd) * KH + kh) * KW + kw] = sum;
    }
}

static void *wgrad_worker(void *arg)
{
    wgrad_job *J = (wgrad_job *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t t = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (t >= J->total) break;
        wgrad_channel(J, t);
    }
    return NULL;
}

/* dw (C_in*(C_out/G)*prod(K) doubles) and, if db != NULL, db (C_out doubles)
 * from x and dy.  Returns 0, or 1 on bad arguments. */
int oracle_convt_backward_weight(int ndim, int64_t N, int64_t C_in, int64_t C_out, int64_t G,
                                 const int64_t *in_size, const int64_t *K, const int64_t *s,
                                 const int64_t *p, const int64_t *op, const int64_t *d,
                                 const float *x, const float *dy, double *dw, double *db, int nthreads)
{
    problem P;
    if (set_problem(&P, ndim, N, C_in, C_out, G, in_size, K, s, p, op, d)) return 1;
    wgrad_job J;
    J.P = &P; J.x = x; J.dy = dy; J.dw = dw;
    J.next = 0; J.total = C_in;
    pthread_mutex_init(&J.lock, NULL);
    int nt = resolve_threads(nthreads);
    if (nt > J.total) nt = (int)J.total;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) return 1;
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, wgrad_worker, &J);
    for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    if (db) {
        const int64_t out_sp = P.L_out[0] * P.L_out[1] * P.L_out[2];
        for (int64_t co = 0; co < C_out; ++co) {
            double sum = 0.0;
            for (int64_t n = 0; n < N; ++n)
                for (int64_t e = 0; e < out_sp; ++e) sum += (double)dy[(n * C_out + co) * out_sp + e];
            db[co] = sum;
        }
    }
    return 0;
}
