// C ABI: validation, closed-form output size, per-axis phase tables, path
// selection and dispatch.  Host-only except for the launches in the per-path
// files; plan creation makes no HIP call.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <string>

#include "backward.h"
#include "wgrad.h"
#include "convt_internal.h"

using convt::AxisPlan;
using convt::kAxes;

namespace {

constexpr int64_t kMaxAxisParam = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxPerSample = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxTotal = int64_t(1) << 40;

// Closed form on every page: L_out = (L_in - 1)*s - 2p + d*(K - 1) + out_pad + 1.
int64_t closed_form(int64_t L_in, int64_t K, int64_t s, int64_t p, int64_t op, int64_t d) {
    return (L_in - 1) * s - 2 * p + d * (K - 1) + op + 1;
}

// Residue classes of the taps: k joins T_r for r = (k*d) mod s, with offset
// c = (k*d - r)/s, so that input i = q - c feeds output o = q*s + r - p.
void build_phase_table(AxisPlan &A) {
    int n = 0;
    for (int r = 0; r < A.s; ++r) {
        A.tap_start[r] = n;
        for (int k = 0; k < A.K; ++k) {
            const int64_t kd = (int64_t)k * A.d;
            if (kd % A.s == r) {
                A.tap_k[n] = k;
                A.tap_c[n] = (int)((kd - r) / A.s);
                ++n;
            }
        }
    }
    A.tap_start[A.s] = n;
}

convt_path choose_path(const convt_plan &P) {
    if (convt::stream1d_supports(P)) return CONVT_PATH_STREAM1D;
    if (convt::igemm3d_supports(P)) return CONVT_PATH_IGEMM3D;
    return CONVT_PATH_GENERIC;
}

bool path_supports(const convt_plan &P, convt_path path) {
    switch (path) {
    case CONVT_PATH_GENERIC: return convt::generic_supports(P);
    case CONVT_PATH_STREAM1D: return convt::stream1d_supports(P);
    case CONVT_PATH_IGEMM3D: return convt::igemm3d_supports(P);
    default: return false;
    }
}

const char *path_name(convt_path p) {
    switch (p) {
    case CONVT_PATH_AUTO: return "auto";
    case CONVT_PATH_GENERIC: return "generic";
    case CONVT_PATH_STREAM1D: return "stream1d";
    case CONVT_PATH_IGEMM3D: return "igemm3d";
    }
    return "?";
}

const char *kernel_name(const convt_plan &P) {
    const bool last = P.layout == CONVT_LAYOUT_CHANNELS_LAST;
    return P.path == CONVT_PATH_STREAM1D ? (last ? "k_stream1d_nlc" : "k_stream1d")
           : P.path == CONVT_PATH_IGEMM3D ? convt::igemm3d_kernel_name(P)
                                          : convt::generic_kernel_name(P);
}

// With CONVT_LOG set (to anything but 0), one line on stderr per planning
// decision: the shape, layout, path and kernel, and whether the shape fell to
// a generic kernel because no specialised one takes it.
void log_plan(const convt_plan &P, const char *why) {
    const char *env = getenv("CONVT_LOG");
    if (!env || !*env || !strcmp(env, "0")) return;
    std::string axes;
    char tmp[160];
    for (int a = kAxes - P.ndim; a < kAxes; ++a) {
        const AxisPlan &A = P.ax[a];
        snprintf(tmp, sizeof tmp, "%s[L=%d K=%d s=%d p=%d op=%d d=%d]", axes.empty() ? "" : " ", A.L_in, A.K, A.s,
                 A.p, A.op, A.d);
        axes += tmp;
    }
    fprintf(stderr, "convt: %s: ndim=%d N=%lld C_in=%lld C_out=%lld groups=%lld %s layout=%s -> path=%s kernel=%s%s\n",
            why, P.ndim, (long long)P.N, (long long)P.C_in, (long long)P.C_out, (long long)P.G, axes.c_str(),
            P.layout == CONVT_LAYOUT_CHANNELS_LAST ? "channels_last" : "channels_first", path_name(P.path),
            kernel_name(P),
            P.path == CONVT_PATH_GENERIC && P.auto_path == CONVT_PATH_GENERIC
                ? " (generic fallback: no specialised kernel takes this shape)"
                : P.path != P.auto_path ? " (forced)" : "");
}

// The planner's path for the plan's shape and layout, then the CONVT_PATH
// environment override (generic, stream1d or igemm3d) where that path applies.
void select_path(convt_plan &P) {
    P.auto_path = choose_path(P);
    P.path = P.auto_path;
    const char *env = getenv("CONVT_PATH");
    if (env && *env && strcmp(env, "auto") != 0) {
        convt_path want = CONVT_PATH_AUTO;
        if (!strcmp(env, "generic")) want = CONVT_PATH_GENERIC;
        else if (!strcmp(env, "stream1d")) want = CONVT_PATH_STREAM1D;
        else if (!strcmp(env, "igemm3d")) want = CONVT_PATH_IGEMM3D;
        if (want != CONVT_PATH_AUTO && path_supports(P, want)) P.path = want;
    }
}

convt_status dispatch(const convt_plan *plan, const float *x, const float *w, const float *bias,
                      const float *add, int act, float *y, void *stream) {
    int e = 0;
    switch (plan->path) {
    case CONVT_PATH_STREAM1D: e = convt::launch_stream1d(*plan, x, w, bias, add, act, y, stream); break;
    case CONVT_PATH_IGEMM3D: e = convt::launch_igemm3d(*plan, x, w, bias, add, act, y, stream); break;
    case CONVT_PATH_GENERIC: e = convt::launch_generic(*plan, x, w, bias, add, act, y, stream); break;
    default: return CONVT_ERR_UNSUPPORTED;
    }
    return e == 0 ? CONVT_OK : CONVT_ERR_HIP;
}

} // namespace

extern "C" {

convt_status convt_plan_create(convt_plan **plan, int ndim, int64_t N, int64_t C_in,
                               int64_t C_out, int64_t groups, const int64_t *in_size,
                               const int64_t *K, const int64_t *stride, const int64_t *pad,
                               const int64_t *out_pad, const int64_t *dilation) {
    if (!plan) return CONVT_ERR_INVALID_ARG;
    *plan = nullptr;
    if (ndim < 1 || ndim > kAxes) return CONVT_ERR_INVALID_ARG;
    if (!in_size || !K || !stride || !pad || !out_pad || !dilation) return CONVT_ERR_INVALID_ARG;
    if (N < 1 || C_in < 1 || C_out < 1 || groups < 1) return CONVT_ERR_INVALID_ARG;
    if (C_in % groups != 0 || C_out % groups != 0) return CONVT_ERR_INVALID_ARG;
    for (int a = 0; a < ndim; ++a) {
        if (in_size[a] < 1 || K[a] < 1 || stride[a] < 1 || dilation[a] < 1 || pad[a] < 0 ||
            out_pad[a] < 0)
            return CONVT_ERR_INVALID_ARG;
    }
    for (int a = 0; a < ndim; ++a) {
        if (in_size[a] > kMaxAxisParam || pad[a] > kMaxAxisParam || out_pad[a] > kMaxAxisParam ||
            dilation[a] > kMaxAxisParam)
            return CONVT_ERR_UNSUPPORTED;
        if (K[a] > convt::kMaxK || stride[a] > convt::kMaxStride) return CONVT_ERR_UNSUPPORTED;
        // The uncropped scatter length (L_in - 1)*s + d*(K - 1) + out_pad + 1
        // bounds every index i*s - p + k*d the kernels form in int; a large
        // padding can cancel it in the closed form, so it is bounded itself.
        if ((in_size[a] - 1) * stride[a] + dilation[a] * (K[a] - 1) + out_pad[a] + 1 > kMaxAxisParam)
            return CONVT_ERR_UNSUPPORTED;
    }
    if (N > kMaxAxisParam || C_in > kMaxAxisParam || C_out > kMaxAxisParam)
        return CONVT_ERR_UNSUPPORTED;

    convt_plan *P = new (std::nothrow) convt_plan;
    if (!P) return CONVT_ERR_NOMEM;
    memset(P, 0, sizeof(*P));
    P->ndim = ndim;
    P->N = N;
    P->C_in = C_in;
    P->C_out = C_out;
    P->G = groups;
    P->Cig = C_in / groups;
    P->Cog = C_out / groups;
    const int lead = kAxes - ndim;
    P->in_sp = P->out_sp = P->k_vol = 1;
    for (int a = 0; a < kAxes; ++a) {
        AxisPlan &A = P->ax[a];
        int64_t L_out = 1;
        if (a < lead) {
            A.L_in = A.K = A.s = A.d = 1;
            A.p = A.op = 0;
        } else {
            const int b = a - lead;
            L_out = closed_form(in_size[b], K[b], stride[b], pad[b], out_pad[b], dilation[b]);
            if (L_out < 1) { delete P; return CONVT_ERR_INVALID_ARG; }
            if (L_out > kMaxAxisParam) { delete P; return CONVT_ERR_UNSUPPORTED; }
            A.L_in = (int)in_size[b];
            A.K = (int)K[b];
            A.s = (int)stride[b];
            A.p = (int)pad[b];
            A.op = (int)out_pad[b];
            A.d = (int)dilation[b];
        }
        A.L_out = (int)L_out;
        build_phase_table(A);
        P->in_sp *= A.L_in;
        P->out_sp *= A.L_out;
        P->k_vol *= A.K;
        if (P->in_sp > kMaxPerSample || P->out_sp > kMaxPerSample) {
            delete P;
            return CONVT_ERR_UNSUPPORTED;
        }
    }
    if (P->C_in * P->in_sp > kMaxPerSample || P->C_out * P->out_sp > kMaxPerSample ||
        P->C_in * P->Cog * P->k_vol > kMaxPerSample || N * P->C_in * P->in_sp > kMaxTotal ||
        N * P->C_out * P->out_sp > kMaxTotal) {
        delete P;
        return CONVT_ERR_UNSUPPORTED;
    }
    if (!convt::generic_supports(*P)) { delete P; return CONVT_ERR_UNSUPPORTED; }
    select_path(*P);
    log_plan(*P, "plan");
    *plan = P;
    return CONVT_OK;
}

convt_status convt_plan_set_layout(convt_plan *plan, int layout) {
    if (!plan) return CONVT_ERR_INVALID_ARG;
    if (layout != CONVT_LAYOUT_CHANNELS_FIRST && layout != CONVT_LAYOUT_CHANNELS_LAST) return CONVT_ERR_INVALID_ARG;
    const int old = plan->layout;
    plan->layout = layout;
    if (!convt::generic_supports(*plan)) {
        plan->layout = old;
        return CONVT_ERR_UNSUPPORTED;
    }
    select_path(*plan);
    log_plan(*plan, "layout");
    return CONVT_OK;
}

int convt_plan_get_layout(const convt_plan *plan) { return plan ? plan->layout : -1; }

convt_status convt_plan_output_size(const convt_plan *plan, int64_t *out_size) {
    if (!plan || !out_size) return CONVT_ERR_INVALID_ARG;
    const int lead = kAxes - plan->ndim;
    for (int b = 0; b < plan->ndim; ++b) out_size[b] = plan->ax[lead + b].L_out;
    return CONVT_OK;
}

convt_status convt_forward(const convt_plan *plan, const float *x, const float *w,
                           const float *bias, float *y, void *stream) {
    if (!plan || !x || !w || !y) return CONVT_ERR_INVALID_ARG;
    return dispatch(plan, x, w, bias, nullptr, CONVT_ACT_NONE, y, stream);
}

convt_status convt_forward_add_hswish(const convt_plan *plan, const float *x, const float *w,
                                      const float *bias, const float *add_input, float *y,
                                      void *stream) {
    if (!plan || !x || !w || !y || !add_input) return CONVT_ERR_INVALID_ARG;
    return dispatch(plan, x, w, bias, add_input, CONVT_ACT_X_HARDSWISH, y, stream);
}

convt_status convt_forward_epilogue(const convt_plan *plan, const float *x, const float *w,
                                    const float *bias, const float *add_input, int activation, float *y,
                                    void *stream) {
    if (!plan || !x || !w || !y) return CONVT_ERR_INVALID_ARG;
    if (activation != CONVT_ACT_NONE && activation != CONVT_ACT_HARDSWISH && activation != CONVT_ACT_X_HARDSWISH)
        return CONVT_ERR_INVALID_ARG;
    return dispatch(plan, x, w, bias, add_input, activation, y, stream);
}

convt_status convt_backward_data(const convt_plan *plan, const float *dy, const float *w, float *dx,
                                 void *stream) {
    if (!plan || !dy || !w || !dx) return CONVT_ERR_INVALID_ARG;
    if (plan->layout != CONVT_LAYOUT_CHANNELS_FIRST || !convt::backward_data_supports(*plan))
        return CONVT_ERR_UNSUPPORTED;
    return convt::launch_backward_data(*plan, dy, w, dx, stream) == 0 ? CONVT_OK : CONVT_ERR_HIP;
}

convt_status convt_backward_weight(const convt_plan *plan, const float *x, const float *dy, float *dw,
                                   float *db, void *stream) {
    if (!plan || !x || !dy || !dw) return CONVT_ERR_INVALID_ARG;
    if (plan->layout != CONVT_LAYOUT_CHANNELS_FIRST || !convt::backward_weight_supports(*plan))
        return CONVT_ERR_UNSUPPORTED;
    return convt::launch_backward_weight(*plan, x, dy, dw, db, stream) == 0 ? CONVT_OK : CONVT_ERR_HIP;
}

void convt_plan_destroy(convt_plan *plan) { delete plan; }

const char *convt_status_string(convt_status s) {
    switch (s) {
    case CONVT_OK: return "ok";
    case CONVT_ERR_INVALID_ARG: return "invalid argument";
    case CONVT_ERR_UNSUPPORTED: return "unsupported";
    case CONVT_ERR_HIP: return "HIP runtime error";
    case CONVT_ERR_NOMEM: return "out of host memory";
    }
    return "unknown status";
}

convt_status convt_plan_set_path(convt_plan *plan, convt_path path) {
    if (!plan) return CONVT_ERR_INVALID_ARG;
    if (path == CONVT_PATH_AUTO) {
        plan->path = plan->auto_path;
        return CONVT_OK;
    }
    if (path != CONVT_PATH_GENERIC && path != CONVT_PATH_STREAM1D && path != CONVT_PATH_IGEMM3D)
        return CONVT_ERR_INVALID_ARG;
    if (!path_supports(*plan, path)) return CONVT_ERR_UNSUPPORTED;
    plan->path = path;
    log_plan(*plan, "set_path");
    return CONVT_OK;
}

convt_path convt_plan_get_path(const convt_plan *plan) {
    return plan ? plan->path : CONVT_PATH_AUTO;
}

int64_t convt_plan_describe(const convt_plan *plan, char *buf, int64_t len) {
    if (!plan) return -1;
    std::string s;
    char tmp[256];
    const bool last = plan->layout == CONVT_LAYOUT_CHANNELS_LAST;
    const char *kernel = kernel_name(*plan);
    snprintf(tmp, sizeof tmp,
             "convt plan: ndim=%d N=%lld C_in=%lld C_out=%lld groups=%lld layout=%s path=%s kernel=%s\n",
             plan->ndim, (long long)plan->N, (long long)plan->C_in, (long long)plan->C_out,
             (long long)plan->G, last ? "channels_last" : "channels_first", path_name(plan->path), kernel);
    s += tmp;
    for (int a = kAxes - plan->ndim; a < kAxes; ++a) {
        const AxisPlan &A = plan->ax[a];
        snprintf(tmp, sizeof tmp, "  axis %d: L_in=%d K=%d s=%d p=%d op=%d d=%d -> L_out=%d;",
                 a - (kAxes - plan->ndim), A.L_in, A.K, A.s, A.p, A.op, A.d, A.L_out);
        s += tmp;
        for (int r = 0; r < A.s; ++r) {
            s += " r" + std::to_string(r) + ":{";
            for (int j = A.tap_start[r]; j < A.tap_start[r + 1]; ++j) {
                snprintf(tmp, sizeof tmp, "%sk%d/c%d", j > A.tap_start[r] ? "," : "", A.tap_k[j],
                         A.tap_c[j]);
                s += tmp;
            }
            s += "}";
        }
        s += "\n";
    }
    if (!last && convt::backward_data_supports(*plan)) {
        s += "  input gradient: kernel=";
        s += convt::backward_data_kernel_name(*plan);
        s += "\n";
    }
    if (!last && convt::backward_weight_supports(*plan)) {
        s += "  weight gradient: kernel=";
        s += convt::backward_weight_kernel_name(*plan);
        s += "\n";
    }
    if (buf && len > 0) {
        const size_t n = s.size() < (size_t)(len - 1) ? s.size() : (size_t)(len - 1);
        memcpy(buf, s.data(), n);
        buf[n] = '\0';
    }
    return (int64_t)s.size();
}

} // extern "C"
