/*
 * convt.h -- transposed-convolution forward pass on AMD Instinct MI355X (gfx950).
 *
 * The operation (the scatter definition the source pages settle on):
 *   every input element x[n, ci, i] (i a position per spatial axis) times every
 *   kernel tap w[ci, co_l, k] of its group is added to
 *   y[n, g*(C_out/G) + co_l, o] at o = i*s - p + k*d on each axis; writes
 *   outside [0, L_out) are dropped; bias[co] is added once to every output
 *   element; input channel ci belongs to group g = ci / (C_in/G).
 *   Sources: "Kimi-K2.6 l1_p79" transcript (ConvTranspose1d, dilation 2),
 *   scatter-then-crop derivation and its two-input worked example;
 *   "Kimi-K2.6 l1_p72" transcript (ConvTranspose3d, groups 4), the per-group
 *   reference loop with bias.
 *
 * Output size per axis (closed form, all three pages):
 *   L_out = (L_in - 1)*s - 2p + d*(K - 1) + out_pad + 1
 *
 * Layouts (all float32, contiguous, row-major, caller-owned DEVICE memory):
 *   x         (N, C_in, L_in...)             NCL / NCHW / NCDHW
 *   w         (C_in, C_out/groups, K...)     used as stored (no flip)
 *   bias      (C_out)                        may be NULL (no bias)
 *   add_input (N, C_out, L_out...)           same shape as y
 *   y         (N, C_out, L_out...)           every element is written
 * or, after convt_plan_set_layout(plan, CONVT_LAYOUT_CHANNELS_LAST), x as
 * (N, L_in..., C_in) and y and add_input as (N, L_out..., C_out).
 * No alignment is required of any pointer beyond that of float.
 *
 * Ownership and threading: a plan holds host metadata only; it allocates no
 * device memory, and no call allocates device memory.  Calls are asynchronous
 * on the given HIP stream (hipStream_t passed as void*; NULL = null stream)
 * and never synchronise.  A plan is immutable after creation apart from
 * convt_plan_set_path; forward calls on one plan may run concurrently on any
 * streams.
 *
 * Aliasing: x and w must not overlap y.  add_input == y (in place) is allowed:
 * each element is read and then written by the same thread.
 *
 * Errors: status codes only; nothing is thrown across this boundary.
 *
 * Environment: CONVT_LOG=1 prints one line on stderr per planning decision
 * (plan creation, convt_plan_set_layout, convt_plan_set_path): the shape,
 * the path and kernel chosen, and whether the shape fell to a generic kernel
 * because no specialised one takes it.  CONVT_PATH=generic|stream1d|igemm3d
 * forces that path on every plan it applies to.
 */
#ifndef CONVT_H
#define CONVT_H

#include <stdint.h>

#if defined(__GNUC__)
#define CONVT_API __attribute__((visibility("default")))
#else
#define CONVT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONVT_OK = 0,
    CONVT_ERR_INVALID_ARG = 1, /* NULL pointer, or a shape/parameter the closed form rejects */
    CONVT_ERR_UNSUPPORTED = 2, /* valid, but beyond this library's limits or the forced path */
    CONVT_ERR_HIP = 3,         /* the HIP runtime reported an error (launch or device) */
    CONVT_ERR_NOMEM = 4        /* host allocation of the plan failed */
} convt_status;

typedef enum {
    CONVT_PATH_AUTO = 0,     /* let the planner choose (the default) */
    CONVT_PATH_GENERIC = 1,  /* output-stationary phase-table gather, any shape */
    CONVT_PATH_STREAM1D = 2, /* 1D streaming kernel, MFMA channel contraction */
    CONVT_PATH_IGEMM3D = 3   /* per-phase implicit GEMM on MFMA for 2D and 3D */
} convt_path;

/*
 * Activations of the selectable epilogue ("Kimi-K2.6 l2_p26" transcript,
 * ConvTranspose3d + add + HardSwish: its statement of hardswish and of the
 * forward, which multiplies the sum by its hardswish).
 */
typedef enum {
    CONVT_ACT_NONE = 0,       /* y = t */
    CONVT_ACT_HARDSWISH = 1,  /* y = hardswish(t) = t * min(max(t + 3, 0), 6) / 6 */
    CONVT_ACT_X_HARDSWISH = 2 /* y = t * hardswish(t) */
} convt_activation;

/*
 * Memory layout of x, y and add_input (the weight is always
 * (C_in, C_out/groups, K...)).  Channels last makes the C_out values of one
 * output position contiguous ("Kimi-K2.6 l1_p79" transcript: its fast-kernel
 * section finds the channels-first output stores of neighbouring threads far
 * apart; "Kimi-K2.6 l2_p26" transcript: its note on channels-last 3D
 * tensors for library convolutions).
 */
typedef enum {
    CONVT_LAYOUT_CHANNELS_FIRST = 0, /* NCL / NCHW / NCDHW (the default) */
    CONVT_LAYOUT_CHANNELS_LAST = 1   /* NLC / NHWC / NDHWC */
} convt_layout;

typedef struct convt_plan convt_plan; /* opaque */

/*
 * Create a plan.  ndim is 1, 2 or 3; in_size, K, stride, pad, out_pad and
 * dilation are arrays of ndim entries (outermost spatial axis first).
 * Requirements (else CONVT_ERR_INVALID_ARG): N >= 1, C_in >= 1, C_out >= 1,
 * groups >= 1 dividing both C_in and C_out; per axis L_in >= 1, K >= 1,
 * stride >= 1, dilation >= 1, pad >= 0, out_pad >= 0, and L_out >= 1 by the
 * closed form.  Any out_pad >= 0 is accepted (the pages state no upper
 * bound).  Limits (else CONVT_ERR_UNSUPPORTED): K <= 32 and stride <= 32 per
 * axis, the uncropped length (L_in - 1)*s + d*(K - 1) + out_pad + 1 below
 * 2^31 per axis, every tensor below 2^31 elements per batch sample and below
 * 2^40 elements in total.  Host-only: makes no HIP call.  On success *plan owns a
 * heap object released by convt_plan_destroy.
 */
CONVT_API convt_status convt_plan_create(convt_plan **plan, int ndim, int64_t N, int64_t C_in,
                               int64_t C_out, int64_t groups, const int64_t *in_size,
                               const int64_t *K, const int64_t *stride, const int64_t *pad,
                               const int64_t *out_pad, const int64_t *dilation);

/* Write the ndim output sizes (closed form) to out_size.  Host-only. */
CONVT_API convt_status convt_plan_output_size(const convt_plan *plan, int64_t *out_size);

/*
 * y = conv_transpose(x, w) + bias.  bias may be NULL.  All pointers device
 * memory, layouts above.  Returns CONVT_ERR_INVALID_ARG for NULL plan, x, w
 * or y; CONVT_ERR_HIP if the launch fails.
 */
CONVT_API convt_status convt_forward(const convt_plan *plan, const float *x, const float *w,
                           const float *bias, float *y, void *stream);

/*
 * Fused epilogue ("Kimi-K2.6 l2_p26" transcript, ConvTranspose3d + add +
 * HardSwish, its forward and its statement of hardswish):
 *   t = conv_transpose(x, w) + bias + add_input
 *   y = t * hardswish(t) = t * t * min(max(t + 3, 0), 6) / 6
 * computed in registers, one store per element.  bias may be NULL; add_input
 * may equal y.  Errors as convt_forward (add_input NULL is INVALID_ARG).
 */
CONVT_API convt_status convt_forward_add_hswish(const convt_plan *plan, const float *x, const float *w,
                                      const float *bias, const float *add_input, float *y,
                                      void *stream);

/*
 * Forward with a selectable epilogue, computed in registers before the one
 * store of each output element:
 *   t = conv_transpose(x, w) + bias [+ add_input]
 *   y = t, hardswish(t) or t * hardswish(t)   (activation, see above)
 * bias may be NULL (no bias); add_input may be NULL (no residual add) and may
 * equal y (in place).  convt_forward is this call with add_input NULL and
 * CONVT_ACT_NONE; convt_forward_add_hswish with add_input and
 * CONVT_ACT_X_HARDSWISH.  Every path runs every mode.  Errors as
 * convt_forward, and CONVT_ERR_INVALID_ARG for an activation outside the
 * enum.
 */
CONVT_API convt_status convt_forward_epilogue(const convt_plan *plan, const float *x, const float *w,
                                              const float *bias, const float *add_input, int activation,
                                              float *y, void *stream);

/*
 * Input gradient: dx = the adjoint of the forward's linear part applied to dy
 * (no bias or epilogue term), i.e. for every input position i and channel ci
 * of group g
 *   dx[n, ci, i] = sum over co_l < C_out/G and taps k whose o = i*s - p + k*d
 *                  lies in [0, L_out) on every axis of w[ci, co_l, k] * dy[n, g*(C_out/G) + co_l, o].
 * "Kimi-K2.6 l1_p79" transcript (ConvTranspose1d, dilation 2): the adjoint
 * derivation, the transposed convolution being the transpose of the strided
 * convolution; "Kimi-K2.6 l2_p26" transcript: the matrix C and its transpose.
 * dy has y's layout (N, C_out, L_out...), dx has x's (N, C_in, L_in...), w as
 * in the forward; all device memory, caller-owned; every dx element is
 * written.  dy and w must not overlap dx.  Asynchronous on stream like the
 * forward.  Returns CONVT_ERR_INVALID_ARG for NULL plan, dy, w or dx;
 * CONVT_ERR_UNSUPPORTED if C_out/G > 8192; CONVT_ERR_HIP if the launch
 * fails.
 */
CONVT_API convt_status convt_backward_data(const convt_plan *plan, const float *dy, const float *w,
                                           float *dx, void *stream);

/*
 * Weight and bias gradients for an output gradient dy.  The forward is linear
 * in w and b (the scatter definition above), so
 *   dw[ci, co_l, k] = sum over n and the input positions i whose
 *                     o = i*s - p + k*d lies in [0, L_out) on every axis of
 *                     x[n, ci, i] * dy[n, g*(C_out/G) + co_l, o]
 *   db[co]          = sum over n and every output position of dy[n, co, o]
 * Sources as the forward ("Kimi-K2.6 l1_p79" transcript, the scatter
 * definition; "Kimi-K2.6 l1_p72" transcript, the per-group loop with bias).
 * x and dy as in the forward and the input gradient; dw has w's layout
 * (C_in, C_out/groups, K...), db is (C_out) or NULL (not computed).  dw and db
 * are overwritten (the call clears them, then adds partial sums over ranges
 * of positions with fp32 atomics, so the low bits of the result vary from run
 * to run).  All device memory, caller-owned; dw and db must not overlap x or
 * dy.  Asynchronous on stream; no device allocation.  Returns
 * CONVT_ERR_INVALID_ARG for NULL plan, x, dy or dw; CONVT_ERR_UNSUPPORTED if a
 * group's slice of x or dy for one sample is 2 GiB or more, or N > 65535;
 * CONVT_ERR_HIP if a launch fails.
 */
CONVT_API convt_status convt_backward_weight(const convt_plan *plan, const float *x, const float *dy,
                                             float *dw, float *db, void *stream);

/* Release a plan.  NULL is a no-op. */
CONVT_API void convt_plan_destroy(convt_plan *plan);

/* Static, NUL-terminated description of a status code. */
CONVT_API const char *convt_status_string(convt_status status);

/*
 * Force a kernel path (CONVT_PATH_AUTO restores the planner's choice).
 * Returns CONVT_ERR_UNSUPPORTED, leaving the plan unchanged, if that path
 * cannot run this plan.  Host-only; not safe concurrently with forward calls
 * on the same plan.
 */
CONVT_API convt_status convt_plan_set_path(convt_plan *plan, convt_path path);

/*
 * Set the layout of x, y and add_input for the plan's calls (convt_layout;
 * a new plan is CONVT_LAYOUT_CHANNELS_FIRST).  The planner's path is chosen
 * again for the layout and any forced path is dropped.  Every forward call
 * and every epilogue mode takes both layouts; the gradient calls take
 * channels first only (CONVT_ERR_UNSUPPORTED otherwise).  Returns
 * CONVT_ERR_INVALID_ARG for a NULL plan or a value outside the enum,
 * CONVT_ERR_UNSUPPORTED (plan unchanged) if the shape is beyond the layout's
 * limits.  Host-only; not safe concurrently with calls on the same plan.
 */
CONVT_API convt_status convt_plan_set_layout(convt_plan *plan, int layout);

/* The plan's layout (convt_layout), or -1 for a NULL plan. */
CONVT_API int convt_plan_get_layout(const convt_plan *plan);

/* The path forward calls will take (never CONVT_PATH_AUTO). */
CONVT_API convt_path convt_plan_get_path(const convt_plan *plan);

/*
 * Human-readable summary of the plan (shapes, phase tables, chosen path and
 * the kernel that path runs, and the gradient kernels) into buf (NUL-terminated, truncated to len).  Returns the
 * length the full text needs, excluding the NUL.  Host-only.
 */
CONVT_API int64_t convt_plan_describe(const convt_plan *plan, char *buf, int64_t len);

#ifdef __cplusplus
}
#endif

#endif /* CONVT_H */
