// Internal plan representation and per-kernel launch interfaces.
//
// Phase decomposition (the gather form of the scatter definition): on one axis,
// output position o receives tap k from input i = (o + p - k*d)/s exactly when
// s divides o + p - k*d.  Write t = o + p = q*s + r with 0 <= r < s.  Then tap k
// contributes iff k*d = r (mod s), and then i = q - c_k with
// c_k = (k*d - r)/s >= 0.  So the residue r selects a fixed tap set T_r (a dense
// stride-1 sub-kernel) and every output of that phase is
//   y[o] = bias + sum_{k in T_r, 0 <= q - c_k < L_in} x[q - c_k] * w[k].
// An empty T_r leaves the bias.  "Kimi-K2.6 l1_p79" transcript (ConvTranspose1d,
// dilation 2): the odd-position analysis and the general divisibility test;
// "Kimi-K2.6 l1_p72" transcript (ConvTranspose3d): the per-axis input-range
// formula and the parity-class (phase) blocking.
#pragma once

#include <stdint.h>

#include "convt.h"

namespace convt {

constexpr int kAxes = 3;       // every problem is padded to 3 spatial axes
constexpr int kMaxStride = 32; // per-axis limit on s (table size)
constexpr int kMaxK = 32;      // per-axis limit on K (table size)

// One spatial axis with its phase table.  Padded (unit) axes have
// L_in = L_out = K = s = d = 1, p = out_pad = 0 and one tap {k=0, c=0}.
struct AxisPlan {
    int L_in, L_out, K, s, p, op, d;
    int tap_start[kMaxStride + 1]; // taps of residue r are [tap_start[r], tap_start[r+1])
    int tap_k[kMaxK];              // sorted by k within a residue
    int tap_c[kMaxK];              // i = q - c
};

} // namespace convt

struct convt_plan {
    int ndim;
    int64_t N, C_in, C_out, G, Cig, Cog;
    convt::AxisPlan ax[convt::kAxes]; // [0] = depth (outermost), [2] = width
    int64_t in_sp, out_sp, k_vol;     // spatial volumes
    convt_path auto_path;             // planner's choice
    convt_path path;                  // path the forward calls take
    int layout;                       // convt_layout of x, y and add_input
};

namespace convt {

// Kernel launchers, one per path.  The epilogue is t = acc + bias, plus
// add_input when add != nullptr, then the activation act (kActNone,
// kActHardswish or kActXHardswish, epilogue.hpp).  Each returns hipSuccess or
// the launch error (as int, to keep HIP types out).
bool generic_supports(const convt_plan &P);
// Name of the kernel launch_generic runs for P (phase-class variant when the
// shape has at most 32 phase classes).
const char *generic_kernel_name(const convt_plan &P);
int launch_generic(const convt_plan &P, const float *x, const float *w, const float *bias,
                   const float *add, int act, float *y, void *stream);

// Groups of 8 input and 8 output channels with stride 2 and dilation 1 along W
// (the generic path's first choice when it applies).
bool wpair_supports(const convt_plan &P);
int launch_wpair(const convt_plan &P, const float *x, const float *w, const float *bias, const float *add,
                 int act, float *y, void *stream);

bool stream1d_supports(const convt_plan &P);
int launch_stream1d(const convt_plan &P, const float *x, const float *w, const float *bias,
                    const float *add, int act, float *y, void *stream);

bool igemm3d_supports(const convt_plan &P);
// Name of the kernel launch_igemm3d runs for P (weights in VGPRs or streamed).
const char *igemm3d_kernel_name(const convt_plan &P);
int launch_igemm3d(const convt_plan &P, const float *x, const float *w, const float *bias,
                   const float *add, int act, float *y, void *stream);

} // namespace convt
