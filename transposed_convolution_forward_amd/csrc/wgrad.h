// Launch interface of the weight- and bias-gradient kernels (wgrad.hip).
#pragma once

#include "convt_internal.h"

namespace convt {

// The kernels can run P (buffer offsets of a group's x and dy below 2 GiB,
// grid limits).
bool backward_weight_supports(const convt_plan &P);
// Name of the weight-gradient kernel launch_backward_weight runs for P.
const char *backward_weight_kernel_name(const convt_plan &P);
// dw (and db unless NULL) from x and dy, both cleared first; hipSuccess or the
// launch error (as int).
int launch_backward_weight(const convt_plan &P, const float *x, const float *dy, float *dw, float *db,
                           void *stream);

} // namespace convt
