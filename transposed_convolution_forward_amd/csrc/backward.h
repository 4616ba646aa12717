// Launch interface of the input-gradient kernel (backward.hip).
#pragma once

#include "convt_internal.h"

namespace convt {

// The kernel can run P: one tap's weights of one input channel for a group
// (C_out/G floats) fit in the 32 KB it stages per workgroup.
bool backward_data_supports(const convt_plan &P);
// Name of the kernel launch_backward_data runs for P (matrix-core or VALU).
const char *backward_data_kernel_name(const convt_plan &P);
// dx = the adjoint of the forward's linear part applied to dy; hipSuccess or
// the launch error (as int).
int launch_backward_data(const convt_plan &P, const float *dy, const float *w, float *dx, void *stream);

} // namespace convt
