// Launch interface of the input-gradient kernel (backward.hip).
#pragma once

#include "convt_internal.h"

namespace convt {

// The kernel can run P: one input channel's weights for a group (C_out/G x
// prod(K) floats) fit in the 32 KB it stages per workgroup.
bool backward_data_supports(const convt_plan &P);
// dx = the adjoint of the forward's linear part applied to dy; hipSuccess or
// the launch error (as int).
int launch_backward_data(const convt_plan &P, const float *dy, const float *w, float *dx, void *stream);

} // namespace convt
