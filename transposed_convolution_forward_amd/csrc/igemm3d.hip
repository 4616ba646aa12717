// 3D implicit-GEMM path (placeholder until the MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "convt_internal.h"

namespace convt {
bool igemm3d_supports(const convt_plan &) { return false; }
int launch_igemm3d(const convt_plan &, const float *, const float *, const float *,
                   const float *, float *, void *) {
    return (int)hipErrorInvalidValue;
}
} // namespace convt
