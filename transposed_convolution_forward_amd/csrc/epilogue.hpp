// Output epilogue, applied in registers just before the single store of an
// output element.
//
// Plain:  y = acc + bias
// Fused ("Kimi-K2.6 l2_p26" transcript, ConvTranspose3d + add + HardSwish: its
// forward, then hardswish(t) = t * clamp(t + 3, 0, 6) / 6):
//   t = acc + bias + add_input,  y = t * hardswish(t) = t * t * clamp(t+3,0,6) / 6
#pragma once

#include <hip/hip_runtime.h>

namespace convt {

__device__ __forceinline__ float times_hardswish(float t) {
    // clamp(t+3, 0, 6)/6 = clamp(t/6 + 1/2, 0, 1): one FMA and one clamp (1/6
    // rounded to fp32: within an ulp of dividing), then t*t times it
    const float r = fminf(fmaxf(fmaf(t, 1.0f / 6.0f, 0.5f), 0.0f), 1.0f);
    return (t * t) * r;
}

template <bool FUSED>
__device__ __forceinline__ float epilogue(float acc, float bias, float add) {
    float v = acc + bias;
    if constexpr (FUSED) return times_hardswish(v + add);
    return v;
}

} // namespace convt
