// Output epilogue, applied in registers just before the single store of an
// output element.  A compile-time code EPI selects it:
//   t = acc + bias [+ add_input]     (add_input when epi_add(EPI))
//   y = t                            (epi_act(EPI) == kActNone)
//   y = hardswish(t)                 (kActHardswish)
//   y = t * hardswish(t)             (kActXHardswish)
// with hardswish(t) = t * clamp(t + 3, 0, 6) / 6.  "Kimi-K2.6 l2_p26"
// transcript (ConvTranspose3d + add + HardSwish): its forward adds add_input
// to the convolution and multiplies the sum by its hardswish; the page states
// hardswish as above.  The residual add and the two activations are the parts
// of that forward, offered singly and together.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "convt.h"

namespace convt {

constexpr int kActNone = CONVT_ACT_NONE, kActHardswish = CONVT_ACT_HARDSWISH,
              kActXHardswish = CONVT_ACT_X_HARDSWISH;
constexpr int kNumActs = 3;

constexpr int epi_code(bool add, int act) { return act * 2 + (add ? 1 : 0); }
constexpr bool epi_add(int epi) { return (epi & 1) != 0; }
constexpr int epi_act(int epi) { return epi >> 1; }
constexpr int kEpiPlain = epi_code(false, kActNone);

// clamp(t+3, 0, 6)/6 = clamp(t/6 + 1/2, 0, 1): one FMA and one clamp (1/6
// rounded to fp32: within an ulp of dividing)
__device__ __forceinline__ float hswish_gate(float t) { return fminf(fmaxf(fmaf(t, 1.0f / 6.0f, 0.5f), 0.0f), 1.0f); }

__device__ __forceinline__ float times_hardswish(float t) { return (t * t) * hswish_gate(t); }

template <int EPI> __device__ __forceinline__ float activate(float t) {
    if constexpr (epi_act(EPI) == kActXHardswish) return times_hardswish(t);
    else if constexpr (epi_act(EPI) == kActHardswish) return t * hswish_gate(t);
    else return t;
}

// t = v [+ add], then the activation: v already holds acc + bias.
template <int EPI> __device__ __forceinline__ float finish(float v, float add) {
    if constexpr (epi_add(EPI)) return activate<EPI>(v + add);
    else return activate<EPI>(v);
}

template <int EPI> __device__ __forceinline__ float epilogue(float acc, float bias, float add) {
    return finish<EPI>(acc + bias, add);
}

// Calls f(std::integral_constant<int, EPI>{}) for the code of (add, act);
// act outside [0, kNumActs) is the caller's error (checked at the ABI).
template <typename F> __host__ auto with_epi(bool add, int act, F &&f) {
    const int e = epi_code(add, act);
    switch (e) {
    case 0: return f(std::integral_constant<int, 0>{});
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    default: return f(std::integral_constant<int, 5>{});
    }
}

} // namespace convt
