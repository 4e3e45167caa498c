// Device helpers shared by the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "svdq_internal.h"

namespace svdq {

// Output epilogue of call 2: GELU with the tanh approximation (Hendrycks and
// Gimpel, 2016), 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), for the MLP
// projections the W4A4 layer serves (mind-verse.de, "Effiziente Optimierung
// von Diffusionsmodellen durch Nunchaku 4-Bit-Quantisierung", section "Nunchaku
// Lite: Nahtlose Integration in Diffusers").  With e = exp(2u) the identity
// 0.5 x (1 + tanh u) = x - x / (e + 1) needs one exponential and one
// reciprocal, and gives x for e = inf and 0 for e = 0.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * x, x * x, x);
  const float e = __expf(2.0f * u);
  return x - __fdividef(x, e + 1.0f);
}

}  // namespace svdq
