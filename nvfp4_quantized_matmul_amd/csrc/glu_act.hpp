// Gate activations of the gated MLP projection out = act(gate) * up
// (mlxcel issue "perf(metal): close native NVFP4 prefill gap", sections
// "Hypothesis" and "Activation-path follow-up": the scaled gate/up MLP with
// a GeGLU activation), evaluated in float32.
#pragma once

#include <hip/hip_runtime.h>

#include "nvfp4.h"

namespace nvfp4dev {

// 1 / (1 + e^-t) from the hardware base-2 exponential and reciprocal (each
// about one ulp): e^-t = 2^(-t log2 e).  Large positive t gives 1, large
// negative t an infinite denominator and so 0; NaN stays NaN.
__device__ __forceinline__ float sigmoid(float t) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * t));
}

// GELU's tanh approximation (Hendrycks and Gimpel):
// z/2 (1 + tanh(u)) with u = sqrt(2/pi) (z + 0.044715 z^3), which equals
// z * sigmoid(2u).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float two_u = 1.5957691216057308f * z * __builtin_fmaf(0.044715f * z, z, 1.0f);
  return z * sigmoid(two_u);
}

// GELU, exact form z * Phi(z) with Phi(z) = erfc(-z / sqrt 2) / 2 (the
// device math library's erfc).
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * erfcf(-z * 0.7071067811865476f); }

// SiLU: z * sigmoid(z).
__device__ __forceinline__ float silu(float z) { return z * sigmoid(z); }

// The activation fixed at compile time, for kernels that apply it to many
// elements per lane: no per-element test of the activation type.
template <int kAct>
__device__ __forceinline__ float glu_act_t(float z) {
  if constexpr (kAct == NVFP4_ACT_GELU_TANH) return gelu_tanh(z);
  else if constexpr (kAct == NVFP4_ACT_GELU) return gelu_erf(z);
  else return silu(z);
}

__device__ __forceinline__ float glu_act(float z, int act) {
  if (act == NVFP4_ACT_GELU_TANH) return gelu_tanh(z);
  if (act == NVFP4_ACT_GELU) return gelu_erf(z);
  return silu(z);
}

}  // namespace nvfp4dev
