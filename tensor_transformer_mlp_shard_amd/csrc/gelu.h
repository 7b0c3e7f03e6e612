// GeLU with the exact (erf-based) definition, GeLU(z) = z Phi(z), and its
// derivative Phi(z) + z phi(z), evaluated in fp32 for the GEMM epilogues and
// the elementwise pass.
//
// erf comes from the rational approximation of Abramowitz and Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (after Hastings): for
// x >= 0, with t = 1 / (1 + p x),
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
// |error| <= 1.5e-7 (absolute), far below the bf16 / fp16 resolution of the
// outputs; erf is odd.  With x = |z| / sqrt(2), exp(-x^2) = exp(-z^2 / 2) is
// also the Gaussian density's exponential, so the derivative reuses it.  No
// branches: every lane of a wave evaluates the same instructions.
#pragma once

#include "common.h"

namespace tps {

struct GeluParts {
  float cdf;  // Phi(z) = (1 + erf(z / sqrt(2))) / 2
  float pdf;  // phi(z) = exp(-z^2 / 2) / sqrt(2 pi)
};

__device__ __forceinline__ GeluParts gelu_parts(float z) {
  constexpr float P = 0.3275911f;
  constexpr float A1 = 0.254829592f, A2 = -0.284496736f, A3 = 1.421413741f, A4 = -1.453152027f,
                  A5 = 1.061405429f;
  const float x = __builtin_fabsf(z) * 0.7071067811865475f;                 // |z| / sqrt(2)
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(P, x, 1.0f));
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * x * x);      // exp(-x^2)
  const float poly = t * __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, A5, A4), A3), A2), A1);
  const float erf_abs = __builtin_fmaf(-poly, e, 1.0f);
  const float erf_z = __builtin_copysignf(erf_abs, z);
  return {0.5f + 0.5f * erf_z, 0.3989422804014327f * e};
}

__device__ __forceinline__ float gelu_f(float z) { return z * gelu_parts(z).cdf; }

__device__ __forceinline__ float gelu_grad_f(float z) {
  const GeluParts g = gelu_parts(z);
  return __builtin_fmaf(z, g.pdf, g.cdf);
}

}  // namespace tps
