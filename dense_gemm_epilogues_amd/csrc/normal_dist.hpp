// Standard normal distribution function Phi and density phi for the GELU epilogs, shared by
// the fused epilogue and the unfused elementwise kernels.
//
// Phi(t) = (1 + erf(t / sqrt 2)) / 2, with erf from the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions (1964), formula 7.1.26: for x >= 0,
// erf(x) = 1 - (a1 r + a2 r^2 + a3 r^3 + a4 r^4 + a5 r^5) e^(-x^2) + eps, r = 1 / (1 + p x),
// |eps| <= 1.5e-7.  With x = |t| / sqrt 2 the factor e^(-x^2) is e^(-t^2/2), the same
// exponential as the density, so Phi and phi together cost one hardware exp2, one hardware
// reciprocal and a degree-5 polynomial, without branches.  In fp32 the GELU built on it is
// within 1.3e-5 relative of the exact function wherever |gelu| > 1e-2 (and within 4.3e-7
// absolutely everywhere), below half an fp16 ulp.  t = +-inf gives Phi = 1 / 0; NaN stays NaN.
#pragma once
#include <hip/hip_runtime.h>

namespace ep {

// Phi(-|t|) = erfc(|t| / sqrt 2) / 2, and the density e^(-t^2/2) / sqrt(2 pi) in *pdf (the
// polynomial's coefficients are A&S's a1..a5 halved, which folds in the / 2).  The argument is
// carried as y = |t| sqrt(log2(e) / 2), so that e^(-t^2/2) = 2^(-y^2) and A&S's p x = p' y with
// p' = p / sqrt(log2 e): one multiplication fewer than with x = |t| / sqrt 2.
__device__ __forceinline__ float norm_tail_pdf(float t, float* pdf) {
  const float y = __builtin_fabsf(t) * 0.84932180028801904f;
  const float r = __builtin_amdgcn_rcpf(1.0f + 0.27273748087922250f * y);
  const float half_poly =
      r * (0.127414796f + r * (-0.142248368f + r * (0.7107068705f + r * (-0.7265760135f + r * 0.5307027145f))));
  const float e = __builtin_amdgcn_exp2f(-(y * y));  // e^(-t^2/2)
  *pdf = 0.39894228040143268f * e;                   // 1/sqrt(2 pi) e^(-t^2/2)
  return half_poly * e;
}

__device__ __forceinline__ float norm_cdf_pdf(float t, float* pdf) {
  const float q = norm_tail_pdf(t, pdf);
  return t >= 0.0f ? 1.0f - q : q;
}

// exact-form GELU t Phi(t) = max(t, 0) - |t| Phi(-|t|) (for t >= 0: t - t Phi(-t); for t < 0:
// t Phi(t)), and its derivative Phi(t) + t phi(t).  |t| enters the product clamped to 40:
// Phi(-|t|) is exactly 0 in fp32 well before that, and the clamp keeps t = +-inf from
// multiplying infinity by zero (GELU(-inf) = 0).  The max and the clamp are medians of three
// (one v_med3_f32 each, where fmaxf / fminf also quiet their inputs; the upper bound of the max
// is the largest finite float, which the compiler does not turn back into a max, and which
// rounds to +inf in fp16 and bf16, so GELU(+inf) is still +inf); a NaN t makes the Phi term
// NaN, so GELU(NaN) is NaN whatever the median returns for it.
__device__ __forceinline__ float gelu_f(float t) {
  float pdf;
  const float q = norm_tail_pdf(t, &pdf);
  const float pos = __builtin_amdgcn_fmed3f(t, 0.0f, 3.40282347e38f);
  const float mag = __builtin_amdgcn_fmed3f(__builtin_fabsf(t), 0.0f, 40.0f);
  return pos - mag * q;
}
__device__ __forceinline__ float gelu_grad_f(float t) {
  float pdf;
  const float cdf = norm_cdf_pdf(t, &pdf);
  return cdf + t * pdf;
}

}  // namespace ep
