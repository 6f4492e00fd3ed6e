// Fixed-operation fp32 functions of the router gates. Every operation is one
// correctly rounded IEEE fp32 operation (fused multiply-adds where written), in
// a fixed order, so the gate values and the routing decisions they drive are
// reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

#pragma clang fp contract(off)
// Fixed-operation fp32 exponential: Cody-Waite range reduction (Cody & Waite,
// "Software Manual for the Elementary Functions", 1980) with ln2 split in a
// 15-bit head and an fp32 tail, then the degree-7 Taylor polynomial of e^r in
// Horner form with fused multiply-adds, then scaling by 2^n built from the
// exponent bits. Inputs above 86 give +inf and below -86 give 0, so no result
// is subnormal. Every operation is a correctly rounded IEEE fp32 operation.
__device__ __forceinline__ float exp_c(float x) {
  if (x > 86.0f) return __builtin_inff();
  if (x < -86.0f) return 0.0f;
  const float log2e = 1.44269504088896341f;
  const float ln2_hi = 0.693145751953125f;
  const float ln2_lo = 1.42860682030941723e-6f;
  float n = __builtin_rintf(x * log2e);
  float r = __builtin_fmaf(-n, ln2_hi, x);
  r = __builtin_fmaf(-n, ln2_lo, r);
  float p = 1.98412698412698413e-4f;             // 1/7!
  p = __builtin_fmaf(p, r, 1.38888888888888889e-3f);  // 1/6!
  p = __builtin_fmaf(p, r, 8.33333333333333333e-3f);  // 1/5!
  p = __builtin_fmaf(p, r, 4.16666666666666667e-2f);  // 1/4!
  p = __builtin_fmaf(p, r, 1.66666666666666667e-1f);  // 1/3!
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  int ni = (int)n;
  float scale = __uint_as_float((uint32_t)(ni + 127) << 23);
  return p * scale;
}

__device__ __forceinline__ float sigmoid_c(float h) {
  float e = exp_c(-h);
  float den = 1.0f + e;
  return 1.0f / den;
}

// Fixed-operation log(1 + u) for u in [0, 1]: log(1 + u) = 2 artanh(z) with
// z = u / (2 + u) in [0, 1/3]; the artanh series through z^15 (first dropped
// term below 2e-9 relative) as z * P(z^2), P in Horner form with coefficients
// 2/(2i + 1).
__device__ __forceinline__ float log1p_c(float u) {
  const float z = u / (2.0f + u);
  const float z2 = z * z;
  float p = 0.133333333333333333f;
  p = __builtin_fmaf(p, z2, 0.153846153846153846f);
  p = __builtin_fmaf(p, z2, 0.181818181818181818f);
  p = __builtin_fmaf(p, z2, 0.222222222222222222f);
  p = __builtin_fmaf(p, z2, 0.285714285714285714f);
  p = __builtin_fmaf(p, z2, 0.4f);
  p = __builtin_fmaf(p, z2, 0.666666666666666667f);
  p = __builtin_fmaf(p, z2, 2.0f);
  return z * p;
}

// Square root of softplus ([WIKI], DeepSeek-V4's replacement of the sigmoid
// gate): softplus(h) = max(h, 0) + log(1 + e^-|h|), which cannot overflow, then
// the correctly rounded fp32 square root.
// softplus(h) = log(1 + e^h) as max(h, 0) + log1p_c(exp_c(-|h|)): never overflows.
__device__ __forceinline__ float softplus_c(float h) {
  const float u = exp_c(-__builtin_fabsf(h));
  return (h > 0.0f ? h : 0.0f) + log1p_c(u);
}

__device__ __forceinline__ float sqrt_softplus_c(float h) { return __builtin_sqrtf(softplus_c(h)); }
#pragma clang fp contract(on)

}  // namespace moe
