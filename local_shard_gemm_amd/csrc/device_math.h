// Element-wise device math shared by the GEMM epilogues (MFMA and skinny
// kernels), so that both paths produce the same H for the same input.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace shardmm {

// GeLU, tanh form: 0.5 x (1 + tanh(z)), z = sqrt(2/pi) (x + 0.044715 x^3),
// evaluated as x / (1 + exp(-2z)) -- the same function (1 + tanh(z) =
// 2 / (1 + exp(-2z))) without the float32 cancellation of 1 + tanh(z) for
// negative z. With z = x (c0 + c1 x^2), exp(-2z) = 2^(x (c0' + c1' x^2)),
// c0' = -2 log2(e) c0 and c1' = 0.044715 c0', folded in double precision:
// one multiply, one fma and one multiply before the hardware exp2, then a
// hardware reciprocal. Each step adds about one float32 ulp, far below the
// bfloat16 rounding of the stored H.
__device__ __forceinline__ float gelu_tanh_f32(float x) {
  constexpr double kLog2e = 1.4426950408889634, kSqrt2OverPi = 0.7978845608028654, kCubic = 0.044715;
  constexpr float c0 = static_cast<float>(-2.0 * kLog2e * kSqrt2OverPi);
  constexpr float c1 = static_cast<float>(-2.0 * kLog2e * kSqrt2OverPi * kCubic);
  const float e = __builtin_amdgcn_exp2f(x * __builtin_fmaf(c1, x * x, c0));
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// float -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> two bfloat16 packed low-first, round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950 (same results as bf16_rne for every non-NaN).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace shardmm
