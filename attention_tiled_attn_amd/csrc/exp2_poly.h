// exp2_poly.h - 2^x on the multiply-add units, for a share of the softmax
// exponentials (device code, gfx950).
//
// FlashAttention-4 moves part of its exponentials from the hardware unit to
// a polynomial on the multiply-add units (Neuron FA4 explainer,
// "FlashAttention-4: Built for Blackwell", forward-pass fixes). Here: with
// n = floor(x) and f = x - n, 2^x = 2^n p(f), p(f) = 1 + f (a1 + f (a2 + f a3)),
// the coefficients a minimax fit of the relative error on [0, 1] by the
// Remez exchange algorithm (attention_tiled_attn_amd/exp2_poly.py, whose
// float32 rounding these are); largest relative error 8.6e-5. exp2_poly4
// adds a fourth coefficient (2.9e-6), for soft-capping's tanh, whose error
// the cap multiplies. p(0) = 1 and
// the clamp at -127 make a masked score (-inf) give exactly +0: the exponent
// add then cancels the exponent of p(0) = 1.0.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

constexpr float kExp2A1 = 0.69511676f;
constexpr float kExp2A2 = 0.227645f;
constexpr float kExp2A3 = 0.07706704f;

constexpr float kExp2B1 = 0.69304484f;
constexpr float kExp2B2 = 0.2412802f;
constexpr float kExp2B3 = 0.052242473f;
constexpr float kExp2B4 = 0.013426684f;

__device__ inline float exp2_poly(float x) {
  x = __builtin_fmaxf(x, -127.0f);
  const float n = __builtin_floorf(x);
  const float f = x - n;
  float t = __builtin_fmaf(kExp2A3, f, kExp2A2);
  t = __builtin_fmaf(t, f, kExp2A1);
  const float p = __builtin_fmaf(t, f, 1.0f);
  return __int_as_float(__float_as_int(p) + (static_cast<int>(n) << 23));
}

__device__ inline float exp2_poly4(float x) {
  x = __builtin_fmaxf(x, -127.0f);
  const float n = __builtin_floorf(x);
  const float f = x - n;
  float t = __builtin_fmaf(kExp2B4, f, kExp2B3);
  t = __builtin_fmaf(t, f, kExp2B2);
  t = __builtin_fmaf(t, f, kExp2B1);
  const float p = __builtin_fmaf(t, f, 1.0f);
  return __int_as_float(__float_as_int(p) + (static_cast<int>(n) << 23));
}

}  // namespace fa
