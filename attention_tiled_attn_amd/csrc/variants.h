// variants.h - score_mod and mask_mod variants of the attention forward, as
// compile-time functors (device code, gfx950).
//
// FlexAttention lets a user attach a function of (q_idx, k_idx) that modifies a
// score, and mask modifications that drop pairs (NextVector FlexAttention
// article, body; PyTorch FlexAttention FA4-backend post). The variants named on
// the pages are sliding window, document packing, ALiBi and soft-capping (Neuron
// FA4 explainer, "PyTorch Gets the Upgrade Too"; NextVector article, "What
// Happened?"). Here each is a functor chosen at compile time (score mods) or by a
// wave-uniform flag word (masks, evaluated only on partial tiles).
//
// All score functors return t = s' * log2(e), the modified score in base-2
// units, because the softmax exponential is evaluated as exp2 (the unit the
// pages name as the forward-pass wall: Zadouri tweet; Neuron FA4 explainer,
// "FlashAttention-4: Built for Blackwell").
//
// Each also has a per-stage form for the bf16 kernel: stage() prepares, per
// lane, what depends only on the lane's row, the stage's first key kk0 and
// the exponent base b; shifted() then gives u = t - b for the key kk0 + c (c
// a compile-time column), so that the base costs nothing per score.
#pragma once

#include <hip/hip_runtime.h>

#include "exp2_poly.h"
#include "variant_args.h"

// Soft-capping's exponential on the multiply-add units (exp2_poly.h) instead
// of the hardware unit: a build option, 0 by default (measured slower).
#ifndef FLEXATTN_EXP2_POLY_TANH
#define FLEXATTN_EXP2_POLY_TANH 0
#endif

namespace fa {

typedef __attribute__((address_space(3))) float lds_f32;
typedef const __attribute__((address_space(3))) float lds_cf32;

// ---------------------------------------------------------------- score_mod
// s: raw dot product q.k accumulated in fp32; q_idx/k_idx: positions.
template <int MOD>
struct ScoreMod;

// With no modification the scale is folded into the exponent: scores stay raw,
// the running max is taken on raw scores and scaled once (scale > 0), and
// exp2 takes fma(s, c1, -m) directly.
template <>
struct ScoreMod<kModNone> {
  static constexpr bool kFoldScale = true;
  struct Lane {};
  __device__ static Lane lane(const VariantArgs&, int /*h*/, int /*q*/) { return {}; }
  __device__ static float apply(float s, const VariantArgs&, const Lane&, int /*dk*/) { return s; }
  struct Stage { float nb; };
  __device__ static Stage stage(const VariantArgs&, const Lane&, int /*dk0*/, float base) { return {-base}; }
  __device__ static float shifted(float s, const VariantArgs& a, const Lane&, const Stage& st, int /*c*/) {
    return __builtin_fmaf(s, a.c1, st.nb);
  }
};

// ALiBi: s' = scale*q.k + slope[h] * (k_idx - q_idx). The per-lane part
// slope*log2e is prepared once; `dk` is k_idx - q_idx.
template <>
struct ScoreMod<kModAlibi> {
  static constexpr bool kFoldScale = false;
  struct Lane { float sl; };
  __device__ static Lane lane(const VariantArgs& a, int h, int /*q*/) {
    return {a.slopes[h] * kLog2e};
  }
  __device__ static float apply(float s, const VariantArgs& a, const Lane& L, int dk) {
    return __builtin_fmaf(s, a.c1, L.sl * static_cast<float>(dk));
  }
  // the bias is linear in the key: slope * (dk0 + c) - b = fma(slope, c, B)
  struct Stage { float B; };
  __device__ static Stage stage(const VariantArgs&, const Lane& L, int dk0, float base) {
    return {__builtin_fmaf(L.sl, static_cast<float>(dk0), -base)};
  }
  __device__ static float shifted(float s, const VariantArgs& a, const Lane& L, const Stage& st, int c) {
    return __builtin_fmaf(s, a.c1, __builtin_fmaf(L.sl, static_cast<float>(c), st.B));
  }
};

// Soft-capping: s' = cap * tanh(scale*q.k / cap), with
// tanh(x) = 1 - 2 / (exp(2x) + 1) evaluated through exp2 and a reciprocal;
// exp2 overflow to +inf gives tanh = 1 and underflow to 0 gives -1.
template <>
struct ScoreMod<kModSoftcap> {
  static constexpr bool kFoldScale = false;
  struct Lane {};
  __device__ static Lane lane(const VariantArgs&, int, int) { return {}; }
  __device__ static float apply(float s, const VariantArgs& a, const Lane&, int /*dk*/) {
    const float e = __builtin_amdgcn_exp2f(s * a.sc_in);
    const float th = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
    return th * a.sc_out;
  }
  // cap * tanh(x) - b = (cap - b) - 2 cap / (exp(2x) + 1): one fma after the rcp
  struct Stage { float cb; };
  __device__ static Stage stage(const VariantArgs& a, const Lane&, int /*dk0*/, float base) {
    return {a.sc_out - base};
  }
  __device__ static float shifted(float s, const VariantArgs& a, const Lane&, const Stage& st, int /*c*/) {
    const float e = FLEXATTN_EXP2_POLY_TANH ? exp2_poly4(s * a.sc_in) : __builtin_amdgcn_exp2f(s * a.sc_in);
    return __builtin_fmaf(__builtin_amdgcn_rcpf(e + 1.0f), -2.0f * a.sc_out, st.cb);
  }
};

// Relative position bias: s' = scale*q.k + table_h[clip(k_idx - q_idx, -R, R)].
// The kernels stage head h's table in LDS (stage_rel_table) and point `tab`
// at its distance-0 entry.
template <>
struct ScoreMod<kModRelBias> {
  static constexpr bool kFoldScale = false;
  struct Lane { lds_cf32* tab; };
  __device__ static Lane lane(const VariantArgs&, int, int) { return {nullptr}; }
  __device__ static float apply(float s, const VariantArgs& a, const Lane& L, int dk) {
    const int d = min(max(dk, -a.rel_max), a.rel_max);
    return __builtin_fmaf(L.tab[d], kLog2e, s * a.c1);
  }
  struct Stage { float nb; int dk0; };
  __device__ static Stage stage(const VariantArgs&, const Lane&, int dk0, float base) { return {-base, dk0}; }
  __device__ static float shifted(float s, const VariantArgs& a, const Lane& L, const Stage& st, int c) {
    const int d = min(max(st.dk0 + c, -a.rel_max), a.rel_max);
    return __builtin_fmaf(L.tab[d], kLog2e, __builtin_fmaf(s, a.c1, st.nb));
  }
};

// Copy head h's relative-bias table (2R + 1 floats) to `dst` in LDS; every
// thread of the workgroup takes part; the caller synchronises before use.
__device__ inline void stage_rel_table(const VariantArgs& a, int h, lds_f32* dst, int tid, int nthreads) {
  const int n = 2 * a.rel_max + 1;
  const float* src = a.rel_bias + static_cast<size_t>(h) * n;
  for (int i = tid; i < n; i += nthreads) dst[i] = src[i];
}

// ---------------------------------------------------------------- mask_mod
// The kernels evaluate the per-element predicate inline on partial tiles, on
// positions (query row + q_offset, key index): causal q >= k, relaxed to
// q >= k || k < prefix for prefix-LM; window q - k < W; document
// doc[q] == doc[k]; AND-composed by the flag word of the mask kind.

}  // namespace fa
