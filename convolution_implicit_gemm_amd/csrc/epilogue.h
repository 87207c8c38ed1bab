// Fused epilogue: y = act(acc + B[m] + Z[i]) in fp32, one rounding to T at
// the store.  FusedConv README "Inputs" (B broadcast per output channel, Z
// added before the activation), "Attributes" (activation names and
// parameters); the manifest's grouped-kernel notes seed the f32 accumulator
// with the bias -- summation order is free, the result is one fp32 value.
//
// Activation formulas the pages name without writing out use their textbook
// / ONNX forms; the transcendental parts call HIP's device math library.
#pragma once

#include <hip/hip_runtime.h>

#include "conv_params.h"

namespace fc {

typedef _Float16 half_t;

template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }

// erfc-style tail of Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26: for u >= 0, erf(u) = 1 - P(t) exp(-u^2) with t = 1/(1 + p u)
// and a fifth-degree polynomial P; |error| <= 1.5e-7 for the formula, 6e-7
// evaluated in float32 (tests/test_activation_bounds_cpu.py).  Returns P(t) exp(-u^2),
// i.e. 1 - erf(u), so callers form 1 + erf(x) for x < 0 without cancellation.
__device__ __forceinline__ float erfc_as(float u) {
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * u);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  return poly * __expf(-u * u);
}
__device__ __forceinline__ float erf_fast(float x) {
  const float r = 1.0f - erfc_as(fabsf(x));
  return x < 0.0f ? -r : r;
}
// tanh(x) = 1 - 2 / (1 + e^(2x)); saturates correctly at both ends (e^(2x)
// -> inf gives 1, -> 0 gives -1); absolute error ~1e-7.
__device__ __forceinline__ float tanh_fast(float x) {
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __expf(2.0f * x));
}

// Activation A (compile-time) applied to v.  The exp-based ones use the
// hardware exp2 and reciprocal (__expf, v_rcp_f32) and the erf / tanh forms
// above: absolute errors below 1e-6, far inside the fp16 and fp32
// tolerances, at a fraction of the cost of the library routines.
template <int A>
__device__ __forceinline__ float act_t(float v, float a, float b) {
  if constexpr (A == ACT_NONE) return v;
  if constexpr (A == ACT_RELU) return v > 0.0f ? v : 0.0f;
  if constexpr (A == ACT_LEAKYRELU) return v >= 0.0f ? v : a * v;
  if constexpr (A == ACT_SIGMOID) return __builtin_amdgcn_rcpf(1.0f + __expf(-v));
  if constexpr (A == ACT_TANH) return tanh_fast(v);
  if constexpr (A == ACT_HARDSIGMOID) return fminf(fmaxf(a * v + b, 0.0f), 1.0f);
  if constexpr (A == ACT_HARDSWISH) return v * fminf(fmaxf(v * (1.0f / 6.0f) + 0.5f, 0.0f), 1.0f);
  if constexpr (A == ACT_CLIP) return fminf(fmaxf(v, a), b);
  if constexpr (A == ACT_QUICKGELU) return v * __builtin_amdgcn_rcpf(1.0f + __expf(-a * v));
  if constexpr (A == ACT_ELU) return v > 0.0f ? v : a * expm1f(v);
  if constexpr (A == ACT_GELU) {
    // 0.5 v (1 + erf(v / sqrt 2)); for v < 0, 1 + erf = erfc(|v| / sqrt 2).
    // A nonzero "approximate" flag never reaches here: the resolver sends it
    // to FastGelu, the same tanh form.
    const float c = erfc_as(fabsf(v) * 0.70710678118654752f);
    return 0.5f * v * (v < 0.0f ? c : 2.0f - c);
  }
  if constexpr (A == ACT_FASTGELU)
    return 0.5f * v * (1.0f + tanh_fast(0.79788456080286536f * (v + 0.044715f * v * v * v)));
  if constexpr (A == ACT_SOFTPLUS) return fmaxf(v, 0.0f) + log1pf(__expf(-fabsf(v)));
  if constexpr (A == ACT_THRESHOLDEDRELU) return v > a ? v : 0.0f;
  if constexpr (A == ACT_ERF) return erf_fast(v);
  return v;
}

template <int A> struct ActTag { static constexpr int value = A; };

// Call f(ActTag<act>{}) with the activation as a compile-time constant, so a
// loop inside f carries no per-element dispatch.
template <typename F>
__device__ __forceinline__ void with_act(int act, F&& f) {
  switch (act) {
    case ACT_RELU: f(ActTag<ACT_RELU>{}); break;
    case ACT_LEAKYRELU: f(ActTag<ACT_LEAKYRELU>{}); break;
    case ACT_SIGMOID: f(ActTag<ACT_SIGMOID>{}); break;
    case ACT_TANH: f(ActTag<ACT_TANH>{}); break;
    case ACT_HARDSIGMOID: f(ActTag<ACT_HARDSIGMOID>{}); break;
    case ACT_HARDSWISH: f(ActTag<ACT_HARDSWISH>{}); break;
    case ACT_CLIP: f(ActTag<ACT_CLIP>{}); break;
    case ACT_QUICKGELU: f(ActTag<ACT_QUICKGELU>{}); break;
    case ACT_ELU: f(ActTag<ACT_ELU>{}); break;
    case ACT_GELU: f(ActTag<ACT_GELU>{}); break;
    case ACT_FASTGELU: f(ActTag<ACT_FASTGELU>{}); break;
    case ACT_SOFTPLUS: f(ActTag<ACT_SOFTPLUS>{}); break;
    case ACT_THRESHOLDEDRELU: f(ActTag<ACT_THRESHOLDEDRELU>{}); break;
    case ACT_ERF: f(ActTag<ACT_ERF>{}); break;
    default: f(ActTag<ACT_NONE>{}); break;
  }
}

// Four values at once: one dispatch per 4 outputs.
typedef float act4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ act4_t act_apply4(int act, act4_t v, float a, float b) {
  act4_t r = v;
  with_act(act, [&](auto tag) {
    constexpr int A = decltype(tag)::value;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = act_t<A>(v[k], a, b);
  });
  return r;
}

// Compile-time form for kernels specialised per activation.
template <int A>
__device__ __forceinline__ act4_t act4(act4_t v, float a, float b) {
  act4_t r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = act_t<A>(v[k], a, b);
  return r;
}

// Runtime-dispatched form, for code where the activation is applied once per
// output outside any hot loop.
__device__ __forceinline__ float act_apply(int act, float v, float a, float b) {
  float r = v;
  with_act(act, [&](auto tag) { r = act_t<decltype(tag)::value>(v, a, b); });
  return r;
}

// Derivative of activation A at v, the backward of act_t: the textbook
// derivatives of the forms above; where a piecewise activation has no
// derivative, the branch its comparison selects (Relu 0 at 0, LeakyRelu
// alpha at 0, Clip 1 on [min, max], HardSigmoid alpha strictly inside
// (0, 1), HardSwish v/3 + 1/2 strictly inside (-3, 3), ThresholdedRelu 0 at
// alpha).
template <int A>
__device__ __forceinline__ float dact_t(float v, float a, float b) {
  if constexpr (A == ACT_NONE) return 1.0f;
  if constexpr (A == ACT_RELU) return v > 0.0f ? 1.0f : 0.0f;
  if constexpr (A == ACT_LEAKYRELU) return v > 0.0f ? 1.0f : a;
  if constexpr (A == ACT_SIGMOID) {
    const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-v));
    return s * (1.0f - s);
  }
  if constexpr (A == ACT_TANH) {
    const float t = tanh_fast(v);
    return 1.0f - t * t;
  }
  if constexpr (A == ACT_HARDSIGMOID) {
    const float u = a * v + b;
    return (u > 0.0f && u < 1.0f) ? a : 0.0f;
  }
  if constexpr (A == ACT_HARDSWISH) return v <= -3.0f ? 0.0f : (v >= 3.0f ? 1.0f : v * (1.0f / 3.0f) + 0.5f);
  if constexpr (A == ACT_CLIP) return (v >= a && v <= b) ? 1.0f : 0.0f;
  if constexpr (A == ACT_QUICKGELU) {
    const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-a * v));
    return s + a * v * s * (1.0f - s);
  }
  if constexpr (A == ACT_ELU) return v > 0.0f ? 1.0f : a * __expf(v);
  if constexpr (A == ACT_GELU) {
    // Phi(v) + v phi(v): Phi the normal CDF (erfc form as in act_t), phi its density
    const float c = erfc_as(fabsf(v) * 0.70710678118654752f);
    const float phi_cdf = v < 0.0f ? 0.5f * c : 1.0f - 0.5f * c;
    return phi_cdf + v * 0.39894228040143268f * __expf(-0.5f * v * v);
  }
  if constexpr (A == ACT_FASTGELU) {
    const float k = 0.79788456080286536f;
    const float t = tanh_fast(k * (v + 0.044715f * v * v * v));
    return 0.5f * (1.0f + t) + 0.5f * v * (1.0f - t * t) * k * (1.0f + 0.134145f * v * v);
  }
  if constexpr (A == ACT_SOFTPLUS) return __builtin_amdgcn_rcpf(1.0f + __expf(-v));
  if constexpr (A == ACT_THRESHOLDEDRELU) return v > a ? 1.0f : 0.0f;
  if constexpr (A == ACT_ERF) return 1.12837916709551257f * __expf(-v * v);
  return 1.0f;
}

// Runtime-dispatched derivative.
__device__ __forceinline__ float dact_apply(int act, float v, float a, float b) {
  float r = 1.0f;
  with_act(act, [&](auto tag) { r = dact_t<decltype(tag)::value>(v, a, b); });
  return r;
}

// Four derivatives at once: one dispatch per 4 outputs.
__device__ __forceinline__ act4_t dact_apply4(int act, act4_t v, float a, float b) {
  act4_t r = v;
  with_act(act, [&](auto tag) {
    constexpr int A = decltype(tag)::value;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = dact_t<A>(v[k], a, b);
  });
  return r;
}

// acc: the convolution sum for output (n, m, o) at flat Y index yi.  The
// backward-data form (cp.bwd) returns (acc + Z) * act'(P[yi]) instead.
template <typename T>
__device__ __forceinline__ T epilogue(float acc, int m, int64_t yi, const ConvParams& cp,
                                      const T* bias, const T* z, const T* pre) {
  if (cp.has_bias) acc += to_f32(bias[m]);
  if (cp.has_z) acc += to_f32(z[yi]);
  if (cp.bwd)
    return from_f32<T>(cp.act == ACT_NONE ? acc
                                          : acc * dact_apply(cp.act, to_f32(pre[yi]), cp.alpha, cp.beta));
  return from_f32<T>(act_apply(cp.act, acc, cp.alpha, cp.beta));
}

}  // namespace fc
