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

__device__ __forceinline__ float act_apply(int act, float v, float a, float b) {
  switch (act) {
    case ACT_NONE: return v;
    case ACT_RELU: return v > 0.0f ? v : 0.0f;
    case ACT_LEAKYRELU: return v >= 0.0f ? v : a * v;
    case ACT_SIGMOID: return 1.0f / (1.0f + expf(-v));
    case ACT_TANH: return tanhf(v);
    case ACT_HARDSIGMOID: return fminf(fmaxf(a * v + b, 0.0f), 1.0f);
    case ACT_HARDSWISH: return v * fminf(fmaxf(v * (1.0f / 6.0f) + 0.5f, 0.0f), 1.0f);
    case ACT_CLIP: return fminf(fmaxf(v, a), b);
    case ACT_QUICKGELU: return v / (1.0f + expf(-a * v));
    case ACT_ELU: return v > 0.0f ? v : a * expm1f(v);
    case ACT_GELU:
      if (a == 0.0f) return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
      // nonzero "approximate" flag: tanh form
      return 0.5f * v * (1.0f + tanhf(0.79788456080286536f * (v + 0.044715f * v * v * v)));
    case ACT_FASTGELU:
      return 0.5f * v * (1.0f + tanhf(0.79788456080286536f * (v + 0.044715f * v * v * v)));
    case ACT_SOFTPLUS: return fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v)));
    case ACT_THRESHOLDEDRELU: return v > a ? v : 0.0f;
    case ACT_ERF: return erff(v);
    default: return v;
  }
}

// acc: the convolution sum for output (n, m, o) at flat Y index yi.
template <typename T>
__device__ __forceinline__ T epilogue(float acc, int m, int64_t yi, const ConvParams& cp,
                                      const T* bias, const T* z) {
  if (cp.has_bias) acc += to_f32(bias[m]);
  if (cp.has_z) acc += to_f32(z[yi]);
  return from_f32<T>(act_apply(cp.act, acc, cp.alpha, cp.beta));
}

}  // namespace fc
