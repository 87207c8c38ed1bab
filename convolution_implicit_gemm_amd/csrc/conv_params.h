// Resolved problem and plan, shared by the host resolver/planner and the
// device kernels.  Plain structs only: passed to kernels by value.
#pragma once

#include <stdint.h>

namespace fc {

// Activation ids, in the order of the FusedConv manifest.json activation list
// ("attributeConstraints.activation"), 0 = none.
enum Act : int32_t {
  ACT_NONE = 0, ACT_RELU, ACT_LEAKYRELU, ACT_SIGMOID, ACT_TANH, ACT_HARDSIGMOID,
  ACT_HARDSWISH, ACT_CLIP, ACT_QUICKGELU, ACT_ELU, ACT_GELU, ACT_FASTGELU, ACT_SOFTPLUS,
  ACT_THRESHOLDEDRELU, ACT_ERF, ACT_COUNT
};

// The convolution after attribute resolution.  Spatial axes are stored as
// (D, H, W) right-aligned: a 2-D problem has D = OD = KD = 1, a 1-D problem
// also H = OH = KH = 1 (the manifest's inputDepth / inputHeight defaults).
// Pads are the effective begin pads; end pads only shape the output size.
struct ConvParams {
  int64_t n;            // batch
  int32_t C, M, G;      // input channels, output channels, groups
  int32_t Cg, Mg;       // per group
  int32_t D, H, W;      // input spatial
  int32_t OD, OH, OW;   // output spatial
  int32_t KD, KH, KW;   // kernel spatial
  int32_t sd, sh, sw;   // strides
  int32_t dd, dh, dw;   // dilations
  int32_t pd, ph, pw;   // effective begin pads
  int32_t taps;         // KD*KH*KW
  int32_t K;            // Cg*taps: GEMM reduction length
  int64_t in_sz;        // D*H*W
  int64_t out_sz;       // OD*OH*OW
  int64_t P;            // n*out_sz: GEMM columns
  int32_t act;          // Act
  float alpha, beta;    // activation parameters after defaulting
  int32_t has_bias, has_z;
  // 1: transposed convolution (fusedconv_create_transposed).  Then C and Cg
  // count X's channels, M and Mg Y's, W is [C][M/G][k...], (D, H, W) is X's
  // extent and (OD, OH, OW) Y's, and the pads are Y's begin offsets.
  int32_t transposed;
  // 1: the input gradient of a convolution (fusedconv_create_backward_data).
  // X is then the gradient G of that convolution's output, Y the gradient of
  // the pre-activation P of its input, and the epilogue computes
  // Y = (acc + Z) * act'(P): Z the optional residual gradient, act the
  // activation that produced the convolution's input (no bias).
  int32_t bwd;
  // 1: the POINTWISE GEMM view of an explicit im2col column matrix, with pixel
  // tiles over the flattened (image, pixel) axis of n * in_sz entries (in_sz
  // the padded column row, out_sz the valid pixels of each image), so that
  // images smaller than a tile fill whole tiles.
  int32_t flat;
};

// True when the depth axis is trivial, i.e. the problem is really 1-D or 2-D:
// one input and one output plane, a one-tap kernel and no depth pad.  Only
// then does output plane 0 read input plane 0; a 3-D problem with D = KD = 1
// can still have several output planes (end pads, output_padding) or read
// the zero padding (a begin pad), which the 2-D-only kernels cannot express.
inline bool depth_trivial(const ConvParams& cp) {
  return cp.D == 1 && cp.KD == 1 && cp.OD == 1 && cp.pd == 0;
}

}  // namespace fc
