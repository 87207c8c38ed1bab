// Shape / attribute resolver: every rule fusedconv_create enforces.
// Host only; no HIP dependency.
//
// Rules follow the FusedConv manifest.json "derive" block (spatial-dim
// extraction, attribute length and value checks, SAME/VALID padding, expected
// output dims, group/bias/residual/activation checks) and the FusedConv
// README "Attributes" table.  Readings where the pages are silent:
//   * an output dim < 1 or a zero-sized input is rejected (OUTPUT_SHAPE);
//   * LeakyRelu / HardSigmoid / Clip parameters are mandatory (the README's
//     "exactly ... is required" wins over the derive defaults, which then
//     only matter for the optional-parameter activations);
//   * parameter-free activations ignore activation_params of any length.
#include <string.h>

#include <string>

#include "internal.h"

namespace fc {
namespace {

const char* const kActNames[] = {
    "Relu", "LeakyRelu", "Sigmoid", "Tanh", "HardSigmoid", "HardSwish", "Clip",
    "QuickGelu", "Elu", "Gelu", "FastGelu", "Softplus", "ThresholdedRelu", "Erf"};

int fail(std::string& err, int code, const std::string& msg) {
  err = msg;
  return code;
}

// Output size and effective begin pad of one axis.  Manifest derive
// samePad{Depth,Height,Width}, samePad{Front,Top,Left}, effectivePad*,
// expectedOutput*.  mode: 0 NOTSET, 1 SAME_UPPER, 2 SAME_LOWER, 3 VALID.
void axis_out(int64_t in, int64_t k, int64_t s, int64_t d, int mode, int64_t pb, int64_t pe,
              int64_t& out, int64_t& pad_begin) {
  if (mode == 1 || mode == 2) {
    out = (in + s - 1) / s;
    int64_t need = (out - 1) * s + (k - 1) * d + 1 - in;
    if (need < 0) need = 0;
    pad_begin = (mode == 1) ? need / 2 : need - need / 2;
    return;
  }
  if (mode == 3) pb = pe = 0;
  int64_t room = in + pb + pe - ((k - 1) * d + 1);
  // floor(room / s) + 1 with floor toward -inf for negative room
  out = (room >= 0) ? room / s + 1 : -((-room + s - 1) / s) + 1;
  pad_begin = pb;
}

}  // namespace

int resolve(const fusedconv_desc& d, Geometry& g, std::string& err) {
  memset(&g, 0, sizeof(g));
  ConvParams& cp = g.cp;
  if (d.dtype != FUSEDCONV_F32 && d.dtype != FUSEDCONV_F16)
    return fail(err, FUSEDCONV_ERR_DTYPE, "dtype must be FUSEDCONV_F32 or FUSEDCONV_F16");
  g.dtype = d.dtype;
  if (!d.x.present || !d.w.present)
    return fail(err, FUSEDCONV_ERR_NULL_ARG, "x and w are required inputs");

  // ranks: X, W and Y share one rank of 3..5 (manifest derive spatialRank,
  // conv1dRanksOk / nchwRanksOk / conv3dRanksOk)
  if (d.x.rank < 3 || d.x.rank > 5)
    return fail(err, FUSEDCONV_ERR_RANK, "x rank must be 3, 4 or 5 (1 to 3 spatial dims)");
  if (d.w.rank != d.x.rank) return fail(err, FUSEDCONV_ERR_RANK, "w rank must equal x rank");
  const int nsp = d.x.rank - 2;
  g.nsp = nsp;
  for (int i = 0; i < d.x.rank; ++i) {
    if (d.x.dims[i] < 0 || d.w.dims[i] < 0)
      return fail(err, FUSEDCONV_ERR_RANK, "negative dimension in x or w");
  }
  for (int i = 2; i < d.w.rank; ++i) {
    if (d.w.dims[i] < 1)
      return fail(err, FUSEDCONV_ERR_ATTR_VALUE, "kernel extents must be >= 1");
  }

  // attribute lengths (derive kernelShapeLengthOk ... padsLengthOk)
  if ((d.kernel_shape && d.n_kernel_shape != nsp) || (d.strides && d.n_strides != nsp) ||
      (d.dilations && d.n_dilations != nsp) || (d.pads && d.n_pads != 2 * nsp))
    return fail(err, FUSEDCONV_ERR_ATTR_LENGTH,
                "kernel_shape/strides/dilations need one entry per spatial axis, pads two");
  if (d.kernel_shape) {
    for (int i = 0; i < nsp; ++i)
      if (d.kernel_shape[i] != d.w.dims[2 + i])
        return fail(err, FUSEDCONV_ERR_KERNEL_SHAPE, "kernel_shape does not match w");
  }
  int64_t s[3], dl[3], pb[3], pe[3];
  for (int i = 0; i < nsp; ++i) {
    s[i] = d.strides ? d.strides[i] : 1;
    dl[i] = d.dilations ? d.dilations[i] : 1;
    pb[i] = d.pads ? d.pads[i] : 0;
    pe[i] = d.pads ? d.pads[nsp + i] : 0;
    if (s[i] < 1) return fail(err, FUSEDCONV_ERR_ATTR_VALUE, "strides must be >= 1");
    if (dl[i] < 1) return fail(err, FUSEDCONV_ERR_ATTR_VALUE, "dilations must be >= 1");
    if (pb[i] < 0 || pe[i] < 0) return fail(err, FUSEDCONV_ERR_ATTR_VALUE, "pads must be >= 0");
  }
  int mode = 0;
  if (d.auto_pad) {
    if (!strcmp(d.auto_pad, "NOTSET")) mode = 0;
    else if (!strcmp(d.auto_pad, "SAME_UPPER")) mode = 1;
    else if (!strcmp(d.auto_pad, "SAME_LOWER")) mode = 2;
    else if (!strcmp(d.auto_pad, "VALID")) mode = 3;
    else return fail(err, FUSEDCONV_ERR_ATTR_VALUE, "auto_pad must be NOTSET, SAME_UPPER, "
                     "SAME_LOWER or VALID");
  }
  if (mode != 0 && d.pads)
    return fail(err, FUSEDCONV_ERR_PADS_WITH_AUTO_PAD, "pads cannot be combined with auto_pad");

  // channels and groups (derive groupOk)
  const int64_t n = d.x.dims[0], C = d.x.dims[1], M = d.w.dims[0], wc = d.w.dims[1];
  if (d.group < 1) return fail(err, FUSEDCONV_ERR_GROUP, "group must be >= 1");
  if (M % d.group != 0 || wc * d.group != C)
    return fail(err, FUSEDCONV_ERR_GROUP, "need M % group == 0 and w.shape[1] * group == C");
  if (n == 0 || C == 0 || M == 0)
    return fail(err, FUSEDCONV_ERR_OUTPUT_SHAPE, "zero-sized batch or channel dimension");

  // spatial dims and output size (derive expectedOutput*)
  int64_t in3[3] = {1, 1, 1}, k3[3] = {1, 1, 1}, s3[3] = {1, 1, 1}, d3[3] = {1, 1, 1},
          p3[3] = {0, 0, 0}, o3[3] = {1, 1, 1};
  for (int i = 0; i < nsp; ++i) {
    const int j = 3 - nsp + i;
    in3[j] = d.x.dims[2 + i];
    k3[j] = d.w.dims[2 + i];
    s3[j] = s[i];
    d3[j] = dl[i];
    if (in3[j] == 0)
      return fail(err, FUSEDCONV_ERR_OUTPUT_SHAPE, "zero-sized spatial dimension");
    axis_out(in3[j], k3[j], s3[j], d3[j], mode, pb[i], pe[i], o3[j], p3[j]);
    if (o3[j] < 1)
      return fail(err, FUSEDCONV_ERR_OUTPUT_SHAPE,
                  "output size < 1: the dilated kernel is larger than the padded input");
  }
  g.y_rank = d.x.rank;
  g.y_dims[0] = n;
  g.y_dims[1] = M;
  for (int i = 0; i < nsp; ++i) g.y_dims[2 + i] = o3[3 - nsp + i];

  // bias: rank 1, length M (derive biasOk)
  if (d.bias.present && (d.bias.rank != 1 || d.bias.dims[0] != M))
    return fail(err, FUSEDCONV_ERR_BIAS_SHAPE, "bias must be rank 1 with M entries");

  // activation name and parameter count (derive activationOk, activationParamsOk)
  int act = ACT_NONE;
  if (d.activation) {
    act = -1;
    for (int i = 0; i < ACT_COUNT - 1; ++i)
      if (!strcmp(d.activation, kActNames[i])) act = i + 1;
    if (act < 0)
      return fail(err, FUSEDCONV_ERR_ACTIVATION, std::string("unknown activation '") +
                  d.activation + "'");
  }
  const int np = d.activation_params ? d.n_activation_params : -1;  // -1 = absent
  if (d.activation_params && d.n_activation_params < 0)
    return fail(err, FUSEDCONV_ERR_ACTIVATION_PARAMS, "negative activation_params count");
  if (act == ACT_LEAKYRELU && np != 1)
    return fail(err, FUSEDCONV_ERR_ACTIVATION_PARAMS, "LeakyRelu needs exactly [alpha]");
  if ((act == ACT_HARDSIGMOID || act == ACT_CLIP) && np != 2)
    return fail(err, FUSEDCONV_ERR_ACTIVATION_PARAMS,
                "HardSigmoid needs exactly [alpha, beta] and Clip exactly [min, max]");
  if ((act == ACT_QUICKGELU || act == ACT_ELU || act == ACT_THRESHOLDEDRELU ||
       act == ACT_GELU) && np > 1)
    return fail(err, FUSEDCONV_ERR_ACTIVATION_PARAMS,
                "QuickGelu, Elu, ThresholdedRelu and Gelu take at most one parameter");
  // derive actAlpha / actBeta
  float alpha = 0.0f, beta = 0.0f;
  if (np >= 1) alpha = d.activation_params[0];
  else if (act == ACT_HARDSIGMOID) alpha = 0.2f;
  else if (act == ACT_LEAKYRELU) alpha = 0.01f;
  else if (act == ACT_QUICKGELU) alpha = 1.702f;
  else if (act == ACT_ELU || act == ACT_THRESHOLDEDRELU) alpha = 1.0f;
  if (np >= 2) beta = d.activation_params[1];
  else if (act == ACT_HARDSIGMOID) beta = 0.5f;
  // Gelu with a nonzero approximate flag is the tanh form, which is FastGelu's
  // formula exactly; routing it there keeps Gelu's kernels free of a per-output
  // test of the flag
  if (act == ACT_GELU && alpha != 0.0f) {
    act = ACT_FASTGELU;
    alpha = 0.0f;
  }

  // residual: exactly Y's shape (derive zOk)
  if (d.z.present) {
    bool same = d.z.rank == g.y_rank;
    for (int i = 0; same && i < g.y_rank; ++i) same = d.z.dims[i] == g.y_dims[i];
    if (!same) return fail(err, FUSEDCONV_ERR_Z_SHAPE, "z must have exactly the shape of y");
  }

  // index limits of the kernels: per-image tensors and GEMM extents in int32
  const int64_t in_sz = in3[0] * in3[1] * in3[2], out_sz = o3[0] * o3[1] * o3[2];
  const int64_t taps = k3[0] * k3[1] * k3[2];
  const int64_t lim = (int64_t)1 << 31;
  if (C * in_sz >= lim || M * out_sz >= lim || wc * taps >= lim || M * wc * taps >= lim ||
      n * out_sz >= lim || n >= lim || in3[0] >= lim || in3[1] >= lim || in3[2] >= lim ||
      s3[0] * o3[0] >= lim || s3[1] * o3[1] >= lim || s3[2] * o3[2] >= lim ||
      d3[0] * k3[0] >= lim || d3[1] * k3[1] >= lim || d3[2] * k3[2] >= lim ||
      p3[0] >= lim || p3[1] >= lim || p3[2] >= lim)
    return fail(err, FUSEDCONV_ERR_TOO_LARGE,
                "tensor exceeds the int32 per-image / GEMM-extent index limits");

  cp.n = n;
  cp.C = (int32_t)C;
  cp.M = (int32_t)M;
  cp.G = (int32_t)d.group;
  cp.Cg = (int32_t)wc;
  cp.Mg = (int32_t)(M / d.group);
  cp.D = (int32_t)in3[0]; cp.H = (int32_t)in3[1]; cp.W = (int32_t)in3[2];
  cp.OD = (int32_t)o3[0]; cp.OH = (int32_t)o3[1]; cp.OW = (int32_t)o3[2];
  cp.KD = (int32_t)k3[0]; cp.KH = (int32_t)k3[1]; cp.KW = (int32_t)k3[2];
  cp.sd = (int32_t)s3[0]; cp.sh = (int32_t)s3[1]; cp.sw = (int32_t)s3[2];
  cp.dd = (int32_t)d3[0]; cp.dh = (int32_t)d3[1]; cp.dw = (int32_t)d3[2];
  cp.pd = (int32_t)p3[0]; cp.ph = (int32_t)p3[1]; cp.pw = (int32_t)p3[2];
  cp.taps = (int32_t)taps;
  cp.K = (int32_t)(wc * taps);
  cp.in_sz = in_sz;
  cp.out_sz = out_sz;
  cp.P = n * out_sz;
  cp.act = act;
  cp.alpha = alpha;
  cp.beta = beta;
  cp.has_bias = d.bias.present ? 1 : 0;
  cp.has_z = d.z.present ? 1 : 0;
  return FUSEDCONV_OK;
}

// Transposed convolution: the adjoint of the cross-correlation above (X is
// scattered through W into Y).  Output size per axis s*(in - 1) +
// output_padding + (k - 1)*d + 1 - pad_begin - pad_end.  Everything the
// forward rules check is checked on the forward problem that maps Y back to
// X with the same W (read as a [C, M/group, k...] conv weight): it must be
// valid and give X's extent, which holds for 0 <= output_padding < stride.
// auto_pad other than NOTSET and kernel_shape other than W's are refused.
int resolve_transposed(const fusedconv_desc& d, const int64_t* op, int32_t nop, Geometry& g,
                       std::string& err) {
  memset(&g, 0, sizeof(g));
  if (d.auto_pad && strcmp(d.auto_pad, "NOTSET") != 0)
    return fail(err, FUSEDCONV_ERR_ATTR_VALUE, "transposed: only auto_pad NOTSET is supported");
  if (!d.x.present || !d.w.present)
    return fail(err, FUSEDCONV_ERR_NULL_ARG, "x and w are required inputs");
  if (d.x.rank < 3 || d.x.rank > 5 || d.w.rank != d.x.rank)
    return fail(err, FUSEDCONV_ERR_RANK, "x and w ranks must be equal and 3, 4 or 5");
  const int nsp = d.x.rank - 2;
  if ((op && nop != nsp) || (!op && nop != 0))
    return fail(err, FUSEDCONV_ERR_ATTR_LENGTH, "output_padding needs one entry per spatial axis");
  if ((d.strides && d.n_strides != nsp) || (d.dilations && d.n_dilations != nsp) ||
      (d.pads && d.n_pads != 2 * nsp) || (d.kernel_shape && d.n_kernel_shape != nsp))
    return fail(err, FUSEDCONV_ERR_ATTR_LENGTH,
                "kernel_shape/strides/dilations need one entry per spatial axis, pads two");
  const int64_t n = d.x.dims[0], C = d.x.dims[1], wc = d.w.dims[0], mg = d.w.dims[1];
  if (d.group < 1) return fail(err, FUSEDCONV_ERR_GROUP, "group must be >= 1");
  if (wc != C || C % d.group != 0)
    return fail(err, FUSEDCONV_ERR_GROUP, "transposed: need w.shape[0] == C and C % group == 0");
  const int64_t M = mg * d.group;
  int64_t out[3];
  for (int i = 0; i < nsp; ++i) {
    const int64_t s = d.strides ? d.strides[i] : 1, dl = d.dilations ? d.dilations[i] : 1;
    const int64_t pb = d.pads ? d.pads[i] : 0, pe = d.pads ? d.pads[nsp + i] : 0;
    const int64_t o = op ? op[i] : 0, k = d.w.dims[2 + i];
    if (s < 1 || dl < 1 || pb < 0 || pe < 0 || k < 1 || d.x.dims[2 + i] < 1)
      return fail(err, FUSEDCONV_ERR_ATTR_VALUE,
                  "strides, dilations, kernel and input extents >= 1, pads >= 0");
    if (o < 0 || o >= s)
      return fail(err, FUSEDCONV_ERR_ATTR_VALUE, "output_padding must be in [0, stride)");
    out[i] = s * (d.x.dims[2 + i] - 1) + o + (k - 1) * dl + 1 - pb - pe;
    if (out[i] < 1) return fail(err, FUSEDCONV_ERR_OUTPUT_SHAPE, "transposed output size < 1");
  }
  // the forward problem Y -> X, without bias and residual (their shapes are
  // checked below), with the activation (its name and parameters)
  fusedconv_desc f = d;
  f.x.rank = d.x.rank;
  f.x.dims[0] = n;
  f.x.dims[1] = M;
  for (int i = 0; i < nsp; ++i) f.x.dims[2 + i] = out[i];
  f.bias.present = 0;
  f.z.present = 0;
  Geometry gf;
  int rc = resolve(f, gf, err);
  if (rc != FUSEDCONV_OK) return rc;
  for (int i = 0; i < nsp; ++i)
    if (gf.y_dims[2 + i] != d.x.dims[2 + i])
      return fail(err, FUSEDCONV_ERR_OUTPUT_SHAPE, "transposed: inconsistent output size");
  if (d.bias.present && (d.bias.rank != 1 || d.bias.dims[0] != M))
    return fail(err, FUSEDCONV_ERR_BIAS_SHAPE, "bias must be rank 1 with M entries");
  g.dtype = gf.dtype;
  g.nsp = nsp;
  g.y_rank = d.x.rank;
  g.y_dims[0] = n;
  g.y_dims[1] = M;
  for (int i = 0; i < nsp; ++i) g.y_dims[2 + i] = out[i];
  if (d.z.present) {
    bool same = d.z.rank == g.y_rank;
    for (int i = 0; same && i < g.y_rank; ++i) same = d.z.dims[i] == g.y_dims[i];
    if (!same) return fail(err, FUSEDCONV_ERR_Z_SHAPE, "z must have exactly the shape of y");
  }
  // geometry of the transposed problem: the forward one with X and Y swapped
  ConvParams& cp = g.cp;
  const ConvParams& fp = gf.cp;
  cp = fp;
  cp.C = (int32_t)C;
  cp.M = (int32_t)M;
  cp.Cg = (int32_t)(C / d.group);
  cp.Mg = (int32_t)mg;
  cp.D = fp.OD; cp.H = fp.OH; cp.W = fp.OW;
  cp.OD = fp.D; cp.OH = fp.H; cp.OW = fp.W;
  cp.K = cp.Cg * cp.taps;
  cp.in_sz = fp.out_sz;
  cp.out_sz = fp.in_sz;
  cp.P = n * cp.out_sz;
  cp.has_bias = d.bias.present ? 1 : 0;
  cp.has_z = d.z.present ? 1 : 0;
  cp.transposed = 1;
  return FUSEDCONV_OK;
}

}  // namespace fc
