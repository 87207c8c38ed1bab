/*
 * FusedConv oracle: a plain, slow, double-precision CPU loop nest.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file.  Its only callers are the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark.  It shares no code, header, table or
 * constant with the HIP library: it has its own padding and output-size
 * arithmetic, its own activation code and its own argument conventions.
 *
 * What it computes (FusedConv README, "Description", "Inputs", "Outputs";
 * FusedConv manifest.json, "derive" block):
 *
 *   for every batch n, output channel m and output spatial index o:
 *     g    = m / (M / group)                      channel group of m
 *     acc  = sum over input channels c' < C/group and every kernel tap t of
 *              X[n, g*(C/group) + c', o*s - pad_begin + t*d] * W[m, c', t]
 *            (a tap whose input coordinate is outside [0, in) on any axis
 *             contributes nothing: zero padding)
 *     pre  = acc + B[m] (if B is given) + Z[n, m, o] (if Z is given)
 *     Y    = act(pre)
 *
 * The kernel is not flipped (cross-correlation); this is the coordinate rule
 * ih = oh*sH - pH + kh*dH of the ExecuTorch im2col-GEMM conv page (PR #20873
 * description) and of the tinygrad im2col program.  Everything is accumulated
 * in double over the exact input values (fp16 and fp32 inputs convert to
 * double without error).  Spatial arrays are given outermost-first
 * (D, H, W for rank 5; H, W for rank 4; W for rank 3).
 *
 * Activation formulas the pages name but do not write out (Sigmoid, Tanh,
 * HardSwish, Elu, Softplus, ThresholdedRelu, Erf, the Gelu forms) follow
 * their textbook / ONNX definitions.  Each is pinned in the tests against a
 * library routine or a special value.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

/* auto_pad modes, FusedConv manifest.json "attributeConstraints.auto_pad". */
enum { OR_PAD_NOTSET = 0, OR_PAD_SAME_UPPER = 1, OR_PAD_SAME_LOWER = 2, OR_PAD_VALID = 3 };

/* activation ids: position in the manifest's "attributeConstraints.activation"
 * list, plus 1; 0 means no activation. */
enum {
  OR_ACT_NONE = 0, OR_ACT_RELU, OR_ACT_LEAKYRELU, OR_ACT_SIGMOID, OR_ACT_TANH,
  OR_ACT_HARDSIGMOID, OR_ACT_HARDSWISH, OR_ACT_CLIP, OR_ACT_QUICKGELU, OR_ACT_ELU,
  OR_ACT_GELU, OR_ACT_FASTGELU, OR_ACT_SOFTPLUS, OR_ACT_THRESHOLDEDRELU, OR_ACT_ERF
};

static int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
  return q;
}

/*
 * One spatial axis: output size and the effective begin pad.
 * FusedConv manifest.json, derive: samePad*, samePad{Front,Top,Left},
 * effectivePad*, expectedOutput*.  README "Attributes": SAME modes give
 * ceil(input / stride) outputs; VALID uses no padding; NOTSET uses pads.
 * Returns 0, or -1 when the output size is not positive.
 */
int oracle_axis(int64_t in, int64_t k, int64_t s, int64_t d, int mode,
                int64_t pad_b, int64_t pad_e, int64_t* out, int64_t* pad_begin) {
  int64_t o, pb;
  if (mode == OR_PAD_SAME_UPPER || mode == OR_PAD_SAME_LOWER) {
    int64_t total;
    o = (in + s - 1) / s;
    total = (o - 1) * s + (k - 1) * d + 1 - in;
    if (total < 0) total = 0;
    pb = (mode == OR_PAD_SAME_UPPER) ? total / 2 : total - total / 2;
  } else {
    int64_t span = (k - 1) * d + 1;
    int64_t padded = in + ((mode == OR_PAD_VALID) ? 0 : pad_b + pad_e);
    o = floor_div(padded - span, s) + 1;
    pb = (mode == OR_PAD_VALID) ? 0 : pad_b;
  }
  *out = o;
  *pad_begin = pb;
  return o >= 1 ? 0 : -1;
}

static double sigmoid(double v) {
  if (v >= 0) return 1.0 / (1.0 + exp(-v));
  double e = exp(v);
  return e / (1.0 + e);
}

/*
 * Activation applied to pre = conv + B + Z.  Names and parameters: FusedConv
 * README "Attributes" (activation, activation_params); parameter defaults:
 * FusedConv manifest.json derive actAlpha / actBeta.
 */
double oracle_activation(int act, double v, double alpha, double beta) {
  const double pi = 3.14159265358979323846;
  switch (act) {
    case OR_ACT_NONE: return v;
    case OR_ACT_RELU: return v > 0 ? v : 0.0;
    case OR_ACT_LEAKYRELU: return v >= 0 ? v : alpha * v;
    case OR_ACT_SIGMOID: return sigmoid(v);
    case OR_ACT_TANH: return tanh(v);
    case OR_ACT_HARDSIGMOID: {
      double t = alpha * v + beta;
      return t < 0 ? 0.0 : (t > 1 ? 1.0 : t);
    }
    case OR_ACT_HARDSWISH: {
      double t = v / 6.0 + 0.5;
      t = t < 0 ? 0.0 : (t > 1 ? 1.0 : t);
      return v * t;
    }
    case OR_ACT_CLIP: {
      double t = v < alpha ? alpha : v;
      return t > beta ? beta : t;
    }
    case OR_ACT_QUICKGELU: return v * sigmoid(alpha * v);
    case OR_ACT_ELU: return v > 0 ? v : alpha * (exp(v) - 1.0);
    case OR_ACT_GELU:
      if (alpha == 0.0) return 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
      /* nonzero "approximate" flag: the tanh form */
      return 0.5 * v * (1.0 + tanh(sqrt(2.0 / pi) * (v + 0.044715 * v * v * v)));
    case OR_ACT_FASTGELU:
      return 0.5 * v * (1.0 + tanh(sqrt(2.0 / pi) * (v + 0.044715 * v * v * v)));
    case OR_ACT_SOFTPLUS: return (v > 0 ? v : 0.0) + log1p(exp(-fabs(v)));
    case OR_ACT_THRESHOLDEDRELU: return v > alpha ? v : 0.0;
    case OR_ACT_ERF: return erf(v);
    default: return NAN;
  }
}

/* Resolved problem, built by oracle_setup from the raw attributes. */
typedef struct {
  int nsp;
  int64_t n, C, M, group, Cg, Mg;
  int64_t in[3], k[3], s[3], d[3], pb[3], out[3];
  int64_t in_sz, out_sz, k_sz;
  int act;
  double alpha, beta;
} or_problem;

/*
 * xs: X shape (nsp + 2 dims), ws: W shape, strides/dilations: nsp entries or
 * NULL (all ones), pads: 2*nsp entries in ONNX order [begins..., ends...] or
 * NULL (zeros).  Returns 0 or -1 (bad output size or channel split).
 */
static int oracle_setup(or_problem* p, int nsp, const int64_t* xs, const int64_t* ws,
                        int64_t group, const int64_t* strides, const int64_t* dilations,
                        int mode, const int64_t* pads, int act, const double* params,
                        int n_params) {
  int i;
  p->nsp = nsp;
  p->n = xs[0];
  p->C = xs[1];
  p->M = ws[0];
  p->group = group;
  if (group < 1 || p->C % group != 0 || p->M % group != 0) return -1;
  p->Cg = p->C / group;
  p->Mg = p->M / group;
  if (ws[1] != p->Cg) return -1;
  p->in_sz = p->out_sz = p->k_sz = 1;
  for (i = 0; i < nsp; ++i) {
    p->in[i] = xs[2 + i];
    p->k[i] = ws[2 + i];
    p->s[i] = strides ? strides[i] : 1;
    p->d[i] = dilations ? dilations[i] : 1;
    if (oracle_axis(p->in[i], p->k[i], p->s[i], p->d[i], mode, pads ? pads[i] : 0,
                    pads ? pads[nsp + i] : 0, &p->out[i], &p->pb[i]) != 0)
      return -1;
    p->in_sz *= p->in[i];
    p->out_sz *= p->out[i];
    p->k_sz *= p->k[i];
  }
  p->act = act;
  /* manifest derive actAlpha / actBeta: the given parameters, else defaults */
  p->alpha = n_params >= 1 ? params[0]
           : act == OR_ACT_HARDSIGMOID ? 0.2
           : act == OR_ACT_LEAKYRELU ? 0.01
           : act == OR_ACT_QUICKGELU ? 1.702
           : (act == OR_ACT_ELU || act == OR_ACT_THRESHOLDEDRELU) ? 1.0
           : 0.0;
  p->beta = n_params >= 2 ? params[1] : (act == OR_ACT_HARDSIGMOID ? 0.5 : 0.0);
  return 0;
}

/* The pre-activation sum for one output element (n, m, o[]). */
static double oracle_pre(const or_problem* p, const double* x, const double* w,
                         const double* b, const double* z, int64_t n, int64_t m,
                         const int64_t* o) {
  int64_t g = m / p->Mg;
  double acc = 0.0;
  int64_t c, t;
  for (c = 0; c < p->Cg; ++c) {
    const double* xc = x + (n * p->C + g * p->Cg + c) * p->in_sz;
    const double* wc = w + (m * p->Cg + c) * p->k_sz;
    for (t = 0; t < p->k_sz; ++t) {
      /* split the flat tap index into per-axis taps, innermost axis last */
      int64_t rem = t, off = 0, stride_in = 1;
      int inside = 1, i;
      for (i = p->nsp - 1; i >= 0; --i) {
        int64_t tap = rem % p->k[i];
        int64_t pos = o[i] * p->s[i] - p->pb[i] + tap * p->d[i];
        rem /= p->k[i];
        if (pos < 0 || pos >= p->in[i]) { inside = 0; break; }
        off += pos * stride_in;
        stride_in *= p->in[i];
      }
      if (inside) acc += xc[off] * wc[t];
    }
  }
  if (b) acc += b[m];
  if (z) {
    int64_t flat = 0;
    int i;
    for (i = 0; i < p->nsp; ++i) flat = flat * p->out[i] + o[i];
    acc += z[(n * p->M + m) * p->out_sz + flat];
  }
  return acc;
}

static void unflatten(const or_problem* p, int64_t flat, int64_t* o) {
  int i;
  for (i = p->nsp - 1; i >= 0; --i) {
    o[i] = flat % p->out[i];
    flat /= p->out[i];
  }
}

/*
 * Output spatial sizes and effective begin pads for all axes.
 * Returns 0, or -1 when some output size is not positive.
 */
int oracle_output_dims(int nsp, const int64_t* in, const int64_t* k, const int64_t* strides,
                       const int64_t* dilations, int mode, const int64_t* pads, int64_t* out,
                       int64_t* pad_begin) {
  int i, rc = 0;
  for (i = 0; i < nsp; ++i) {
    if (oracle_axis(in[i], k[i], strides ? strides[i] : 1, dilations ? dilations[i] : 1, mode,
                    pads ? pads[i] : 0, pads ? pads[nsp + i] : 0, &out[i], &pad_begin[i]) != 0)
      rc = -1;
  }
  return rc;
}

/*
 * Full output for batch images [n0, n1): y holds (n1 - n0) * M * out_sz
 * doubles, NC(D)(H)W order.  b and z may be NULL.  Parallel over (n, m)
 * with OpenMP when built with it; the arithmetic per element is serial.
 */
int oracle_fusedconv(int nsp, const int64_t* xs, const int64_t* ws, const double* x,
                     const double* w, const double* b, const double* z, int64_t group,
                     const int64_t* strides, const int64_t* dilations, int mode,
                     const int64_t* pads, int act, const double* params, int n_params,
                     int64_t n0, int64_t n1, double* y) {
  or_problem p;
  int64_t job, njobs;
  if (oracle_setup(&p, nsp, xs, ws, group, strides, dilations, mode, pads, act, params,
                   n_params) != 0)
    return -1;
  if (n0 < 0 || n1 > p.n || n0 > n1) return -1;
  njobs = (n1 - n0) * p.M;
#pragma omp parallel for schedule(dynamic)
  for (job = 0; job < njobs; ++job) {
    int64_t n = n0 + job / p.M, m = job % p.M, flat;
    int64_t o[3];
    double* yo = y + job * p.out_sz;
    for (flat = 0; flat < p.out_sz; ++flat) {
      unflatten(&p, flat, o);
      yo[flat] = oracle_activation(p.act, oracle_pre(&p, x, w, b, z, n, m, o), p.alpha, p.beta);
    }
  }
  return 0;
}

/*
 * Selected outputs only: idx[i] is a flat index into Y (NC(D)(H)W order).
 * Used where the whole output would take the oracle too long.
 */
int oracle_fusedconv_at(int nsp, const int64_t* xs, const int64_t* ws, const double* x,
                        const double* w, const double* b, const double* z, int64_t group,
                        const int64_t* strides, const int64_t* dilations, int mode,
                        const int64_t* pads, int act, const double* params, int n_params,
                        const int64_t* idx, int64_t npts, double* out) {
  or_problem p;
  int64_t i;
  if (oracle_setup(&p, nsp, xs, ws, group, strides, dilations, mode, pads, act, params,
                   n_params) != 0)
    return -1;
#pragma omp parallel for schedule(dynamic, 64)
  for (i = 0; i < npts; ++i) {
    int64_t flat = idx[i] % p.out_sz;
    int64_t nm = idx[i] / p.out_sz;
    int64_t o[3];
    unflatten(&p, flat, o);
    out[i] = oracle_activation(p.act, oracle_pre(&p, x, w, b, z, nm / p.M, nm % p.M, o),
                               p.alpha, p.beta);
  }
  return 0;
}

/* Activation over an array (for the activation pins). */
void oracle_activation_array(int act, const double* params, int n_params, const double* v,
                             int64_t count, double* out) {
  or_problem p;
  int64_t xs[3] = {1, 1, 1}, ws[3] = {1, 1, 1};
  int64_t i;
  oracle_setup(&p, 1, xs, ws, 1, NULL, NULL, OR_PAD_NOTSET, NULL, act, params, n_params);
  for (i = 0; i < count; ++i) out[i] = oracle_activation(act, v[i], p.alpha, p.beta);
}
