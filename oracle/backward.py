"""Backward oracle of the FusedConv layer, float64, numpy.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and
the CPU-baseline leg of the benchmark, never by the product package.  It
shares no code with the HIP library.

What it computes.  The forward layer is Y = act(conv(X, W) + B + Z) (FusedConv
README, "Inputs" and "Attributes"; conv = the cross-correlation of
fusedconv()).  Its training side (the tinygrad compare page,
tinygrad/codegen/opt/reduce.py: direct_conv_bwd_activation_program, a 3x3
convolution's input gradient as nine per-tap GEMMs with the QuickGelu
derivative fused, and col2im_program, the same gradient assembled from
per-tap columns with an optional fused activation derivative) needs, for a
gradient G of the loss with respect to the layer's pre-activation
Pre = conv(X, W) + B + Z:

  * the input gradient of the convolution, fused with the derivative of the
    activation that produced X (its pre-activation P, X = act_in(P)) and an
    optional residual gradient R of X's shape:
        dP = (conv^T(G, W) + R) * act_in'(P)                 conv_backward_data
    conv^T being the adjoint of the cross-correlation in X: every output
    position o of channel m sends G[n, m, o] * W[m, c, k] back to input
    position o*stride - pad_begin + k*dilation of channel g*(C/group) + c;
  * the weight gradient  dW[m, c, k] = sum over n, o of
        G[n, m, o] * X[n, g*(C/group) + c, o*stride - pad_begin + k*dilation]
    (zero outside X)                                          conv_backward_weight
  * the bias gradient    dB[m] = sum over n, o of G[n, m, o]  conv_backward_bias

and, for a loss gradient dY with respect to Y, G = dY * act'(Pre)
(activation_grad).  The pages name the activations without writing out
their derivatives (and the tinygrad page fuses only QuickGelu's); the
derivatives here are those of the textbook forms the forward oracle uses.
At the points where a piecewise activation has no derivative the reading
is the one-sided value of the branch that the comparison in the formula
below selects (Relu: 0 at 0; LeakyRelu: alpha at 0; Clip: 1 on the closed
interval [min, max]; HardSigmoid: alpha only strictly inside (0, 1);
HardSwish: x/3 + 1/2 only strictly inside (-3, 3), 0 at -3 and 1 at 3;
ThresholdedRelu: 0 at alpha) -- the values PyTorch's autograd gives there.

Each function is plain loops over groups and kernel taps, one numpy einsum
contraction per tap; padding and auto_pad are resolved by the forward
oracle's output_dims().
"""
from __future__ import annotations

import math

import numpy as np

from . import oracle

# forward-parameter defaults of the FusedConv README "Attributes" table
_DEFAULT_ALPHA = {"QuickGelu": 1.702, "Elu": 1.0, "ThresholdedRelu": 1.0}


def _params(name, params):
    p = list(params) if params is not None else []
    if name in _DEFAULT_ALPHA:
        return [p[0] if p else _DEFAULT_ALPHA[name]]
    return p


def _sigmoid(v):
    # sign-stable logistic
    e = np.exp(-np.abs(v))
    return np.where(v >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def activation_grad(name, v, params=None):
    """d act(v) / dv, elementwise, float64 (name None = identity)."""
    v = np.asarray(v, dtype=np.float64)
    if name is None:
        return np.ones_like(v)
    p = _params(name, params)
    if name == "Relu":
        return (v > 0).astype(np.float64)
    if name == "LeakyRelu":
        return np.where(v > 0, 1.0, p[0])
    if name == "Sigmoid":
        s = _sigmoid(v)
        return s * (1.0 - s)
    if name == "Tanh":
        return 1.0 - np.tanh(v) ** 2
    if name == "HardSigmoid":
        u = p[0] * v + p[1]
        return np.where((u > 0) & (u < 1), p[0], 0.0)
    if name == "HardSwish":
        return np.where(v <= -3.0, 0.0, np.where(v >= 3.0, 1.0, v / 3.0 + 0.5))
    if name == "Clip":
        return ((v >= p[0]) & (v <= p[1])).astype(np.float64)
    if name == "QuickGelu":
        s = _sigmoid(p[0] * v)
        return s + p[0] * v * s * (1.0 - s)
    if name == "Elu":
        return np.where(v > 0, 1.0, p[0] * np.exp(np.minimum(v, 0.0)))
    if name == "Gelu" and not (p and p[0] != 0):
        # 0.5 v (1 + erf(v / sqrt 2)): Phi(v) + v phi(v)
        erf = np.vectorize(math.erf)
        return 0.5 * (1.0 + erf(v / math.sqrt(2.0))) + v * np.exp(-0.5 * v * v) / math.sqrt(2 * math.pi)
    if name in ("FastGelu", "Gelu"):
        # 0.5 v (1 + tanh(c (v + 0.044715 v^3))), c = sqrt(2 / pi)
        c = math.sqrt(2.0 / math.pi)
        t = np.tanh(c * (v + 0.044715 * v ** 3))
        return 0.5 * (1.0 + t) + 0.5 * v * (1.0 - t * t) * c * (1.0 + 3 * 0.044715 * v * v)
    if name == "Softplus":
        return _sigmoid(v)
    if name == "ThresholdedRelu":
        return (v > p[0]).astype(np.float64)
    if name == "Erf":
        return 2.0 / math.sqrt(math.pi) * np.exp(-v * v)
    raise ValueError(name)


def _geometry(x_shape, w_shape, strides, dilations, auto_pad, pads):
    nsp = len(x_shape) - 2
    s = list(strides) if strides is not None else [1] * nsp
    d = list(dilations) if dilations is not None else [1] * nsp
    out = oracle.output_dims(list(x_shape[2:]), list(w_shape[2:]), s, d, auto_pad, pads)
    if out is None:
        raise ValueError("oracle: output size not positive")
    return nsp, s, d, out[0], out[1]


def conv_backward_data(dy, w, x_shape, *, group=1, strides=None, dilations=None,
                       auto_pad="NOTSET", pads=None, pre=None, residual=None,
                       input_activation=None, input_activation_params=None):
    """dP = (conv^T(dy, W) + R) * act_in'(P), float64, X's shape."""
    dy = np.asarray(dy, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    nsp, s, d, out, pb = _geometry(x_shape, w.shape, strides, dilations, auto_pad, pads)
    n, C = x_shape[:2]
    insp = list(x_shape[2:])
    ksp = list(w.shape[2:])
    M, Cg = w.shape[0], w.shape[1]
    Mg = M // group
    assert list(dy.shape) == [n, M] + out
    # positions i + pad_begin of the padded input, then the window of X
    full = [max((out[i] - 1) * s[i] + (ksp[i] - 1) * d[i] + 1, pb[i] + insp[i]) for i in range(nsp)]
    buf = np.zeros([n, C] + full, np.float64)
    for g in range(group):
        dyg = dy[:, g * Mg:(g + 1) * Mg]
        wg = w[g * Mg:(g + 1) * Mg]
        for tap in np.ndindex(*ksp):
            contrib = np.einsum("nm...,mc->nc...", dyg, wg[(slice(None), slice(None)) + tap],
                                optimize=True)
            sl = tuple(slice(tap[i] * d[i], tap[i] * d[i] + s[i] * (out[i] - 1) + 1, s[i])
                       for i in range(nsp))
            buf[(slice(None), slice(g * Cg, (g + 1) * Cg)) + sl] += contrib
    win = tuple(slice(pb[i], pb[i] + insp[i]) for i in range(nsp))
    dx = buf[(slice(None), slice(None)) + win].copy()
    if residual is not None:
        dx += np.asarray(residual, dtype=np.float64)
    if input_activation is not None:
        dx *= activation_grad(input_activation, pre, input_activation_params)
    return dx


def conv_backward_weight(x, dy, w_shape, *, group=1, strides=None, dilations=None,
                         auto_pad="NOTSET", pads=None):
    """dW [M, C/group, k...], float64."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    nsp, s, d, out, pb = _geometry(x.shape, w_shape, strides, dilations, auto_pad, pads)
    n, C = x.shape[:2]
    insp = list(x.shape[2:])
    ksp = list(w_shape[2:])
    M, Cg = w_shape[0], w_shape[1]
    Mg = M // group
    full = [max((out[i] - 1) * s[i] + (ksp[i] - 1) * d[i] + 1, pb[i] + insp[i]) for i in range(nsp)]
    xp = np.zeros([n, C] + full, np.float64)
    xp[(slice(None), slice(None)) + tuple(slice(pb[i], pb[i] + insp[i]) for i in range(nsp))] = x
    dw = np.zeros(list(w_shape), np.float64)
    for g in range(group):
        dyg = dy[:, g * Mg:(g + 1) * Mg]
        xg = xp[:, g * Cg:(g + 1) * Cg]
        for tap in np.ndindex(*ksp):
            sl = tuple(slice(tap[i] * d[i], tap[i] * d[i] + s[i] * (out[i] - 1) + 1, s[i])
                       for i in range(nsp))
            xs = xg[(slice(None), slice(None)) + sl]
            dw[(slice(g * Mg, (g + 1) * Mg), slice(None)) + tap] = np.einsum(
                "nmp,ncp->mc", dyg.reshape(n, Mg, -1), xs.reshape(n, Cg, -1), optimize=True)
    return dw


def conv_backward_bias(dy):
    """dB [M], float64."""
    dy = np.asarray(dy, dtype=np.float64)
    return dy.sum(axis=tuple(i for i in range(dy.ndim) if i != 1))
