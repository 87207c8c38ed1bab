"""Pins for the backward oracle (oracle/backward.py), independent of its code.

The input and weight gradients are checked against PyTorch's float64
autograd of its own convolution, against the adjoint identities with the
forward oracle's C code (<conv(X, W), G> = <X, conv^T(G, W)> = <W, dW(X, G)>),
against an explicit Jacobian on tiny problems, and, through the whole layer
loss <act(conv(X, W) + B + Z), dY>, against central finite differences of
the forward oracle in every input (X, W, B, Z).  The activation derivatives
are checked against central differences of the forward oracle's activations,
against PyTorch's autograd of its activation routines (which also fixes the
one-sided values at the kinks) and against closed-form values.  A dropped
term, a flipped kernel, a wrong tap offset or a transposed operand fails at
least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import backward as bwd
from oracle import oracle
from workloads import random_tensors

ACTS = [("Relu", None), ("LeakyRelu", [0.2]), ("Sigmoid", None), ("Tanh", None),
        ("HardSigmoid", [0.3, 0.4]), ("HardSwish", None), ("Clip", [-0.5, 0.7]),
        ("QuickGelu", None), ("QuickGelu", [1.1]), ("Elu", [0.8]), ("Gelu", None),
        ("Gelu", [1.0]), ("FastGelu", None), ("Softplus", None), ("ThresholdedRelu", [0.3]),
        ("Erf", None)]
# points where the derivative jumps (kept away from in the difference checks)
KINKS = {"Relu": [0.0], "LeakyRelu": [0.0], "HardSigmoid": [-0.4 / 0.3, 0.6 / 0.3],
         "HardSwish": [-3.0, 3.0], "Clip": [-0.5, 0.7], "ThresholdedRelu": [0.3],
         "Elu": [0.0]}  # Elu: slope alpha on the left, 1 on the right


def setup_module(module):
    oracle.build(force=False)


@pytest.mark.parametrize("act,params", ACTS, ids=[a + str(p or "") for a, p in ACTS])
def test_activation_grad_is_the_derivative_of_the_forward_oracle(act, params):
    v = np.linspace(-5.0, 5.0, 2001)
    for k in KINKS.get(act, []):
        v = v[np.abs(v - k) > 1e-3]
    h = 1e-5
    fd = (oracle.activation(act, v + h, params) - oracle.activation(act, v - h, params)) / (2 * h)
    np.testing.assert_allclose(bwd.activation_grad(act, v, params), fd, rtol=0, atol=2e-8)


def _torch_act(act, params, t):
    if act == "Relu":
        return F.relu(t)
    if act == "LeakyRelu":
        return F.leaky_relu(t, params[0])
    if act == "Sigmoid":
        return torch.sigmoid(t)
    if act == "Tanh":
        return torch.tanh(t)
    if act == "HardSigmoid":   # torch's form is alpha = 1/6, beta = 1/2
        return F.hardsigmoid(t)
    if act == "HardSwish":
        return F.hardswish(t)
    if act == "Clip":
        return torch.clamp(t, params[0], params[1])
    if act == "QuickGelu":
        a = params[0] if params else 1.702
        return t * torch.sigmoid(a * t)
    if act == "Elu":
        return F.elu(t, params[0])
    if act == "Gelu":
        return F.gelu(t, approximate="tanh" if params and params[0] else "none")
    if act == "FastGelu":
        return F.gelu(t, approximate="tanh")
    if act == "Softplus":
        return F.softplus(t)
    if act == "ThresholdedRelu":
        return F.threshold(t, params[0], 0.0)
    if act == "Erf":
        return torch.erf(t)
    raise ValueError(act)


@pytest.mark.parametrize("act,params", ACTS, ids=[a + str(p or "") for a, p in ACTS])
def test_activation_grad_matches_torch_autograd(act, params):
    if act == "HardSigmoid":
        params = [1.0 / 6.0, 0.5]
    v = np.concatenate([np.linspace(-6.0, 6.0, 1201), KINKS.get(act, []),
                        [-3.0, 3.0] if act == "HardSigmoid" else []])
    t = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    (g,) = torch.autograd.grad(_torch_act(act, params, t).sum(), t)
    # (torch scales HardSigmoid's gradient by 1/6 rounded to float32)
    tol = 1e-7 if act == "HardSigmoid" else 1e-12
    np.testing.assert_allclose(bwd.activation_grad(act, v, params), g.numpy(), rtol=tol,
                               atol=1e-12)


def test_activation_grad_closed_forms():
    g = bwd.activation_grad
    assert g("QuickGelu", 0.0) == 0.5
    assert g("Sigmoid", 0.0) == 0.25
    assert g("Tanh", 0.0) == 1.0
    assert g("Gelu", 0.0) == 0.5 and g("FastGelu", 0.0) == 0.5
    assert g("Softplus", 0.0) == 0.5
    assert abs(g("Erf", 0.0) - 2.0 / math.sqrt(math.pi)) < 1e-15
    assert abs(g("Elu", -1.0, [0.8]) - 0.8 / math.e) < 1e-15
    assert g("HardSwish", 0.0) == 0.5 and g("HardSwish", 4.0) == 1.0 and g("HardSwish", -4.0) == 0
    assert g("HardSigmoid", 0.0, [0.3, 0.4]) == 0.3
    # QuickGelu'(v) = s + a v s (1 - s), s = sigmoid(a v); at v = 1, a = 1.702
    s = 1.0 / (1.0 + math.exp(-1.702))
    assert abs(g("QuickGelu", 1.0) - (s + 1.702 * s * (1 - s))) < 1e-15
    assert g(None, 3.0) == 1.0


def _resolved(x_shape, w_shape, strides, dilations, auto_pad, pads):
    nsp = len(x_shape) - 2
    out, pb = oracle.output_dims(x_shape[2:], w_shape[2:], strides, dilations, auto_pad, pads)
    pe = [(out[i] - 1) * strides[i] + (w_shape[2 + i] - 1) * dilations[i] + 1 - x_shape[2 + i] - pb[i]
          for i in range(nsp)]
    return out, pb, pe


def _case(rng, nsp):
    group = int(rng.choice([1, 2, 3]))
    cg, mg = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    ks = [int(v) for v in rng.integers(1, 4, size=nsp)]
    ins = [int(v) for v in rng.integers(3, 9, size=nsp)]
    s = [int(v) for v in rng.integers(1, 4, size=nsp)]
    d = [int(v) for v in rng.integers(1, 3, size=nsp)]
    mode = str(rng.choice(["NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID"]))
    pads = [int(v) for v in rng.integers(0, 3, size=2 * nsp)] if mode == "NOTSET" else None
    for i in range(nsp):
        ins[i] = max(ins[i], (ks[i] - 1) * d[i] + 1)
    x_shape = [int(rng.integers(1, 3)), cg * group] + ins
    w_shape = [mg * group, cg] + ks
    return x_shape, w_shape, dict(group=group, strides=s, dilations=d, auto_pad=mode, pads=pads)


@pytest.mark.parametrize("nsp", [1, 2, 3])
def test_backward_matches_torch_autograd(nsp):
    conv = {1: F.conv1d, 2: F.conv2d, 3: F.conv3d}[nsp]
    rng = np.random.default_rng(300 + nsp)
    for trial in range(14):
        x_shape, w_shape, a = _case(rng, nsp)
        out, pb, pe = _resolved(x_shape, w_shape, a["strides"], a["dilations"], a["auto_pad"],
                                a["pads"])
        y_shape = x_shape[:1] + w_shape[:1] + out
        x, w, _, g = random_tensors([30, nsp, trial], "f32", x_shape, w_shape, None, y_shape)
        xt = torch.tensor(x.astype(np.float64), requires_grad=True)
        wt = torch.tensor(w.astype(np.float64), requires_grad=True)
        padv = []
        for i in reversed(range(nsp)):
            padv += [pb[i], pe[i]]
        yt = conv(F.pad(xt, padv), wt, stride=a["strides"], dilation=a["dilations"],
                  groups=a["group"])
        assert list(yt.shape) == y_shape
        gx, gw = torch.autograd.grad(yt, (xt, wt), torch.tensor(g.astype(np.float64)))
        dx = bwd.conv_backward_data(g, w, x_shape, **a)
        dw = bwd.conv_backward_weight(x, g, w_shape, **a)
        np.testing.assert_allclose(dx, gx.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dw, gw.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("nsp", [1, 2, 3])
def test_adjoint_identities_with_the_c_forward(nsp):
    rng = np.random.default_rng(400 + nsp)
    for trial in range(10):
        x_shape, w_shape, a = _case(rng, nsp)
        y = oracle.fusedconv(*random_tensors([40, nsp, trial], "f32", x_shape, w_shape)[:2], **a)
        x, w, _, g = random_tensors([41, nsp, trial], "f32", x_shape, w_shape, None, list(y.shape))
        y = oracle.fusedconv(x, w, **a)
        lhs = float(np.sum(y * g))
        rhs_x = float(np.sum(x.astype(np.float64) * bwd.conv_backward_data(g, w, x_shape, **a)))
        rhs_w = float(np.sum(w.astype(np.float64) * bwd.conv_backward_weight(x, g, w_shape, **a)))
        assert abs(lhs - rhs_x) <= 1e-11 * max(1.0, abs(lhs)), (trial, lhs, rhs_x)
        assert abs(lhs - rhs_w) <= 1e-11 * max(1.0, abs(lhs)), (trial, lhs, rhs_w)


def test_explicit_jacobian_tiny():
    """Y is linear in X: column j of the Jacobian is conv(e_j, W); the input
    gradient is J^T G, the weight gradient likewise with unit weights."""
    x_shape, w_shape = [1, 4, 5, 6], [6, 2, 3, 2]
    a = dict(group=2, strides=[2, 1], dilations=[1, 2], pads=[1, 0, 2, 1])
    x, w, _, _ = random_tensors([50], "f32", x_shape, w_shape)
    y_shape = list(oracle.fusedconv(x, w, **a).shape)
    g = np.random.default_rng(51).standard_normal(y_shape)
    dx = np.zeros(x.size)
    for j in range(x.size):
        e = np.zeros(x.size)
        e[j] = 1.0
        dx[j] = np.sum(oracle.fusedconv(e.reshape(x_shape), w, **a) * g)
    dw = np.zeros(w.size)
    for j in range(w.size):
        e = np.zeros(w.size)
        e[j] = 1.0
        dw[j] = np.sum(oracle.fusedconv(x, e.reshape(w_shape), **a) * g)
    np.testing.assert_allclose(bwd.conv_backward_data(g, w, x_shape, **a).ravel(), dx,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bwd.conv_backward_weight(x, g, w_shape, **a).ravel(), dw,
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act,params", [("QuickGelu", None), ("Gelu", None), ("Elu", [0.8]),
                                        ("Tanh", None), ("Softplus", None), (None, None)])
def test_layer_loss_finite_differences(act, params):
    """L = <act(conv(X, W) + B + Z), dY>.  With G = dY * act'(Pre):
    dL/dW = dW(X, G), dL/dX = conv^T(G, W), dL/dB = sum G, dL/dZ = G; each
    checked as a directional derivative against central differences of the
    forward oracle (C code, activation included)."""
    x_shape, w_shape = [2, 6, 7, 5], [4, 3, 3, 3]
    a = dict(group=2, strides=[1, 2], dilations=[1, 1], pads=[1, 1, 1, 0])
    x, w, b, _ = random_tensors([60], "f32", x_shape, w_shape, [4])
    y_shape = list(oracle.fusedconv(x, w, **a).shape)
    rng = np.random.default_rng(61)
    z = rng.standard_normal(y_shape)
    dy = rng.standard_normal(y_shape)
    x, w, b = x.astype(np.float64), w.astype(np.float64), b.astype(np.float64)

    def loss(x_, w_, b_, z_):
        return float(np.sum(oracle.fusedconv(x_, w_, b_, z_, activation=act,
                                             activation_params=params, **a) * dy))

    pre = oracle.fusedconv(x, w, b, z, **a)
    g = dy * bwd.activation_grad(act, pre, params)
    grads = dict(x=bwd.conv_backward_data(g, w, x_shape, **a),
                 w=bwd.conv_backward_weight(x, g, w_shape, **a),
                 b=bwd.conv_backward_bias(g), z=g)
    base = dict(x=x, w=w, b=b, z=z)
    h = 1e-6
    for name, gr in grads.items():
        v = rng.standard_normal(base[name].shape)
        plus, minus = dict(base), dict(base)
        plus[name] = base[name] + h * v
        minus[name] = base[name] - h * v
        fd = (loss(**{k + "_": t for k, t in plus.items()}) -
              loss(**{k + "_": t for k, t in minus.items()})) / (2 * h)
        an = float(np.sum(gr * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_fused_input_activation_and_residual():
    """dP = (conv^T(G, W) + R) * act_in'(P): with W = identity 1x1 and
    stride 1 the adjoint is G itself, so dP = (G + R) * act_in'(P)."""
    rng = np.random.default_rng(70)
    g = rng.standard_normal([2, 5, 4, 6])
    r = rng.standard_normal([2, 5, 4, 6])
    p = rng.standard_normal([2, 5, 4, 6]) * 2
    w = np.eye(5).reshape(5, 5, 1, 1)
    got = bwd.conv_backward_data(g, w, [2, 5, 4, 6], pre=p, residual=r,
                                 input_activation="QuickGelu")
    s = 1.0 / (1.0 + np.exp(-1.702 * p))
    np.testing.assert_allclose(got, (g + r) * (s + 1.702 * p * s * (1 - s)), rtol=1e-13, atol=1e-13)
