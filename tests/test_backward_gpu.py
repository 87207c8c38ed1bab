"""GPU parity of the backward entry points against the backward oracle.

Input gradient (fusedconv_backward_data): max|dP_gpu - dP_ref| <= tau *
max|dP_ref| with tau = 2e-2 for fp16 and 1e-4 for fp32 (fp32 accumulation,
one rounding of the output, as for the forward path).  Weight and bias
gradients (fusedconv_backward_weight, float32 outputs): tau = 1e-3 for fp16
inputs (exact fp16 products, fp32 sums in another order) and 1e-4 for fp32.
Every element of every output is compared; the full-size case is the CIFAR
ResNet 3x3 conv (512 x 128 x 16 x 16 -> 256 channels) whose forward is the
benchmark's headline workload.
"""
import sys

import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as fc
from convolution_implicit_gemm_amd import _binding as B
from oracle import backward as bwd
from oracle import oracle
from workloads import WORKLOADS, make_inputs, random_tensors

pytestmark = pytest.mark.gpu
TAU_X = {"f32": 1e-4, "f16": 2e-2}
TAU_W = {"f32": 1e-4, "f16": 1e-3}
ACTS = [(None, None), ("Relu", None), ("LeakyRelu", [0.1]), ("Sigmoid", None), ("Tanh", None),
        ("HardSigmoid", [0.2, 0.5]), ("HardSwish", None), ("Clip", [-0.5, 1.5]),
        ("QuickGelu", [1.702]), ("Elu", [0.8]), ("Gelu", None), ("Gelu", [1.0]),
        ("FastGelu", None), ("Softplus", None), ("ThresholdedRelu", [0.3]), ("Erf", None)]


def log(msg):
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    fc.load()
    oracle.build(force=False)


def f32params(p):
    return None if p is None else [float(np.float32(v)) for v in p]


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(got))
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def fwd_y_shape(xs, ws, attrs):
    a = {k: v for k, v in attrs.items() if k not in ("route", "split_k")}
    return B.Handle("f32", xs, ws, None, None, **a).y_shape


def run_data(dtype, xs, ws, attrs, seed, act=(None, None), residual=False, route="auto",
             split_k=0):
    ys = fwd_y_shape(xs, ws, attrs)
    x, w, _, g = random_tensors(seed, dtype, xs, ws, None, ys, dist="normal",
                                w_std=1.0 / np.sqrt(np.prod(ws[1:])))
    rng = np.random.default_rng(seed + [7])
    pre = (rng.standard_normal(xs) * 2).astype(np.float16 if dtype == "f16" else np.float32)
    r = rng.standard_normal(xs).astype(pre.dtype) if residual else None
    params = f32params(act[1])
    op = fc.ConvBackwardData(xs, ws, dtype, residual, act[0], params, route=route,
                             split_k=split_k, **attrs)
    log(f"CASE bwd-data {dtype} x={xs} w={ws} {attrs} act={act} res={residual} "
        f"route={op.handle.route} ({op.handle.kernel_name})")
    got = op(dev(g), dev(w), dev(pre) if act[0] else None, dev(r))
    torch.cuda.synchronize()
    ref = bwd.conv_backward_data(g, w, xs, pre=pre if act[0] else None, residual=r,
                                 input_activation=act[0], input_activation_params=params,
                                 **attrs)
    e = rel_err(got.cpu().numpy(), ref)
    assert e <= TAU_X[dtype], f"rel err {e:.3e}"
    return op.handle.route


def run_weight(dtype, xs, ws, attrs, seed, bias=True, route="auto"):
    ys = fwd_y_shape(xs, ws, attrs)
    x, w, _, g = random_tensors(seed, dtype, xs, ws, None, ys, dist="normal")
    op = fc.ConvBackwardWeight(xs, ws, dtype, bias, route=route, **attrs)
    log(f"CASE bwd-weight {dtype} x={xs} w={ws} {attrs} bias={bias} route={op.handle.route} "
        f"splits={op.handle.split_k}")
    out = op(dev(x), dev(g))
    dw, db = out if bias else (out, None)
    torch.cuda.synchronize()
    ref = bwd.conv_backward_weight(x, g, ws, **attrs)
    e = rel_err(dw.cpu().numpy(), ref)
    assert e <= TAU_W[dtype], f"dW rel err {e:.3e}"
    if bias:
        eb = rel_err(db.cpu().numpy(), bwd.conv_backward_bias(g))
        assert eb <= TAU_W[dtype], f"dB rel err {eb:.3e}"
    return op.handle.route


DATA_CASES = [
    # (dtype, x, w, attrs, expected route)
    ("f16", [2, 64, 16, 16], [96, 64, 3, 3], dict(pads=[1, 1, 1, 1]), "igemm_halo"),
    ("f16", [2, 32, 20, 12], [48, 16, 3, 3], dict(pads=[1, 1, 1, 1], group=2), "igemm_halo"),
    ("f16", [2, 48, 9, 13], [40, 48, 3, 3], {}, "igemm"),       # full conv; tiles too padded for halo
    ("f16", [1, 32, 12, 12], [32, 32, 5, 5], dict(pads=[2, 2, 2, 2], dilations=[1, 1]), "igemm_halo"),
    ("f16", [2, 12, 11, 11], [20, 12, 3, 3], dict(pads=[1, 1, 1, 1]), "igemm"),
    ("f32", [2, 12, 11, 11], [20, 12, 3, 3], dict(pads=[1, 1, 1, 1]), "igemm"),
    ("f32", [2, 24, 40], [18, 8, 5], dict(group=3, dilations=[2], pads=[4, 2]), "igemm"),
    ("f32", [1, 8, 5, 7, 6], [16, 8, 3, 2, 3], dict(pads=[1, 0, 1, 1, 1, 1]), "igemm"),
    ("f16", [2, 6, 9, 9], [5, 6, 3, 3], dict(pads=[1, 1, 1, 1]), "direct"),
    # strided: the transposed gather kernel
    ("f16", [2, 32, 16, 16], [64, 32, 3, 3], dict(strides=[2, 2], pads=[1, 1, 1, 1]), "transposed"),
    ("f32", [2, 16, 15, 17], [24, 8, 3, 3], dict(strides=[2, 3], group=2), "transposed"),
    ("f16", [2, 32, 16, 16], [64, 32, 2, 2], dict(strides=[2, 2]), "transposed"),
    ("f32", [1, 8, 9, 10, 11], [8, 4, 3, 3, 3], dict(strides=[2, 2, 1], group=2,
                                                      auto_pad="SAME_UPPER"), "transposed"),
]


@pytest.mark.parametrize("ci", range(len(DATA_CASES)))
def test_backward_data(ci):
    dtype, xs, ws, attrs, want = DATA_CASES[ci]
    for k, (act, res) in enumerate([(("QuickGelu", [1.702]), True), ((None, None), False),
                                    (ACTS[(3 * ci) % len(ACTS)], ci % 2 == 0)]):
        route = run_data(dtype, xs, ws, attrs, [9600, ci, k], act, res)
        assert route == want, (route, want)


@pytest.mark.parametrize("act", ACTS, ids=[str(a[0]) + str(a[1] or "") for a in ACTS])
@pytest.mark.parametrize("route", ["igemm_halo", "igemm", "transposed"])
def test_backward_data_every_activation_derivative(act, route):
    # fp32 where the route allows it, so that the derivative's own error shows
    dtype = "f16" if route == "igemm_halo" else "f32"
    run_data(dtype, [2, 32, 12, 12], [32, 32, 3, 3], dict(pads=[1, 1, 1, 1]), [9700], act,
             residual=True, route=route)


def test_backward_data_forced_routes_agree():
    xs, ws, attrs = [2, 32, 12, 12], [48, 32, 3, 3], dict(pads=[1, 1, 1, 1])
    for route in ("igemm_halo", "igemm", "direct", "transposed"):
        assert run_data("f16", xs, ws, attrs, [9800], ("Tanh", None), True, route=route) == route
    assert run_data("f32", xs, ws, attrs, [9801], ("Elu", [0.5]), False, route="igemm",
                    split_k=3) == "igemm"


WEIGHT_CASES = [
    ("f16", [4, 64, 16, 16], [96, 64, 3, 3], dict(pads=[1, 1, 1, 1])),
    ("f16", [3, 32, 20, 12], [48, 16, 3, 3], dict(pads=[1, 1, 1, 1], group=2)),
    ("f16", [2, 12, 32, 32], [64, 12, 3, 3], dict(pads=[1, 1, 1, 1])),        # K 108 (+1) -> 112
    ("f16", [2, 3, 64, 64], [96, 3, 4, 4], dict(strides=[4, 4])),             # patchify, K 48
    ("f16", [2, 3, 56, 56], [64, 3, 7, 7], dict(strides=[2, 2], pads=[3, 3, 3, 3])),  # P 784
    ("f16", [2, 300, 8, 8], [280, 300, 1, 1], {}),                            # 2 m tiles, 3 k tiles
    ("f16", [2, 16, 14, 14], [32, 16, 3, 3], dict(pads=[1, 1, 1, 1])),        # P 196 (rows of 200)
    ("f32", [2, 24, 40], [18, 8, 5], dict(group=3, dilations=[2], pads=[4, 4])),
    ("f32", [1, 8, 4, 8, 8], [16, 8, 3, 3, 3], dict(pads=[1, 1, 1, 1, 1, 1])),
    ("f32", [2, 16, 12, 12], [24, 16, 3, 3], dict(strides=[2, 2], pads=[1, 1, 0, 0])),  # P 36
]


@pytest.mark.parametrize("ci", range(len(WEIGHT_CASES)))
def test_backward_weight(ci):
    # the column-matrix GEMM (the planner's choice for all of these but case 0)
    dtype, xs, ws, attrs = WEIGHT_CASES[ci]
    assert run_weight(dtype, xs, ws, attrs, [9900, ci], bias=True, route="im2col") == "im2col"
    assert run_weight(dtype, xs, ws, attrs, [9901, ci], bias=False, route="im2col") == "im2col"


TAP_CASES = [
    # the shifted-tap kernel: fp16, stride 1, <= 9 taps, W and OW multiples of
    # 8, C/group a multiple of 16
    ([4, 64, 16, 16], [96, 64, 3, 3], dict(pads=[1, 1, 1, 1])),
    ([2, 32, 16, 16], [64, 16, 3, 3], dict(pads=[1, 1, 1, 1], group=2)),
    ([2, 16, 24, 32], [300, 16, 3, 3], dict(pads=[1, 1, 1, 1])),         # 2 output tiles, M 300
    ([1, 32, 8, 64], [32, 32, 1, 3], dict(pads=[0, 1, 0, 1])),           # 1x3
    ([3, 16, 16, 16], [16, 16, 3, 3], dict(pads=[2, 2, 2, 2], dilations=[2, 2])),
    ([2, 32, 64], [48, 32, 5], dict(pads=[2, 2])),                       # 1-D, 5 taps
    ([1, 16, 100, 48], [32, 16, 3, 3], dict(pads=[1, 1, 1, 1])),         # 13 bands of 8 rows
    ([2, 16, 18, 16], [24, 16, 3, 3], dict(pads=[0, 1, 0, 1])),          # valid rows, OH 16
]


@pytest.mark.parametrize("ci", range(len(TAP_CASES)))
def test_backward_weight_shifted_taps(ci):
    xs, ws, attrs = TAP_CASES[ci]
    assert run_weight("f16", xs, ws, attrs, [9920, ci], bias=True) == "igemm_halo"
    assert run_weight("f16", xs, ws, attrs, [9921, ci], bias=False) == "igemm_halo"
    # the same problem on the column-matrix GEMM
    assert run_weight("f16", xs, ws, attrs, [9920, ci], bias=True, route="im2col") == "im2col"


def test_backward_weight_plain_reduction():
    # 15x15 outputs: not a multiple of 4, the planner takes the plain reduction
    assert run_weight("f16", [2, 8, 15, 15], [12, 8, 3, 3], dict(pads=[1, 1, 1, 1]), [9950]) == "direct"
    assert run_weight("f32", [2, 8, 16, 16], [12, 4, 3, 3], dict(group=2), [9951],
                      route="direct") == "direct"


def test_backward_repeated_runs_are_bitwise_identical():
    xs, ws, attrs = [4, 64, 16, 16], [96, 64, 3, 3], dict(pads=[1, 1, 1, 1])
    ys = fwd_y_shape(xs, ws, attrs)
    x, w, _, g = random_tensors([9990], "f16", xs, ws, None, ys, dist="normal")
    pre = dev(np.random.default_rng(9991).standard_normal(xs).astype(np.float16))
    opd = fc.ConvBackwardData(xs, ws, "f16", False, "QuickGelu", None, **attrs)
    opw = fc.ConvBackwardWeight(xs, ws, "f16", True, **attrs)
    gd, wd, xd = dev(g), dev(w), dev(x)
    a1, a2 = opd(gd, wd, pre), opd(gd, wd, pre)
    (w1, b1), (w2, b2) = opw(xd, gd), opw(xd, gd)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(w1, w2) and torch.equal(b1, b2)


def test_full_size_headline_backward():
    """The backward of the CIFAR ResNet 3x3 conv at full size: the input
    gradient with the QuickGelu derivative and a residual gradient (every
    element of dP), then dW and dB (every element)."""
    name = "cifar_resnet_conv3x3_f16"
    wl = WORKLOADS[name]
    inp = make_inputs(name)
    xs, ws = wl["x"], wl["w"]
    attrs = {k: v for k, v in wl["attrs"].items() if k not in ("activation", "activation_params")}
    rng = np.random.default_rng([9999, 1])
    g = (rng.standard_normal(wl["y"]) * 0.1).astype(np.float16)
    pre = (rng.standard_normal(xs) * 2).astype(np.float16)
    r = (rng.standard_normal(xs) * 0.1).astype(np.float16)
    opd = fc.ConvBackwardData(xs, ws, "f16", True, "QuickGelu", [1.702], **attrs)
    log(f"CASE full-size bwd-data {name} route={opd.handle.route} ({opd.handle.kernel_name})")
    dx = opd(dev(g), dev(inp["w"]), dev(pre), dev(r)).cpu().numpy()
    max_err = max_ref = 0.0
    step = 64
    for n0 in range(0, xs[0], step):
        sl = slice(n0, n0 + step)
        ref = bwd.conv_backward_data(g[sl], inp["w"], [min(step, xs[0] - n0)] + xs[1:],
                                     pre=pre[sl], residual=r[sl], input_activation="QuickGelu",
                                     input_activation_params=[float(np.float32(1.702))], **attrs)
        max_err = max(max_err, float(np.max(np.abs(dx[sl].astype(np.float64) - ref))))
        max_ref = max(max_ref, float(np.max(np.abs(ref))))
    rel = max_err / max_ref
    log(f"RESULT full-size bwd-data {name}: {rel:.3e} over {dx.size} outputs")
    assert rel <= TAU_X["f16"]
    opw = fc.ConvBackwardWeight(xs, ws, "f16", True, **attrs)
    log(f"CASE full-size bwd-weight {name} route={opw.handle.route} splits={opw.handle.split_k}")
    dw, db = opw(dev(inp["x"]), dev(g))
    dw, db = dw.cpu().numpy(), db.cpu().numpy()
    ref_w = bwd.conv_backward_weight(inp["x"], g, ws, **attrs)
    ew, eb = rel_err(dw, ref_w), rel_err(db, bwd.conv_backward_bias(g))
    log(f"RESULT full-size bwd-weight {name}: dW {ew:.3e}, dB {eb:.3e}")
    assert ew <= TAU_W["f16"] and eb <= TAU_W["f16"]
