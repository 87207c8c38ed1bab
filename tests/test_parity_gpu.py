"""GPU parity: the HIP path against the oracle, element by element.

Tolerance (stated for this path): max|Y_gpu - Y_ref| <= tau * max|Y_ref| with
tau = 1e-4 for fp32 and 2e-2 for fp16 (fp32 accumulation, one fp16 rounding
of the output), Y_ref being the oracle's unrounded double result on the same
inputs.  Every case compares every output element, the full-size workloads
included: they run in the launch configuration the benchmark times and are
compared against the oracle a few images at a time, with the maximum error
and the maximum |Y_ref| taken over the whole output tensor.
"""
import sys

import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as fc
from convolution_implicit_gemm_amd import _binding as B
from oracle import oracle
from workloads import WORKLOADS, make_inputs, random_tensors

pytestmark = pytest.mark.gpu
TAU = {"f32": 1e-4, "f16": 2e-2}
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
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
    fc.load()  # fails loudly when the library is not built
    oracle.build(force=False)


def f32params(p):
    return None if p is None else [float(np.float32(v)) for v in p]


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(x, w, b, z, **kw):
    y = fc.fused_conv(dev(x), dev(w), dev(b), dev(z), **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


class Ref(np.ndarray):
    """The oracle's Y with `alt`: where not NaN, a second value an output
    may take (see reference())."""
    alt = None


def reference(x, w, b, z, **attrs):
    """oracle.fusedconv(x, w, b, z, **attrs), and for ThresholdedRelu the
    outputs whose decision x > alpha is not fixed by the kernels' precision.
    The kernels decide on an fp32 sum; recursive fp32 summation of K products
    plus bias and residual is within 2 (K + 2) 2^-24 sum|terms| of the exact
    value, and sum|terms| is the oracle run on |X|, |W|, |B|, |Z|.  Where the
    float64 pre-activation lies within that bound of alpha, both 0 and the
    pre-activation are correct outputs."""
    ref = oracle.fusedconv(x, w, b, z, **attrs)
    if attrs.get("activation") != "ThresholdedRelu":
        return ref
    p = attrs.get("activation_params")
    alpha = float(p[0]) if p else 1.0
    base = dict(attrs, activation=None, activation_params=None)
    pre = oracle.fusedconv(x, w, b, z, **base)
    ab = lambda a: None if a is None else np.abs(a)
    mag = oracle.fusedconv(np.abs(x), np.abs(w), ab(b), ab(z), **base)
    k = int(np.prod(w.shape[1:]))
    near = np.abs(pre - alpha) <= 2.0 * (k + 2) * 2.0 ** -24 * mag
    out = np.asarray(ref).view(Ref)
    out.alt = np.where(near, np.where(pre > alpha, 0.0, pre), np.nan)
    return out


def check(got, ref, dtype, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g = got.astype(np.float64)
    assert np.all(np.isfinite(g)), what
    ref_ = np.asarray(ref)
    scale = max(np.max(np.abs(ref_)), 1e-30)
    d = np.abs(g - ref_)
    alt = getattr(ref, "alt", None)
    if alt is not None:  # either side of a ThresholdedRelu decision the kernels' sum leaves open
        d = np.where(np.isnan(alt), d, np.minimum(d, np.abs(g - np.nan_to_num(alt))))
    err = np.max(d) / scale
    assert err <= TAU[dtype], f"{what}: rel err {err:.3e} > {TAU[dtype]}"
    return err


def case_attrs(rng, nsp, allow_group=True):
    group = int(rng.choice([1, 2, 3])) if allow_group else 1
    cg = int(rng.integers(3, 24))
    mg = int(rng.integers(5, 45))
    ks = [int(v) for v in rng.integers(1, 4, nsp)]
    ins = [int(v) for v in rng.integers(5, 14 if nsp == 3 else (22 if nsp == 2 else 300), nsp)]
    ss = [int(v) for v in rng.integers(1, 3, nsp)]
    ds = [int(v) for v in rng.integers(1, 3, nsp)]
    mode = str(rng.choice(["NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID"]))
    pads = [int(v) for v in rng.integers(0, 3, 2 * nsp)] if mode == "NOTSET" else None
    for i in range(nsp):
        ins[i] = max(ins[i], (ks[i] - 1) * ds[i] + 1)
    return dict(n=int(rng.integers(1, 4)), C=cg * group, M=mg * group, group=group, ks=ks,
                ins=ins, strides=ss, dilations=ds, auto_pad=mode, pads=pads)


def run_case(c, dtype, seed, route, split_k=0, act=(None, None), bias=True, resid=True):
    x_shape = [c["n"], c["C"]] + c["ins"]
    w_shape = [c["M"], c["C"] // c["group"]] + c["ks"]
    out = oracle.output_dims(c["ins"], c["ks"], c["strides"], c["dilations"], c["auto_pad"],
                             c["pads"])
    y_shape = [c["n"], c["M"]] + out[0]
    x, w, b, z = random_tensors(seed, dtype, x_shape, w_shape, [c["M"]] if bias else None,
                                y_shape if resid else None)
    attrs = dict(group=c["group"], strides=c["strides"], dilations=c["dilations"],
                 auto_pad=c["auto_pad"], pads=c["pads"], activation=act[0],
                 activation_params=f32params(act[1]))
    what = f"seed={seed} route={route} split={split_k} dtype={dtype} x={x_shape} w={w_shape} {attrs}"
    log("CASE " + what)
    got = run_gpu(x, w, b, z, route=route, split_k=split_k, **attrs)
    ref = reference(x, w, b, z, **attrs)
    return check(got, ref, dtype, what)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("nsp", [1, 2, 3])
@pytest.mark.parametrize("route", ["direct", "igemm"])
def test_routes_random_small(route, nsp, dtype):
    rng = np.random.default_rng([1000, nsp, len(route), dtype == "f16"])
    for trial in range(6):
        c = case_attrs(rng, nsp)
        act = ACTS[int(rng.integers(0, len(ACTS)))]
        run_case(c, dtype, [2000, nsp, trial, len(route)], route, act=act,
                 bias=trial % 3 != 1, resid=trial % 3 != 2)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("split", [2, 3, 7])
def test_igemm_forced_split(split, dtype):
    rng = np.random.default_rng([3000, split])
    for trial in range(3):
        c = case_attrs(rng, 2)
        c["C"] = c["group"] * 40  # K = 40 * taps >= 7 tiles of 32 when taps >= 6
        c["ks"] = [3, 3]
        c["ins"] = [max(v, 5) for v in c["ins"]]
        run_case(c, dtype, [3001, split, trial], "igemm", split_k=split,
                 act=ACTS[trial * 5 % len(ACTS)])


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("act", ACTS, ids=[str(a[0]) + str(a[1] or "") for a in ACTS])
def test_every_activation(act, dtype):
    c = dict(n=2, C=24, M=40, group=1, ks=[3, 3], ins=[13, 17], strides=[1, 1],
             dilations=[1, 1], auto_pad="SAME_UPPER", pads=None)
    for route in ("igemm", "direct"):
        run_case(c, dtype, [4000, ACTS.index(act)], route, act=act)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_depthwise_route(dtype):
    rng = np.random.default_rng(5000)
    for trial in range(10):
        nsp = 1 if trial % 4 == 3 else 2
        C = int(rng.integers(3, 40))
        mult = int(rng.choice([1, 1, 2]))
        ks = [int(v) for v in rng.integers(1, 8, nsp)]
        ds = [int(v) for v in rng.integers(1, 3, nsp)]
        ins = [int(v) for v in rng.integers(5, 70 if nsp == 2 else 3000, nsp)]
        for i in range(nsp):
            ins[i] = max(ins[i], (ks[i] - 1) * ds[i] + 1)
        mode = str(rng.choice(["NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID"]))
        c = dict(n=int(rng.integers(1, 3)), C=C, M=C * mult, group=C, ks=ks, ins=ins,
                 strides=[int(v) for v in rng.integers(1, 3, nsp)], dilations=ds, auto_pad=mode,
                 pads=[int(v) for v in rng.integers(0, 4, 2 * nsp)] if mode == "NOTSET" else None)
        run_case(c, dtype, [5001, trial], "depthwise", act=ACTS[trial % len(ACTS)],
                 bias=trial % 2 == 0, resid=trial % 3 == 0)


DW_FAST_CASES = [
    # (n, C, mult, H, W, k, dilation, auto_pad / pads) for the fp16 dot2 depthwise kernel
    (2, 5, 1, 56, 58, 7, 1, "SAME_UPPER"),     # W % 8 != 0: not the MFMA kernel
    (1, 3, 1, 56, 50, 7, 2, "SAME_UPPER"),
    (2, 4, 2, 17, 23, 5, 1, "SAME_LOWER"),
    (1, 6, 1, 31, 9, 3, 3, "VALID"),
    (3, 2, 1, 13, 61, 7, 1, [3, 1, 2, 0]),
    (1, 7, 1, 1, 300, 5, 2, "SAME_UPPER"),    # 1-D shaped plane
]


@pytest.mark.parametrize("ci", range(len(DW_FAST_CASES)))
def test_depthwise_fast_path(ci):
    n, C, mult, H, W, k, d, pad = DW_FAST_CASES[ci]
    attrs = dict(group=C, dilations=[d, d])
    if isinstance(pad, list):
        attrs["pads"] = pad
    else:
        attrs["auto_pad"] = pad
    xs, ws = [n, C, H, W], [C * mult, 1, k, k]
    h = B.Handle("f16", xs, ws, None, None, route="depthwise", **attrs)
    assert h.kernel_name.startswith("depthwise_dot2"), h.kernel_name
    for kk, (bias, resid) in enumerate([(True, False), (False, True), (True, True)]):
        act, params = ACTS[(3 * ci + 5 * kk) % len(ACTS)]
        x, w, b, z = random_tensors([9200, ci, kk], "f16", xs, ws, [C * mult] if bias else None,
                                    h.y_shape if resid else None, dist="normal")
        a = dict(attrs, activation=act, activation_params=f32params(params))
        log(f"CASE dw fast {ci} x={xs} w={ws} {a}")
        got = run_gpu(x, w, b, z, route="depthwise", **a)
        ref = reference(x, w, b, z, **a)
        check(got, ref, "f16", f"dw fast case {ci}")


@pytest.mark.parametrize("act", [("LeakyRelu", [0.1]), ("Clip", [-0.5, 1.5])],
                         ids=["LeakyRelu", "Clip"])
def test_depthwise_fast_path_parametrised_activations(act):
    # the dot2 kernel's instances for the two activations whose parameters are
    # mandatory, which the case table above does not reach
    xs, ws = [2, 5, 33, 42], [5, 1, 5, 5]
    attrs = dict(group=5, auto_pad="SAME_UPPER", activation=act[0],
                 activation_params=f32params(act[1]))
    h = B.Handle("f16", xs, ws, [5], xs, route="depthwise", **attrs)
    assert h.kernel_name.startswith("depthwise_dot2"), h.kernel_name
    x, w, b, z = random_tensors([9210, len(act[0])], "f16", xs, ws, [5], xs, dist="normal")
    log(f"CASE dw fast {act[0]} x={xs} w={ws}")
    got = run_gpu(x, w, b, z, route="depthwise", **attrs)
    ref = reference(x, w, b, z, **attrs)
    check(got, ref, "f16", f"dw fast {act[0]}")


DWM_CASES = [
    # (n, C, mult, H, W, (kh, kw), (dh, dw), auto_pad / pads) for the banded-MFMA kernel
    (2, 5, 1, 56, 56, (7, 7), (1, 1), "SAME_UPPER"),
    (1, 3, 1, 56, 56, (7, 7), (2, 2), "SAME_UPPER"),
    (2, 4, 2, 16, 24, (5, 5), (1, 1), "SAME_LOWER"),      # channel multiplier 2
    (1, 6, 1, 31, 40, (3, 3), (2, 1), [2, 4, 3, 6]),     # row dilation 2 only, OW = 48
    (3, 2, 1, 13, 64, (7, 3), (1, 2), [3, 2, 3, 2]),     # KH != KW, column dilation 2
    (1, 2, 1, 20, 32, (3, 17), (1, 1), "SAME_UPPER"),    # widest band: 16 + 16 columns
    (2, 3, 1, 18, 16, (5, 9), (1, 2), "SAME_UPPER"),     # dw * (KW-1) = 16
    (1, 4, 1, 8, 8, (3, 3), (1, 1), "SAME_LOWER"),       # one tile column
    (2, 3, 1, 61, 48, (7, 7), (1, 1), [0, 11, 0, 3]),    # large left pad, OH = 55
]


@pytest.mark.parametrize("ci", range(len(DWM_CASES)))
def test_depthwise_mfma_path(ci):
    n, C, mult, H, W, k, d, pad = DWM_CASES[ci]
    attrs = dict(group=C, dilations=list(d))
    if isinstance(pad, list):
        attrs["pads"] = pad
    else:
        attrs["auto_pad"] = pad
    xs, ws = [n, C, H, W], [C * mult, 1] + list(k)
    h = B.Handle("f16", xs, ws, None, None, route="depthwise", **attrs)
    assert h.kernel_name.startswith("depthwise_mfma"), h.kernel_name
    for kk, (bias, resid) in enumerate([(True, False), (False, True), (True, True)]):
        act, params = ACTS[(3 * ci + 5 * kk) % len(ACTS)]
        x, w, b, z = random_tensors([9300, ci, kk], "f16", xs, ws, [C * mult] if bias else None,
                                    h.y_shape if resid else None, dist="normal")
        a = dict(attrs, activation=act, activation_params=f32params(params))
        log(f"CASE dw mfma {ci} x={xs} w={ws} {a}")
        got = run_gpu(x, w, b, z, route="depthwise", **a)
        ref = reference(x, w, b, z, **a)
        check(got, ref, "f16", f"dw mfma case {ci}")


def test_depthwise_mfma_many_images_per_block():
    # enough planes that a block walks several images, with a ragged last run
    xs, ws = [7, 2048, 8, 16], [2048, 1, 3, 3]
    attrs = dict(group=2048, pads=[1, 1, 1, 1], activation="Relu")
    h = B.Handle("f16", xs, ws, None, None, route="depthwise", **attrs)
    assert h.kernel_name.startswith("depthwise_mfma"), h.kernel_name
    x, w, b, z = random_tensors([9310], "f16", xs, ws, [2048], h.y_shape, dist="normal")
    log(f"CASE dw mfma many images x={xs}")
    got = run_gpu(x, w, b, z, route="depthwise", **attrs)
    ref = reference(x, w, b, z, **attrs)
    check(got, ref, "f16", "dw mfma many images")


def test_depthwise_mfma_nonfinite_input_stays_local():
    # an infinite input reaches only the outputs whose window holds it; its
    # plane takes the exact loop, the other planes the matrix cores
    xs, ws = [2, 3, 24, 32], [3, 1, 5, 5]
    attrs = dict(group=3, auto_pad="SAME_UPPER")
    h = B.Handle("f16", xs, ws, None, None, route="depthwise", **attrs)
    assert h.kernel_name.startswith("depthwise_mfma"), h.kernel_name
    x, w, b, _ = random_tensors([9320], "f16", xs, ws, [3], None, dist="normal")
    x[0, 1, 10, 20] = np.inf
    x[1, 2, 3, 4] = -np.inf
    log("CASE dw mfma non-finite")
    got = run_gpu(x, w, b, None, route="depthwise", **attrs).astype(np.float64)
    ref = reference(x, w, b, None, **attrs)
    fin = np.isfinite(ref)
    assert (~fin).sum() == 2 * 25
    assert np.array_equal(np.isfinite(got), fin)
    assert np.array_equal(got[~fin], ref[~fin])
    scale = np.max(np.abs(ref[fin]))
    assert np.max(np.abs(got[fin] - ref[fin])) / scale <= TAU["f16"]


def test_depthwise_mfma_nonfinite_across_channels():
    # runs of several planes per block that cross channels: the exact loop
    # must take each flagged plane's own weights and bias
    xs, ws = [2, 1500, 8, 16], [1500, 1, 3, 3]
    attrs = dict(group=1500, pads=[1, 1, 1, 1], activation="Tanh")
    h = B.Handle("f16", xs, ws, None, None, route="depthwise", **attrs)
    assert h.kernel_name.startswith("depthwise_mfma"), h.kernel_name
    x, w, b, z = random_tensors([9330], "f16", xs, ws, [1500], h.y_shape, dist="normal")
    x[0, 1, 4, 5] = np.inf      # planes (channel 1, image 0) and (channel 0, image 1)
    x[1, 0, 0, 0] = np.nan      # share the first block's run
    x[1, 1499, 7, 15] = -np.inf
    log("CASE dw mfma non-finite across channels")
    got = run_gpu(x, w, b, z, route="depthwise", **attrs).astype(np.float64)
    ref = reference(x, w, b, z, **attrs)
    fin = np.isfinite(ref)
    assert (~fin).sum() > 0
    assert np.array_equal(np.isfinite(got), fin)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    scale = np.max(np.abs(ref[fin]))
    assert np.max(np.abs(got[fin] - ref[fin])) / scale <= TAU["f16"]


HALO_CASES = [
    # (x, w, attrs) for the channel-last halo route (fp16)
    ([2, 64, 16, 16], [96, 64, 3, 3], dict(pads=[1, 1, 1, 1])),            # M tail (96 < 128)
    ([2, 40, 13, 13], [64, 40, 3, 3], dict(pads=[1, 1, 1, 1])),            # partial channel
    # block, W % 8 != 0 (scalar loader), OW % 4 != 0 (residual in the epilogue)
    ([1, 64, 24, 24], [64, 64, 2, 2], dict(strides=[2, 2])),               # patchify, stride 2
    ([2, 64, 500], [64, 32, 5], dict(group=2, auto_pad="SAME_UPPER")),     # 1-D, 2 groups
    ([1, 32, 6, 16, 16], [48, 32, 3, 3, 3], dict(pads=[1] * 6)),           # 3-D
    ([2, 48, 21, 13], [40, 48, 3, 3], dict(dilations=[2, 1], auto_pad="SAME_LOWER")),
    ([1, 64, 40, 40], [300, 64, 3, 3], dict(pads=[1, 1, 1, 1])),           # 3 m blocks
    ([2, 32, 34, 70], [64, 32, 5, 7], dict(strides=[1, 2], pads=[2, 3, 2, 3])),  # 35 taps
    ([2, 96, 16, 16], [64, 96, 1, 1], {}),                                  # 1x1: one tap per block
    ([1, 64, 33, 40], [128, 64, 3, 3], dict(strides=[2, 2], pads=[1, 1, 1, 1])),  # stride 2 3x3
    ([2, 16, 12, 16], [32, 16, 1, 1], {}),                                  # a single K step
    ([1, 32, 4, 20, 32], [64, 32, 1, 3, 3], dict(strides=[1, 2, 2], pads=[0, 1, 1] * 2)),  # 3-D strided
]


@pytest.mark.parametrize("ci", range(len(HALO_CASES)))
def test_halo_route(ci):
    xs, ws, attrs = HALO_CASES[ci]
    h = B.Handle("f16", xs, ws, None, None, route="igemm_halo", **attrs)
    y_shape = h.y_shape
    for k, (bias, resid) in enumerate([(True, True), (False, False), (True, False)]):
        act, params = ACTS[(5 * ci + 7 * k) % len(ACTS)]
        x, w, b, z = random_tensors([9100, ci, k], "f16", xs, ws, [ws[0]] if bias else None,
                                    y_shape if resid else None, dist="normal",
                                    w_std=1.0 / np.sqrt(np.prod(ws[1:])))
        a = dict(attrs, activation=act, activation_params=f32params(params))
        log(f"CASE halo {ci} x={xs} w={ws} {a} bias={bias} z={resid}")
        got = run_gpu(x, w, b, z, route="igemm_halo", **a)
        ref = reference(x, w, b, z, **a)
        check(got, ref, "f16", f"halo case {ci}")


SMALLC_CASES = [
    # (x, w, attrs) for the few-input-channel route (fp16)
    ([2, 3, 64, 64], [32, 3, 7, 7], dict(strides=[4, 4], pads=[3, 3, 3, 3])),  # stem, aligned
    ([2, 3, 63, 80], [64, 3, 3, 3], dict(strides=[2, 2], pads=[1, 1, 1, 1])),  # stride 2
    ([2, 4, 20, 30], [40, 4, 5, 5], dict(pads=[2, 2, 2, 2])),                  # stride 1
    ([1, 2, 16, 40], [16, 2, 3, 11], dict(pads=[1, 5, 1, 5])),                 # 2 chunks per row
    ([2, 3, 300], [24, 3, 9], dict(auto_pad="SAME_UPPER")),                    # 1-D
    ([2, 8, 20, 20], [32, 4, 3, 3], dict(group=2, pads=[1, 1, 1, 1])),         # groups
    ([1, 3, 30, 30], [16, 3, 3, 3], dict(dilations=[2, 1])),                   # dilated rows
    ([1, 3, 32, 32], [200, 3, 3, 3], dict(pads=[1, 1, 1, 1])),                 # 2 m blocks
    ([2, 3, 27, 27], [16, 3, 3, 3], dict(strides=[2, 2])),                     # OW % 4 != 0
    ([2, 3, 64, 64], [32, 3, 7, 7], dict(strides=[4, 4], pads=[1, 1, 1, 1])),  # no tap shift fits
    ([1, 3, 64, 72], [48, 3, 6, 6], dict(strides=[4, 4], pads=[2, 2, 2, 2])),  # tap shift 2
]


@pytest.mark.parametrize("ci", range(len(SMALLC_CASES)))
def test_smallc_route(ci):
    xs, ws, attrs = SMALLC_CASES[ci]
    h = B.Handle("f16", xs, ws, None, None, route="smallc", **attrs)
    for k, (bias, resid) in enumerate([(True, True), (False, False), (True, False)]):
        act, params = ACTS[(3 * ci + 5 * k) % len(ACTS)]
        x, w, b, z = random_tensors([9300, ci, k], "f16", xs, ws, [ws[0]] if bias else None,
                                    h.y_shape if resid else None, dist="normal",
                                    w_std=1.0 / np.sqrt(np.prod(ws[1:])))
        a = dict(attrs, activation=act, activation_params=f32params(params))
        log(f"CASE smallc {ci} x={xs} w={ws} {a} bias={bias} z={resid}")
        got = run_gpu(x, w, b, z, route="smallc", **a)
        ref = reference(x, w, b, z, **a)
        check(got, ref, "f16", f"smallc case {ci}")


@pytest.mark.parametrize("act", ["Gelu", "Erf"])
def test_smallc_phi_table_activations(act):
    """The few-channel route evaluates the erf-form Gelu and Erf from an LDS table
    of the normal CDF with linear interpolation.  Pre-activations here spread
    well past +-6 (the table's range) and cover its interior densely; Erf's
    outputs lie in [-1, 1], so its bound is absolute: the table's error
    (<= 1.5e-5 in erf, 4.4e-5 in Gelu), the fp32 sums' error carried through
    the activation (~1e-5 here) and one fp16 rounding (<= 2^-11 * |y|)."""
    xs, ws = [2, 3, 64, 64], [64, 3, 7, 7]
    attrs = dict(strides=[2, 2], pads=[3, 3, 3, 3], activation=act)
    h = B.Handle("f16", xs, ws, [64], None, route="smallc", **attrs)
    x, w, b, _ = random_tensors([9350, len(act)], "f16", xs, ws, [64], None, dist="normal",
                                w_std=0.5)
    log(f"CASE smallc phi table {act} {h.kernel_name}")
    got = run_gpu(x, w, b, None, route="smallc", **attrs).astype(np.float64)
    ref = reference(x, w, b, None, **attrs)
    pre = reference(x, w, b, None, **dict(attrs, activation=None))
    assert np.abs(pre).max() > 8 and np.mean(np.abs(pre) < 6) > 0.3  # both regions covered
    err = np.abs(got - ref)
    if act == "Erf":
        assert err.max() <= 1e-4 + 2.0 ** -11, err.max()
    else:
        assert np.all(err <= 1e-4 + 2.0 ** -11 * np.abs(ref)), err.max()


# Grids of 1024 work units (4 blocks per CU), XCD-remapped block order, full
# output compared; the second shape's tiles run partly past the output (12 of
# 16 rows).
LARGE_GRID_CASES = [
    ([1024, 32, 16, 16], [128, 32, 3, 3], dict(pads=[1, 1, 1, 1])),
    ([1024, 32, 12, 16], [128, 32, 3, 3], dict(pads=[1, 1, 1, 1])),
]


@pytest.mark.parametrize("ci", range(len(LARGE_GRID_CASES)))
def test_halo_large_grid(ci):
    xs, ws, attrs = LARGE_GRID_CASES[ci]
    h = B.Handle("f16", xs, ws, [ws[0]], None, route="igemm_halo", **attrs)
    x, w, b, z = random_tensors([9200, ci], "f16", xs, ws, [ws[0]], h.y_shape, dist="normal",
                                w_std=1.0 / np.sqrt(np.prod(ws[1:])))
    a = dict(attrs, activation="QuickGelu", activation_params=f32params([1.702]))
    log(f"CASE halo large grid {ci} x={xs} w={ws} {a}")
    got = run_gpu(x, w, b, z, route="igemm_halo", **a)
    ref = reference(x, w, b, z, **a)
    check(got, ref, "f16", f"halo large grid case {ci}")


# Blocks of 256 output channels (8 waves on one input box, one block per CU):
# more than 128 output channels per group, an input box at least twice the
# tile (strided) and at least 256 tiles.  Full output compared.
WIDE_CASES = [
    ([64, 32, 32, 64], [256, 32, 2, 2], dict(strides=[2, 2])),              # BM = 256 exactly
    ([64, 48, 32, 64], [200, 48, 2, 2], dict(strides=[2, 2])),              # M and channel tails
    ([32, 32, 64, 64], [256, 32, 3, 3], dict(strides=[2, 2], pads=[1] * 4)),  # stride 2 3x3
    ([64, 32, 24, 72], [256, 32, 2, 2], dict(strides=[2, 2])),              # tiles past the output
    ([64, 64, 32, 64], [384, 32, 2, 2], dict(group=2, strides=[2, 2])),     # two groups
    ([64, 32, 32, 60], [160, 32, 2, 2], dict(strides=[2, 2])),              # W % 8 != 0
]


@pytest.mark.parametrize("ci", range(len(WIDE_CASES)))
def test_halo_wide_blocks(ci):
    xs, ws, attrs = WIDE_CASES[ci]
    h = B.Handle("f16", xs, ws, [ws[0]], None, route="igemm_halo", **attrs)
    assert h.kernel_name.startswith("igemm_halo_f16_m256_"), h.kernel_name
    x, w, b, z = random_tensors([9250, ci], "f16", xs, ws, [ws[0]], h.y_shape, dist="normal",
                                w_std=1.0 / np.sqrt(np.prod(ws[1:])))
    a = dict(attrs, activation="QuickGelu", activation_params=f32params([1.702]))
    log(f"CASE halo wide {ci} x={xs} w={ws} {a}")
    got = run_gpu(x, w, b, z, route="igemm_halo", **a)
    ref = reference(x, w, b, z, **a)
    check(got, ref, "f16", f"halo wide case {ci}")


@pytest.mark.parametrize("route", ["direct", "igemm", "depthwise"])
def test_edge_shapes(route):
    cases = [
        # 1x1 kernel, stride 2 (pure subsample + channel mix)
        dict(n=1, C=5, M=7, group=1, ks=[1, 1], ins=[9, 11], strides=[2, 2], dilations=[1, 1],
             auto_pad="NOTSET", pads=None),
        # kernel as large as the input: 1x1 output
        dict(n=2, C=3, M=4, group=1, ks=[5, 6], ins=[5, 6], strides=[1, 1], dilations=[1, 1],
             auto_pad="VALID", pads=None),
        # stride larger than the kernel, big asymmetric pads
        dict(n=1, C=4, M=4, group=1, ks=[2, 2], ins=[10, 10], strides=[5, 3], dilations=[1, 1],
             auto_pad="NOTSET", pads=[3, 0, 0, 4]),
        # single channel, single output channel
        dict(n=3, C=1, M=1, group=1, ks=[3, 3], ins=[7, 7], strides=[1, 1], dilations=[2, 2],
             auto_pad="SAME_LOWER", pads=None),
        # pads wider than the kernel span
        dict(n=1, C=2, M=2, group=1, ks=[2, 1], ins=[3, 4], strides=[1, 1], dilations=[1, 1],
             auto_pad="NOTSET", pads=[4, 4, 4, 4]),
    ]
    for i, c in enumerate(cases):
        if route == "depthwise":
            c = dict(c, M=c["C"], group=c["C"])
        for dtype in ("f32", "f16"):
            run_case(c, dtype, [6000, i], route, act=ACTS[(3 * i) % len(ACTS)])


def test_starved_grid_splits_and_matches_unsplit():
    c = dict(n=1, C=512, M=64, group=1, ks=[3, 3], ins=[8, 8], strides=[1, 1],
             dilations=[1, 1], auto_pad="NOTSET", pads=[1, 1, 1, 1])
    x, w, b, z = random_tensors([7000], "f32", [1, 512, 8, 8], [64, 512, 3, 3], [64],
                                [1, 64, 8, 8], w_std=1 / 48)
    attrs = dict(pads=[1, 1, 1, 1], activation="Gelu")
    h = B.Handle("f32", [1, 512, 8, 8], [64, 512, 3, 3], [64], [1, 64, 8, 8], **attrs)
    assert h.split_k > 1
    log(f"CASE starved split={h.split_k}")
    ys = run_gpu(x, w, b, z, **attrs)
    y1 = run_gpu(x, w, b, z, route="igemm", split_k=1, **attrs)
    ref = reference(x, w, b, z, **attrs)
    check(ys, ref, "f32", "split")
    check(y1, ref, "f32", "unsplit")
    check(ys, y1.astype(np.float64), "f32", "split vs unsplit")


@pytest.mark.parametrize("route", ["direct", "igemm", "depthwise", "igemm_halo"])
def test_deterministic_and_inplace_residual(route):
    C = 16 if route != "igemm_halo" else 64
    M, grp = (C, C) if route == "depthwise" else (24, 1)
    x, w, b, z = random_tensors([8000], "f16", [2, C, 19, 23], [M, C // grp, 3, 3], [M],
                                [2, M, 19, 23])
    attrs = dict(group=grp, auto_pad="SAME_UPPER", activation="QuickGelu", route=route)
    log(f"CASE determinism route={route}")
    xd, wd, bd = dev(x), dev(w), dev(b)
    y1 = fc.fused_conv(xd, wd, bd, dev(z), **attrs)
    y2 = fc.fused_conv(xd, wd, bd, dev(z), **attrs)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    # Y written into Z's buffer (in-place residual)
    zd = dev(z)
    op = fc.FusedConv([2, C, 19, 23], [M, C // grp, 3, 3], "f16", True, True,
                      group=grp, auto_pad="SAME_UPPER", activation="QuickGelu", route=route)
    y3 = op(xd, wd, bd, zd, out=zd)
    torch.cuda.synchronize()
    assert y3.data_ptr() == zd.data_ptr()
    assert torch.equal(y3, y1)


POINTWISE_CASES = [
    # (x, w, attrs) for the 1x1 route (fp16): ragged pixel tiles, partial
    # channel blocks, odd and partial reduction steps, groups, 1-D and 3-D
    ([2, 64, 16, 16], [96, 64, 1, 1], {}),                  # Mg < 128, 2 pixel tiles
    ([2, 256, 14, 16], [256, 256, 1, 1], {}),               # 224 pixels: a partial tile; 2 m blocks
    ([2, 64, 8, 8], [64, 32, 1, 1], dict(group=2)),         # groups
    ([1, 40, 12, 12], [200, 40, 1, 1], {}),                 # C/group 40: one partial step
    ([2, 136, 8, 16], [64, 136, 1, 1], {}),                 # 3 steps, the last partial
    ([2, 128, 72], [128, 128, 1], {}),                      # 1-D
    ([1, 32, 4, 8, 8], [48, 32, 1, 1, 1], {}),              # 3-D
    ([1, 16, 8, 8], [32, 16, 1, 1], dict(dilations=[2, 2])),  # C/group 16; dilation is moot
    ([1, 1024, 8, 8], [64, 1024, 1, 1], {}),                # 16 steps
    # 2x2 with stride 2 (patch form): reduction k = c*4 + kh*2 + kw
    ([2, 64, 32, 32], [96, 64, 2, 2], dict(strides=[2, 2])),            # 256 pixels, 4 steps
    ([1, 40, 20, 48], [64, 40, 2, 2], dict(strides=[2, 2])),            # 240 pixels; 2.5 steps
    ([2, 16, 17, 16], [32, 16, 2, 2], dict(strides=[2, 2])),            # odd H (last row unused)
    ([1, 32, 16, 16], [32, 8, 2, 2], dict(strides=[2, 2], group=4)),    # groups, C/group 8
    ([1, 128, 32, 64], [256, 128, 2, 2], dict(strides=[2, 2])),         # 2 m blocks, 8 steps
]


@pytest.mark.parametrize("ci", range(len(POINTWISE_CASES)))
def test_pointwise_route(ci):
    xs, ws, attrs = POINTWISE_CASES[ci]
    h = B.Handle("f16", xs, ws, None, None, route="pointwise", **attrs)
    assert h.route == "pointwise"
    for k, (bias, resid) in enumerate([(True, True), (False, False), (True, False)]):
        act, params = ACTS[(3 * ci + 5 * k) % len(ACTS)]
        x, w, b, z = random_tensors([9400, ci, k], "f16", xs, ws, [ws[0]] if bias else None,
                                    h.y_shape if resid else None, dist="normal",
                                    w_std=1.0 / np.sqrt(np.prod(ws[1:])))
        a = dict(attrs, activation=act, activation_params=f32params(params))
        log(f"CASE pointwise {ci} x={xs} w={ws} {a} bias={bias} z={resid}")
        got = run_gpu(x, w, b, z, route="pointwise", **a)
        ref = reference(x, w, b, z, **a)
        check(got, ref, "f16", f"pointwise case {ci}")


IM2COL_CASES = [
    # (x, w, attrs) for the explicit im2col route (fp16): patchify shapes,
    # K not a multiple of 8 (W padded in the workspace), P not a multiple of
    # 8 (padded column rows), groups, 1-D and 3-D, padding and dilation
    ([2, 3, 64, 64], [96, 3, 4, 4], dict(strides=[4, 4])),             # K 48, P 256
    ([2, 3, 224, 224], [64, 3, 16, 16], dict(strides=[16, 16])),       # K 768, P 196 (rows of 200)
    ([1, 8, 28, 28], [32, 8, 14, 14], dict(strides=[14, 14])),         # P 4 (rows of 8), K 1568
    ([4, 12, 32, 32], [64, 12, 3, 3], dict(pads=[1, 1, 1, 1])),        # K 108 -> 112
    ([2, 3, 20, 20], [16, 3, 3, 3], dict(pads=[1, 1, 1, 1])),          # K 27 -> 32, M 16
    ([2, 32, 8, 8], [64, 8, 3, 3], dict(group=4, pads=[1, 1, 1, 1])),  # groups, K 72
    ([1, 8, 8, 16, 16], [32, 8, 2, 4, 4], dict(strides=[2, 4, 4])),    # 3-D patchify, P 64
    ([3, 4, 96], [16, 4, 5], dict(strides=[2], pads=[2, 2])),          # 1-D, K 20 -> 24, P 48
    ([1, 3, 20, 20], [16, 3, 5, 5], dict(dilations=[2, 2])),           # dilation, K 75 -> 80
    ([2, 64, 32, 32], [300, 64, 4, 4], dict(strides=[4, 4])),          # 2 m blocks of 256, K 1024
    ([2, 1, 16, 16], [5, 1, 2, 2], dict(strides=[2, 2])),              # K 4 -> 16, M 5
    ([3, 16, 30, 30], [24, 16, 5, 5], dict(strides=[5, 5])),           # P 36 (rows of 40), n 3
    # staging of X rows: W % 8 != 0 (2-byte row loads) with 11 pixel chunks,
    # stride 2 with an end pad and 9 chunks, 3-D rows, and rows too wide to
    # stage (the per-element gather kernel)
    ([1, 1, 40, 1100], [8, 1, 3, 3], dict(pads=[1, 1, 1, 1])),
    ([1, 1, 9, 5000], [8, 1, 2, 3], dict(strides=[1, 2], pads=[0, 1, 0, 1])),
    ([1, 2, 4, 20, 30], [8, 2, 3, 3, 3], dict(strides=[1, 2, 2], pads=[1, 1, 1, 1, 1, 1])),
    ([1, 2, 3, 8200], [8, 2, 2, 2], dict(strides=[1, 2])),
]


@pytest.mark.parametrize("ci", range(len(IM2COL_CASES)))
def test_im2col_route(ci):
    xs, ws, attrs = IM2COL_CASES[ci]
    h = B.Handle("f16", xs, ws, None, None, route="im2col", **attrs)
    assert h.route == "im2col"
    for k, (bias, resid) in enumerate([(True, True), (False, False), (True, False)]):
        act, params = ACTS[(5 * ci + 3 * k) % len(ACTS)]
        x, w, b, z = random_tensors([9500, ci, k], "f16", xs, ws, [ws[0]] if bias else None,
                                    h.y_shape if resid else None, dist="normal",
                                    w_std=1.0 / np.sqrt(np.prod(ws[1:])))
        a = dict(attrs, activation=act, activation_params=f32params(params))
        log(f"CASE im2col {ci} x={xs} w={ws} {a} bias={bias} z={resid}")
        got = run_gpu(x, w, b, z, route="im2col", **a)
        ref = reference(x, w, b, z, **a)
        check(got, ref, "f16", f"im2col case {ci}")


HALO32_CASES = [
    # (x, w, attrs) for the fp32 halo kernel: 1-D grouped and dilated, 2-D
    # with asymmetric pads, 3-D,
    # channel tails (C/group not a multiple of 16), M/group above 64
    # (128-channel blocks) with a tail, W not a multiple of 4 (element
    # loads), OW not a multiple of 4 (element stores)
    ([2, 48, 300], [48, 16, 9], dict(group=3, dilations=[3], auto_pad="SAME_LOWER")),
    ([2, 20, 31, 33], [40, 20, 3, 3], dict(pads=[1, 1, 1, 1])),
    ([1, 32, 24, 40], [72, 32, 3, 3], dict(pads=[1, 2, 1, 0])),
    ([1, 16, 4, 16, 16], [24, 16, 1, 3, 3], dict(pads=[0, 1, 1, 0, 1, 1])),
    ([2, 24, 16, 64], [150, 24, 1, 5], dict(pads=[0, 2, 0, 2])),
    ([3, 8, 19, 21], [12, 4, 3, 2], dict(group=2, dilations=[2, 1])),
    # depth-stepped boxes (3-D, one input depth plane per box): stride 1;
    # depth stride 2 with asymmetric pads (planes skipped at the borders);
    # depth dilation 2, stride 2 in-plane, W and OW not multiples of 4
    ([1, 32, 6, 16, 16], [48, 32, 3, 3, 3], dict(pads=[1] * 6)),
    ([2, 20, 5, 24, 40], [24, 20, 3, 3, 3], dict(strides=[2, 2, 2], pads=[1, 0, 1, 2, 1, 0])),
    ([1, 16, 7, 30, 30], [32, 16, 3, 5, 5], dict(strides=[1, 2, 2], dilations=[2, 1, 1],
                                                 pads=[0, 2, 2, 1, 2, 2])),
]


@pytest.mark.parametrize("ci", range(len(HALO32_CASES)))
def test_halo32_route(ci):
    xs, ws, attrs = HALO32_CASES[ci]
    h = B.Handle("f32", xs, ws, None, None, route="igemm_halo", **attrs)
    assert h.kernel_name.startswith("igemm_halo_f32"), h.kernel_name
    for k, (bias, resid) in enumerate([(True, True), (False, False), (True, False)]):
        act, params = ACTS[(7 * ci + 5 * k) % len(ACTS)]
        x, w, b, z = random_tensors([9650, ci, k], "f32", xs, ws, [ws[0]] if bias else None,
                                    h.y_shape if resid else None, dist="uniform")
        a = dict(attrs, activation=act, activation_params=f32params(params))
        log(f"CASE halo32 {ci} x={xs} w={ws} {a} bias={bias} z={resid}")
        got = run_gpu(x, w, b, z, route="igemm_halo", **a)
        ref = reference(x, w, b, z, **a)
        check(got, ref, "f32", f"halo32 case {ci}")


@pytest.mark.parametrize("route", ["igemm_halo", "igemm", "depthwise", "smallc", "pointwise",
                                   "pointwise_patch2x2", "im2col", "im2col_oddk", "halo32"])
def test_prepared_weights_match_plain_run(route):
    patch = route == "pointwise_patch2x2"
    oddk = route == "im2col_oddk"   # K 27: W padded to 32 columns in the workspace
    f32 = route == "halo32"         # the fp32 halo kernel's repacked weights
    dt = "f32" if f32 else "f16"
    route = "pointwise" if patch else ("im2col" if oddk else ("igemm_halo" if f32 else route))
    C = {"depthwise": 16, "smallc": 3}.get(route, 3 if oddk else 64)
    M, grp = (C, C) if route == "depthwise" else (96, 1)
    k = 2 if patch else (1 if route == "pointwise" else 3)
    xs, ws = [2, C, 16, 16], [M, C // grp, k, k]
    x, w, b, z = random_tensors([8100], dt, xs, ws, [M], None, dist="normal", w_std=0.05)
    attrs = dict(group=grp, pads=[1, 1, 1, 1] if k == 3 else [0, 0, 0, 0], activation="Relu",
                 route=route)
    if patch:
        attrs["strides"] = [2, 2]
    op = fc.FusedConv(xs, ws, dt, True, False, **attrs)
    xd, wd, bd = dev(x), dev(w), dev(b)
    ws_t = torch.empty(max(op.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    log(f"CASE prepared route={route} patch={patch} {op.handle.kernel_name}")
    if f32:
        assert op.handle.kernel_name.startswith("igemm_halo_f32"), op.handle.kernel_name
    if patch:
        assert op.handle.kernel_name.startswith("pointwise_f16_patch2x2"), op.handle.kernel_name
    y1 = op(xd, wd, bd, workspace=ws_t)
    op.prepare_weights(wd, ws_t)
    y2 = op(xd, wd, bd, workspace=ws_t, weights_prepared=True)
    y3 = op(xd, wd, bd, workspace=ws_t, weights_prepared=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y2, y3)
    ref = reference(x, w, b, None, **{k_: v for k_, v in attrs.items() if k_ != "route"})
    check(y1.cpu().numpy(), ref, dt, f"prepared {route}")


@pytest.mark.parametrize("route", ["igemm_halo", "pointwise"])
def test_graph_replay_matches_eager(route):
    """A captured call (weight preparation + convolution, as bench.py times
    it) replayed several times, with eager work and synchronizations between
    the replays, gives the eager result every time."""
    k = 1 if route == "pointwise" else 3
    xs, ws = [4, 64, 16, 16], [96, 64, k, k]
    x, w, b, z = random_tensors([8200, k], "f16", xs, ws, [96], [4, 96, 16, 16], dist="normal",
                                w_std=0.05)
    attrs = dict(pads=[1, 1, 1, 1] if k == 3 else [0, 0, 0, 0], activation="QuickGelu",
                 activation_params=f32params([1.702]), route=route)
    op = fc.FusedConv(xs, ws, "f16", True, True, **attrs)
    xd, wd, bd, zd = dev(x), dev(w), dev(b), dev(z)
    ws_t = torch.empty(max(op.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    log(f"CASE graph replay route={route}")
    ref = op(xd, wd, bd, zd, workspace=ws_t)
    torch.cuda.synchronize()
    y = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op.prepare_weights(wd, ws_t)
        op(xd, wd, bd, zd, out=y, workspace=ws_t, weights_prepared=True)
    for rep in range(4):
        y.zero_()
        other = op(xd, wd, bd, zd, workspace=ws_t)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"
        assert torch.equal(other, ref)


def test_run_errors_on_device():
    h = B.Handle("f32", [1, 3, 8, 8], [4, 3, 3, 3], None, None)
    x = torch.zeros(1 * 3 * 8 * 8 + 4, device="cuda")
    w = torch.zeros(4 * 27, device="cuda")
    y = torch.zeros(4 * 36, device="cuda")
    with pytest.raises(B.FusedConvError) as e:
        h.run(x.data_ptr() + 4, w.data_ptr(), None, None, y.data_ptr(), None, 0, 0)
    assert e.value.status == "FUSEDCONV_ERR_ALIGNMENT"
    hs = B.Handle("f32", [1, 512, 8, 8], [64, 512, 3, 3], None, None, pads=[1, 1, 1, 1],
                  split_k=4)
    with pytest.raises(B.FusedConvError) as e:
        hs.run(x.data_ptr(), w.data_ptr(), None, None, y.data_ptr(), None, 0, 0)
    assert e.value.status == "FUSEDCONV_ERR_WORKSPACE"
    with pytest.raises(B.FusedConvError):
        fc.fused_conv(torch.zeros(1, 3, 8, 8), torch.zeros(4, 3, 3, 3))  # host tensors


def chunks(n, per_image_outputs, limit=1 << 25):
    """Image ranges [n0, n1) holding at most `limit` outputs (at least one image)."""
    step = max(1, limit // max(per_image_outputs, 1))
    return [(i, min(n, i + step)) for i in range(0, n, step)]


def full_size_check(name, route=None):
    wl = WORKLOADS[name]
    log(f"CASE workload {name} route={route or 'auto'} x={wl['x']} w={wl['w']}")
    inp = make_inputs(name)
    attrs = dict(wl["attrs"])
    attrs["activation_params"] = f32params(attrs.get("activation_params"))
    rattrs = dict(attrs, route=route) if route else attrs
    got = run_gpu(inp["x"], inp["w"], inp["b"], inp["z"], **rattrs)
    assert list(got.shape) == wl["y"]
    assert np.all(np.isfinite(got)), name
    n = wl["x"][0]
    max_err = max_ref = 0.0
    for n0, n1 in chunks(n, int(np.prod(wl["y"][1:]))):
        zi = inp["z"][n0:n1] if inp["z"] is not None else None
        if attrs.get("transposed"):
            kw = {k: v for k, v in attrs.items() if k != "transposed"}
            ref = oracle.conv_transpose(inp["x"][n0:n1], inp["w"], inp["b"], zi, **kw)
        else:
            ref = reference(inp["x"][n0:n1], inp["w"], inp["b"], zi, **attrs)
        assert ref.shape == got[n0:n1].shape
        max_err = max(max_err, float(np.max(np.abs(got[n0:n1].astype(np.float64) - ref))))
        max_ref = max(max_ref, float(np.max(np.abs(ref))))
        del ref
    rel = max_err / max(max_ref, 1e-30)
    log(f"RESULT workload {name} route {route or 'auto'}: max |Y - Y_ref| / max |Y_ref| = "
        f"{rel:.3e} over all {got.size} outputs (tau {TAU[wl['dtype']]})")
    assert rel <= TAU[wl["dtype"]], f"{name} {route}: rel err {rel:.3e}"


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size_workloads(name):
    """The whole output tensor of every workload, in the launch configuration
    bench.py times, against the oracle (image ranges, so that the float64
    reference of one range at a time stays in memory)."""
    full_size_check(name)


COMPARED = [(name, r) for name, wl in WORKLOADS.items() for r in wl.get("compare_routes", [])]


@pytest.mark.parametrize("name,route", COMPARED, ids=[f"{n}-{r}" for n, r in COMPARED])
def test_full_size_compared_routes(name, route):
    """Every route bench.py times a workload on (implicit against explicit
    im2col; halo, gathered IGEMM and direct for the fp32 convs), whole output
    tensor against the oracle."""
    wl = WORKLOADS[name]
    h = B.Handle(wl["dtype"], wl["x"], wl["w"], wl["b"], wl["z"], **wl["attrs"])
    if h.route == route:
        pytest.skip("the planner's own route: test_full_size_workloads covers it")
    full_size_check(name, route)


TRANSPOSED_CASES = [
    # (dtype, x, w [C, M/group, k...], attrs)
    ("f32", [2, 4, 5, 6], [4, 3, 3, 2], dict(strides=[2, 3], pads=[1, 0, 2, 1], dilations=[1, 2],
                                             output_padding=[1, 2])),
    ("f16", [1, 6, 37], [6, 2, 4], dict(group=3, strides=[2], pads=[1, 2])),
    ("f32", [2, 4, 3, 4, 3], [4, 2, 2, 3, 2], dict(group=2, strides=[1, 2, 2],
                                                  pads=[0, 1, 0, 1, 0, 1], output_padding=[0, 1, 1])),
    ("f16", [2, 32, 12, 16], [32, 24, 2, 2], dict(strides=[2, 2])),           # patch upsampling
    ("f16", [1, 16, 9, 11], [16, 8, 3, 3], dict(strides=[1, 1], pads=[1, 1, 1, 1])),
    # the GEMM form (2x2 stride 2): ragged pixel tiles and column blocks,
    # cropped output_padding, groups, 256-column blocks
    ("f16", [1, 48, 5, 24], [48, 40, 2, 2], dict(strides=[2, 2], pads=[0, 0, 1, 1],
                                                 output_padding=[1, 1])),
    ("f16", [2, 64, 8, 8], [64, 12, 2, 2], dict(group=2, strides=[2, 2])),
    ("f16", [1, 16, 16, 32], [16, 200, 2, 2], dict(strides=[2, 2])),
]


@pytest.mark.parametrize("ci", range(len(TRANSPOSED_CASES)))
def test_transposed_route(ci):
    dtype, xs, ws, attrs = TRANSPOSED_CASES[ci]
    M = ws[1] * attrs.get("group", 1)
    h = B.Handle(dtype, xs, ws, None, None, transposed=True, **attrs)
    for k, (bias, resid) in enumerate([(True, True), (False, False), (True, False)]):
        act, params = ACTS[(3 * ci + 5 * k) % len(ACTS)]
        x, w, b, z = random_tensors([9500, ci, k], dtype, xs, ws, [M] if bias else None,
                                    h.y_shape if resid else None, dist="normal",
                                    w_std=1.0 / np.sqrt(ws[0]))
        a = dict(attrs, activation=act, activation_params=f32params(params))
        log(f"CASE transposed {ci} {h.kernel_name} x={xs} w={ws} {a} bias={bias} z={resid}")
        got = run_gpu(x, w, b, z, transposed=True, **a)
        ref = oracle.conv_transpose(x, w, b, z, **a)
        check(got, ref, dtype, f"transposed case {ci}")


def test_transposed_gemm_form_prepared_weights():
    # the GEMM form with weights prepared once and reused
    xs, ws = [2, 32, 6, 16], [32, 24, 2, 2]
    h = B.Handle("f16", xs, ws, [24], None, transposed=True, strides=[2, 2], activation="Relu")
    assert h.kernel_name.startswith("transposed_2x2s2_pointwise"), h.kernel_name
    x, w, b, _ = random_tensors([9510], "f16", xs, ws, [24], None, dist="normal")
    dx, dw, db = dev(x), dev(w), dev(b)
    y = torch.empty(h.y_shape, dtype=torch.float16, device="cuda")
    wsb = torch.empty(h.workspace_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    h.prepare_weights(dw.data_ptr(), wsb.data_ptr(), h.workspace_bytes, stream)
    ref = oracle.conv_transpose(x, w, b, strides=[2, 2], activation="Relu")
    outs = []
    for _ in range(2):
        y.zero_()
        h.run(dx.data_ptr(), dw.data_ptr(), db.data_ptr(), None, y.data_ptr(), wsb.data_ptr(),
              h.workspace_bytes, stream, flags=B.RUN_WEIGHTS_PREPARED)
        torch.cuda.synchronize()
        check(y.cpu().numpy(), ref, "f16", "transposed prepared")
        outs.append(y.clone())
    assert torch.equal(outs[0], outs[1]), "two runs with the same prepared weights differ"


# 3-D problems with one input plane and a one-tap kernel along depth but
# several output planes, or a leading depth pad: they must take a route that
# handles the depth axis (the planner keeps them off the 2-D-only kernels).
DEPTH_ONE_CASES = [
    ("f16", [2, 16, 1, 16, 16], [32, 16, 1, 2, 2], dict(strides=[1, 2, 2], pads=[0, 0, 0, 1, 0, 0])),
    ("f16", [2, 16, 1, 56, 56], [16, 1, 1, 7, 7], dict(group=16, pads=[0, 3, 3, 1, 3, 3])),
    ("f16", [2, 16, 1, 24, 32], [16, 1, 1, 7, 7], dict(group=16, pads=[1, 3, 3, 0, 3, 3])),
    ("f32", [2, 16, 1, 20, 20], [16, 1, 1, 3, 3], dict(group=16, pads=[0, 1, 1, 2, 1, 1])),
    ("f16", [2, 3, 1, 64, 64], [32, 3, 1, 7, 7], dict(strides=[1, 4, 4], pads=[0, 3, 3, 1, 3, 3])),
    ("f16", [2, 64, 1, 8, 8], [64, 64, 1, 1, 1], dict(pads=[0, 0, 0, 1, 0, 0])),
]


@pytest.mark.parametrize("ci", range(len(DEPTH_ONE_CASES)))
def test_depth_one_3d_problems(ci):
    dt, xs, ws, attrs = DEPTH_ONE_CASES[ci]
    h = B.Handle(dt, xs, ws, [ws[0]], None, **attrs)
    x, w, b, z = random_tensors([9600, ci], dt, xs, ws, [ws[0]], h.y_shape, dist="normal",
                                w_std=1.0 / np.sqrt(np.prod(ws[1:])))
    a = dict(attrs, activation="Relu")
    log(f"CASE depth one {ci} {h.kernel_name} x={xs} w={ws} {a}")
    got = run_gpu(x, w, b, z, **a)
    ref = reference(x, w, b, z, **a)
    check(got, ref, dt, f"depth one case {ci}")


def test_depth_one_transposed_with_depth_output_padding():
    xs, ws = [1, 32, 1, 8, 8], [32, 16, 1, 2, 2]
    attrs = dict(strides=[2, 2, 2], output_padding=[1, 0, 0])
    x, w, b, _ = random_tensors([9610], "f16", xs, ws, [16], None, dist="normal", w_std=0.2)
    log("CASE depth one transposed output_padding")
    got = run_gpu(x, w, b, None, transposed=True, **attrs)
    ref = oracle.conv_transpose(x, w, b, **attrs)
    check(got, ref, "f16", "depth one transposed")


def test_planned_call_rejects_mismatched_tensors():
    op = fc.FusedConv([2, 64, 16, 16], [96, 64, 3, 3], "f16", True, False, pads=[1, 1, 1, 1])
    x = torch.zeros(2, 64, 16, 16, dtype=torch.float16, device="cuda")
    w = torch.zeros(96, 64, 3, 3, dtype=torch.float16, device="cuda")
    b = torch.zeros(96, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        op(x, w, b, out=torch.empty(2, 96, 16, 15, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        op(x[:1], w, b)
    with pytest.raises(ValueError):
        op(x.float(), w, b)
    with pytest.raises(ValueError):
        op(x, w)                                   # bias planned, not given
    with pytest.raises(B.FusedConvError) as e:     # prepared weights need their workspace
        op(x, w, b, weights_prepared=True)
    assert e.value.status == "FUSEDCONV_ERR_WORKSPACE"
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.FusedConvError):
        op(x, w, b, workspace=small)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["cifar_resnet_conv3x3_f16", "conv1d_grouped_dil3_f32"])
def test_timed_run_matches_untimed(name):
    """fusedconv_run_timed computes what fusedconv_run computes, and the
    interval between its dispatch-recorded events is positive."""
    wl = WORKLOADS[name]
    inp = make_inputs(name)
    attrs = dict(wl["attrs"])
    attrs["activation_params"] = f32params(attrs.get("activation_params"))
    op = fc.FusedConv(wl["x"], wl["w"], wl["dtype"], wl["b"] is not None, wl["z"] is not None,
                      **attrs)
    t = {k: dev(v) for k, v in inp.items()}
    ws_t = torch.empty(max(op.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    log(f"CASE timed run {name} {op.handle.kernel_name}")
    y1 = op(t["x"], t["w"], t["b"], t["z"], workspace=ws_t)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()
    y2 = op(t["x"], t["w"], t["b"], t["z"], workspace=ws_t, events=ev)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    assert torch.equal(y1, y2)
    assert 0.0 < ms < 1000.0, ms
    h = op.handle
    with pytest.raises(B.FusedConvError) as e:   # one event alone is an error
        h.run(t["x"].data_ptr(), t["w"].data_ptr(), None if t["b"] is None else t["b"].data_ptr(),
              None if t["z"] is None else t["z"].data_ptr(), y2.data_ptr(), ws_t.data_ptr(),
              op.workspace_bytes, 0, events=(ev[0].cuda_event, None))
    assert e.value.status == "FUSEDCONV_ERR_NULL_ARG"
