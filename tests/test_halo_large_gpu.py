"""GPU parity of the fp16 halo route at large shapes, whole tensors.

Problems of a few hundred images with 128-256 channels run the halo kernel
in the launch shape of the benchmark (two blocks per CU, two rounds of
blocks); every output element is compared with the oracle to the fp16 bar
of the parity suite (max |Y - Y_ref| <= 2e-2 * max |Y_ref|, Y_ref the
oracle's float64 result).  The cases: image-sized tiles, four tiles per
image (boxes with different image borders), ragged output tiles and
channel blocks, groups, dilation, asymmetric padding, eight channel blocks,
and every activation at the headline shape -- ThresholdedRelu's jump is
decided on the kernel's fp32 sum, so outputs whose float64 pre-activation
lies within the kernel's error of alpha may take either side and are
checked to be one of the two.
"""
import sys

import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as fc
from convolution_implicit_gemm_amd import _binding as B
from oracle import oracle
from workloads import random_tensors

pytestmark = pytest.mark.gpu
TAU = 2e-2


def log(msg):
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    fc.load()
    oracle.build(force=False)


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def f32params(p):
    return None if p is None else [float(np.float32(v)) for v in p]


CASES = [
    # (id, x shape, w shape, bias, residual, attrs)
    ("image_tiles", [256, 128, 16, 16], [256, 128, 3, 3], False, True,
     dict(pads=[1, 1, 1, 1], activation="QuickGelu", activation_params=[1.702])),
    ("four_tiles_per_image", [128, 128, 32, 32], [128, 128, 3, 3], True, True,
     dict(pads=[1, 1, 1, 1], activation="Relu")),
    ("ragged_channel_block", [256, 128, 16, 16], [200, 128, 3, 3], True, False,
     dict(pads=[1, 1, 1, 1], activation="Tanh")),
    ("ragged_tiles_uneven_units", [192, 128, 24, 24], [128, 128, 3, 3], True, True,
     dict(pads=[1, 1, 1, 1], activation="Sigmoid")),
    ("dilated", [256, 128, 16, 16], [256, 128, 3, 3], False, True,
     dict(pads=[2, 2, 2, 2], dilations=[2, 2], activation="Gelu")),
    ("grouped", [256, 256, 16, 16], [256, 128, 3, 3], True, True,
     dict(group=2, pads=[1, 1, 1, 1], activation="HardSwish")),
    ("eight_channel_blocks", [512, 256, 16, 16], [128, 256, 3, 3], True, False,
     dict(pads=[1, 1, 1, 1], activation="Elu", activation_params=[0.8])),
    ("asymmetric_pads", [256, 128, 16, 16], [256, 128, 3, 3], True, True,
     dict(pads=[0, 2, 2, 0])),
]


def compare(got, x, w, b, z, attrs, what):
    """Whole tensor against the oracle, a few images at a time."""
    n = x.shape[0]
    per = max(1, (1 << 24) // int(np.prod(got.shape[1:])))
    max_err = max_ref = 0.0
    for n0 in range(0, n, per):
        n1 = min(n, n0 + per)
        zi = z[n0:n1] if z is not None else None
        ref = oracle.fusedconv(x[n0:n1], w, b, zi, **attrs)
        max_err = max(max_err, float(np.max(np.abs(got[n0:n1].astype(np.float64) - ref))))
        max_ref = max(max_ref, float(np.max(np.abs(ref))))
    rel = max_err / max(max_ref, 1e-30)
    log(f"RESULT {what}: rel err {rel:.3e}")
    assert rel <= TAU, f"{what}: rel err {rel:.3e} > {TAU}"
    return rel


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
def test_halo_large(ci):
    name, xs, ws, has_b, has_z, attrs = CASES[ci]
    attrs = dict(attrs)
    attrs["activation_params"] = f32params(attrs.get("activation_params"))
    kw = {k: v for k, v in attrs.items() if v is not None}
    out = oracle.output_dims(xs[2:], ws[2:], attrs.get("strides"), attrs.get("dilations"),
                             "NOTSET", attrs.get("pads"))
    ys = [xs[0], ws[0]] + out[0]
    h = B.Handle("f16", xs, ws, [ws[0]] if has_b else None, ys if has_z else None, **kw)
    assert h.route == "igemm_halo", (h.route, h.kernel_name)
    x, w, b, z = random_tensors([7100, ci], "f16", xs, ws, [ws[0]] if has_b else None,
                                ys if has_z else None, dist="normal",
                                w_std=1.0 / np.sqrt(ws[1] * 9))
    log(f"CASE halo {name} {h.kernel_name} x={xs} w={ws} bias={has_b} z={has_z} {kw}")
    got = fc.fused_conv(dev(x), dev(w), dev(b), dev(z), **kw)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.all(np.isfinite(got)), name
    compare(got, x, w, b, z, kw, name)


ACTS = [(None, None), ("Relu", None), ("LeakyRelu", [0.1]), ("Sigmoid", None), ("Tanh", None),
        ("HardSigmoid", [0.2, 0.5]), ("HardSwish", None), ("Clip", [-0.5, 1.5]),
        ("QuickGelu", [1.702]), ("Elu", [0.8]), ("Gelu", None), ("Gelu", [1.0]),
        ("FastGelu", None), ("Softplus", None), ("ThresholdedRelu", [0.3]), ("Erf", None)]


def test_halo_large_every_activation():
    """One problem, every activation: the pre-activation sum comes from the
    oracle once, each activation is the oracle's activation of it."""
    xs, ws = [256, 128, 16, 16], [256, 128, 3, 3]
    x, w, b, z = random_tensors([7200], "f16", xs, ws, [256], [256, 256, 16, 16], dist="normal",
                                w_std=1.0 / np.sqrt(128 * 9))
    pre = oracle.fusedconv(x, w, b, z, pads=[1, 1, 1, 1])
    for name, params in ACTS:
        p = f32params(params)
        kw = dict(pads=[1, 1, 1, 1], activation=name, activation_params=p)
        kw = {k: v for k, v in kw.items() if v is not None}
        h = B.Handle("f16", xs, ws, [256], [256, 256, 16, 16], **kw)
        assert h.route == "igemm_halo", (h.route, h.kernel_name)
        log(f"CASE halo activation {name} {p}")
        got = fc.fused_conv(dev(x), dev(w), dev(b), dev(z), **kw)
        torch.cuda.synchronize()
        got = got.cpu().numpy().astype(np.float64)
        ref = pre if name is None else oracle.activation(name, pre, p)
        scale = max(np.max(np.abs(ref)), 1e-30)
        if name == "ThresholdedRelu":
            # the jump at alpha is decided on the kernel's own sum; where the
            # float64 sum lies within the kernel's error of alpha either side
            # is correct: there the output must be 0 or the pre-activation
            amb = np.abs(pre - p[0]) <= 1e-3 * np.max(np.abs(pre))
            okv = (np.abs(got) <= TAU * scale) | (np.abs(got - pre) <= TAU * scale)
            assert np.all(okv[amb]), "ThresholdedRelu: invalid output near alpha"
            log(f"ThresholdedRelu: {int(amb.sum())} outputs within the decision band")
            got, ref = got[~amb], ref[~amb]
        rel = float(np.max(np.abs(got - ref)) / scale)
        log(f"RESULT activation {name}: rel err {rel:.3e}")
        assert rel <= TAU, f"{name}: rel err {rel:.3e}"


def test_halo_large_prepared_weights_and_repeats():
    """Prepared weights and a plain run give identical bits, and so do two
    runs in a row, at the launch shape of the benchmark."""
    xs, ws = [256, 128, 16, 16], [256, 128, 3, 3]
    x, w, b, z = random_tensors([7300], "f16", xs, ws, [256], [256, 256, 16, 16], dist="normal",
                                w_std=1.0 / np.sqrt(128 * 9))
    kw = dict(pads=[1, 1, 1, 1], activation="QuickGelu", activation_params=[1.702])
    h = B.Handle("f16", xs, ws, [256], [256, 256, 16, 16], **kw)
    assert h.route == "igemm_halo", (h.route, h.kernel_name)
    xd, wd, bd, zd = dev(x), dev(w), dev(b), dev(z)
    op = fc.FusedConv(xs, ws, "f16", True, True, **kw)
    wsp = torch.empty(max(op.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    y1 = op(xd, wd, bd, zd, workspace=wsp)
    y2 = op(xd, wd, bd, zd, workspace=wsp)
    op.prepare_weights(wd, wsp)
    y3 = op(xd, wd, bd, zd, workspace=wsp, weights_prepared=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1, y3)
    ref = oracle.fusedconv(x, w, b, z, **kw)
    rel = float(np.max(np.abs(y1.cpu().numpy().astype(np.float64) - ref)) / np.max(np.abs(ref)))
    assert rel <= TAU, rel
