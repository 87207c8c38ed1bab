"""Pins for the oracle: every check here is independent of the oracle's own code.

Each test ties the oracle to something other than itself: brute-force
counting of window positions, closed forms (identity 1x1 kernel, single tap,
all-ones kernel = box sum via summed-area tables, delta input = kernel
readout), an explicit im2col-then-matmul formulation, PyTorch's float64
convolution and activation routines, and values printed on the pages
(tests/golden/).  A dropped term, a wrong sign or index, a flipped kernel or
a transposed operand in the oracle fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle
from workloads import WORKLOADS, random_tensors

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def setup_module(module):
    oracle.build(force=False)


# ----------------------------------------------------------------------------
# Output size and padding (FusedConv manifest.json derive: samePad*,
# effectivePad*, expectedOutput*; README "Attributes": auto_pad).
# ----------------------------------------------------------------------------

def _count_windows(inp, k, s, d, pb, pe):
    """Brute force: number of window starts o*s (o >= 0) whose dilated window
    fits inside the padded axis of length inp + pb + pe."""
    span = (k - 1) * d + 1
    n = 0
    while n * s + span <= inp + pb + pe:
        n += 1
    return n


def test_output_size_notset_and_valid_bruteforce():
    rng = np.random.default_rng(7)
    checked = 0
    for inp, k, s, d in itertools.product(range(1, 21), range(1, 8), range(1, 5), range(1, 4)):
        pb, pe = (int(v) for v in rng.integers(0, 4, size=2))
        expect = _count_windows(inp, k, s, d, pb, pe)
        got = oracle.output_dims([inp], [k], [s], [d], "NOTSET", [pb, pe])
        if expect == 0:
            assert got is None
        else:
            assert got == ([expect], [pb])
        expect_v = _count_windows(inp, k, s, d, 0, 0)
        got_v = oracle.output_dims([inp], [k], [s], [d], "VALID", None)
        if expect_v == 0:
            assert got_v is None
        else:
            assert got_v == ([expect_v], [0])
        checked += 1
    assert checked == 20 * 7 * 4 * 3


@pytest.mark.parametrize("mode", ["SAME_UPPER", "SAME_LOWER"])
def test_output_size_same_invariants(mode):
    for inp, k, s, d in itertools.product(range(1, 21), range(1, 8), range(1, 5), range(1, 4)):
        got = oracle.output_dims([inp], [k], [s], [d], mode, None)
        assert got is not None
        (out,), (pb,) = got
        # each output is one stride step: out = ceil(in / s), found by counting
        assert out == sum(1 for start in range(0, inp, s))
        # the minimal total pad that lets the last window fit, by search
        total = 0
        while (out - 1) * s + (k - 1) * d + 1 > inp + total:
            total += 1
        pe = total - pb
        assert 0 <= pb and 0 <= pe and abs(pb - pe) <= 1
        if mode == "SAME_UPPER":
            assert pe >= pb
        else:
            assert pb >= pe
        # with these pads the explicit-pad rule gives the same count
        assert _count_windows(inp, k, s, d, pb, pe) == out


def test_readme_example_shape():
    rows = dict((ln.split()[0], [int(v) for v in ln.split()[1:]])
                for ln in open(os.path.join(GOLDEN, "readme_example.txt"))
                if ln.strip() and not ln.startswith("#"))
    x, w, y = rows["x"], rows["w"], rows["y"]
    out, _ = oracle.output_dims(x[2:], w[2:])
    assert [x[0], w[0]] + out == y


def test_workload_shapes():
    for name, wl in WORKLOADS.items():
        a = wl["attrs"]
        if a.get("transposed"):
            # the transposed oracle's own shape on a zero input of the workload's size
            y = oracle.conv_transpose(np.zeros([1] + wl["x"][1:]), np.zeros(wl["w"]),
                                      strides=a.get("strides"), dilations=a.get("dilations"),
                                      pads=a.get("pads"), output_padding=a.get("output_padding"))
            assert [wl["x"][0]] + list(y.shape[1:]) == wl["y"], name
            continue
        got = oracle.output_dims(wl["x"][2:], wl["w"][2:], a.get("strides"), a.get("dilations"),
                                 a.get("auto_pad", "NOTSET"), a.get("pads"))
        assert got is not None, name
        assert [wl["x"][0], wl["w"][0]] + got[0] == wl["y"], name


# ----------------------------------------------------------------------------
# Activations (README "Attributes"; manifest derive actAlpha/actBeta).
# Library routines and special values, never a retyped formula.
# ----------------------------------------------------------------------------

V = np.concatenate([np.linspace(-8, 8, 401), [-30.0, -12.5, 0.0, 1e-6, -1e-6, 12.5, 30.0]])
T = torch.tensor(V, dtype=torch.float64)


def _act(name, params=None):
    return oracle.activation(name, V, params)


def test_activation_library_routines():
    close = dict(rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(_act("Relu"), torch.relu(T).numpy(), **close)
    np.testing.assert_allclose(_act("LeakyRelu", [0.1]), F.leaky_relu(T, 0.1).numpy(), **close)
    np.testing.assert_allclose(_act("Sigmoid"), torch.sigmoid(T).numpy(), **close)
    np.testing.assert_allclose(_act("Tanh"), np.array([math.tanh(v) for v in V]), **close)
    np.testing.assert_allclose(_act("HardSigmoid", [1 / 6, 0.5]), F.hardsigmoid(T).numpy(), **close)
    np.testing.assert_allclose(_act("HardSwish"), F.hardswish(T).numpy(), **close)
    np.testing.assert_allclose(_act("Clip", [-0.5, 2.0]), torch.clamp(T, -0.5, 2.0).numpy(), **close)
    np.testing.assert_allclose(_act("QuickGelu", [1.0]), F.silu(T).numpy(), **close)
    np.testing.assert_allclose(_act("Elu", [0.7]), F.elu(T, 0.7).numpy(), **close)
    np.testing.assert_allclose(_act("Gelu"), F.gelu(T).numpy(), **close)
    np.testing.assert_allclose(_act("Gelu", [1.0]), F.gelu(T, approximate="tanh").numpy(), **close)
    np.testing.assert_allclose(_act("FastGelu"), F.gelu(T, approximate="tanh").numpy(), **close)
    sp = F.softplus(T, beta=1.0, threshold=1e9).numpy()
    np.testing.assert_allclose(_act("Softplus"), sp, **close)
    np.testing.assert_allclose(_act("ThresholdedRelu", [0.75]), F.threshold(T, 0.75, 0.0).numpy(),
                               **close)
    np.testing.assert_allclose(_act("Erf"), np.array([math.erf(v) for v in V]), **close)
    np.testing.assert_array_equal(oracle.activation(None, V), V)


def test_activation_special_values():
    assert oracle.activation("HardSwish", [-3.0, 3.0, 0.0]).tolist() == [0.0, 3.0, 0.0]
    assert oracle.activation("Softplus", [0.0])[0] == pytest.approx(math.log(2.0), abs=1e-15)
    assert oracle.activation("Erf", [0.0])[0] == 0.0
    assert oracle.activation("Sigmoid", [0.0])[0] == 0.5
    # ThresholdedRelu passes only values strictly above alpha
    assert oracle.activation("ThresholdedRelu", [1.0, 1.0 + 1e-12], [1.0]).tolist() == [0.0, 1.0 + 1e-12]
    # HardSigmoid saturates at 0 and 1
    assert oracle.activation("HardSigmoid", [-100.0, 100.0], [0.2, 0.5]).tolist() == [0.0, 1.0]
    # Gelu(x) - Gelu(-x) = x for the erf form, since Phi(x) + Phi(-x) = 1
    g = oracle.activation("Gelu", V) - oracle.activation("Gelu", -V)
    np.testing.assert_allclose(g, V, atol=1e-13)


def test_quickgelu_exp2_constant_golden():
    vals = dict(ln.split() for ln in open(os.path.join(GOLDEN, "quickgelu_exp2_constant.txt"))
                if ln.strip() and not ln.startswith("#"))
    alpha, c = float(vals["alpha"]), float(vals["alpha_log2e"])
    expect = V / (1.0 + np.power(2.0, -c * V))
    np.testing.assert_allclose(_act("QuickGelu", [alpha]), expect, rtol=1e-14, atol=1e-15)


def test_activation_defaults_golden():
    for ln in open(os.path.join(GOLDEN, "activation_defaults.txt")):
        if not ln.strip() or ln.startswith("#"):
            continue
        name, a, b = ln.split()
        a, b = float(a), float(b)
        explicit = [a, b] if name == "HardSigmoid" else [a]
        np.testing.assert_array_equal(oracle.activation(name, V), oracle.activation(name, V, explicit))
    # defaults agree with the library's own defaults where it has one
    np.testing.assert_allclose(_act("LeakyRelu"), F.leaky_relu(T).numpy(), rtol=1e-12)
    np.testing.assert_allclose(_act("Elu"), F.elu(T).numpy(), rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------
# Convolution core.
# ----------------------------------------------------------------------------

def _torch_ref(x, w, b, z, group, strides, dilations, pad_begin, pad_end, act, params):
    """PyTorch float64: F.pad with the resolved pads, then F.conv{1,2,3}d, + B + Z, act."""
    nsp = x.ndim - 2
    xt = torch.tensor(x.astype(np.float64))
    wt = torch.tensor(w.astype(np.float64))
    padarg = []
    for i in reversed(range(nsp)):
        padarg += [pad_begin[i], pad_end[i]]
    xt = F.pad(xt, padarg)
    conv = {1: F.conv1d, 2: F.conv2d, 3: F.conv3d}[nsp]
    y = conv(xt, wt, None, stride=strides, dilation=dilations, groups=group)
    if b is not None:
        y = y + torch.tensor(b.astype(np.float64)).reshape([1, -1] + [1] * nsp)
    if z is not None:
        y = y + torch.tensor(z.astype(np.float64))
    return oracle.activation(act, y.numpy(), params) if act else y.numpy()


def _resolved(x_shape, w_shape, strides, dilations, auto_pad, pads):
    nsp = len(x_shape) - 2
    res = oracle.output_dims(x_shape[2:], w_shape[2:], strides, dilations, auto_pad, pads)
    assert res is not None
    out, pb = res
    # end pads that make F.pad + a VALID conv produce exactly `out` outputs
    pe = [(out[i] - 1) * strides[i] + (w_shape[2 + i] - 1) * dilations[i] + 1 - x_shape[2 + i] - pb[i]
          for i in range(nsp)]
    return out, pb, pe


def _random_case(rng, nsp):
    group = int(rng.choice([1, 2, 3]))
    cg, mg = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    n = int(rng.integers(1, 3))
    ks = [int(v) for v in rng.integers(1, 4, size=nsp)]
    ins = [int(v) for v in rng.integers(3, 9, size=nsp)]
    strides = [int(v) for v in rng.integers(1, 3, size=nsp)]
    dil = [int(v) for v in rng.integers(1, 3, size=nsp)]
    mode = str(rng.choice(["NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID"]))
    pads = [int(v) for v in rng.integers(0, 3, size=2 * nsp)] if mode == "NOTSET" else None
    for i in range(nsp):  # keep the output size positive
        ins[i] = max(ins[i], (ks[i] - 1) * dil[i] + 1)
    return dict(n=n, group=group, C=cg * group, M=mg * group, ks=ks, ins=ins, strides=strides,
                dil=dil, mode=mode, pads=pads)


@pytest.mark.parametrize("nsp", [1, 2, 3])
def test_conv_matches_torch_float64(nsp):
    rng = np.random.default_rng(100 + nsp)
    acts = [None, "Relu", ("LeakyRelu", [0.2]), "Sigmoid", "Tanh", ("HardSigmoid", [0.3, 0.4]),
            "HardSwish", ("Clip", [-0.5, 0.5]), "QuickGelu", "Elu", "Gelu", ("Gelu", [1.0]),
            "FastGelu", "Softplus", "ThresholdedRelu", "Erf"]
    for trial in range(16):
        c = _random_case(rng, nsp)
        x_shape = [c["n"], c["C"]] + c["ins"]
        w_shape = [c["M"], c["C"] // c["group"]] + c["ks"]
        out, pb, pe = _resolved(x_shape, w_shape, c["strides"], c["dil"], c["mode"], c["pads"])
        y_shape = [c["n"], c["M"]] + out
        x, w, b, z = random_tensors([5, nsp, trial], "f32", x_shape, w_shape, [c["M"]], y_shape)
        if trial % 4 == 1:
            b = None
        if trial % 4 == 2:
            z = None
        a = acts[trial % len(acts)]
        act, params = (a if isinstance(a, tuple) else (a, None))
        got = oracle.fusedconv(x, w, b, z, group=c["group"], strides=c["strides"],
                               dilations=c["dil"], auto_pad=c["mode"], pads=c["pads"],
                               activation=act, activation_params=params)
        ref = _torch_ref(x, w, b, z, c["group"], c["strides"], c["dil"], pb, pe, act, params)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def _im2col_matmul(x, w, group, strides, dil, pb, out):
    """Explicit im2col on a zero-padded copy of X, then one matmul per group."""
    nsp = x.ndim - 2
    n, C = x.shape[:2]
    M = w.shape[0]
    ks = list(w.shape[2:])
    cg, mg = C // group, M // group
    hi = [pb[i] + (out[i] - 1) * strides[i] + (ks[i] - 1) * dil[i] + 1 for i in range(nsp)]
    xp = np.zeros([n, C] + [max(hi[i], pb[i] + x.shape[2 + i]) for i in range(nsp)])
    xp[(slice(None), slice(None)) + tuple(slice(pb[i], pb[i] + x.shape[2 + i]) for i in range(nsp))] = x
    taps = list(itertools.product(*[range(k) for k in ks]))
    cols = np.zeros([n, C, len(taps), int(np.prod(out))])
    for ti, t in enumerate(taps):
        sl = tuple(slice(t[i] * dil[i], t[i] * dil[i] + (out[i] - 1) * strides[i] + 1, strides[i])
                   for i in range(nsp))
        cols[:, :, ti, :] = xp[(slice(None), slice(None)) + sl].reshape(n, C, -1)
    y = np.zeros([n, M, int(np.prod(out))])
    for g in range(group):
        a = w[g * mg:(g + 1) * mg].reshape(mg, cg * len(taps)).astype(np.float64)
        bmat = cols[:, g * cg:(g + 1) * cg].reshape(n, cg * len(taps), -1)
        y[:, g * mg:(g + 1) * mg] = np.einsum("mk,nkp->nmp", a, bmat)
    return y.reshape([n, M] + out)


@pytest.mark.parametrize("nsp", [1, 2, 3])
def test_conv_matches_explicit_im2col(nsp):
    rng = np.random.default_rng(200 + nsp)
    for trial in range(12):
        c = _random_case(rng, nsp)
        x_shape = [c["n"], c["C"]] + c["ins"]
        w_shape = [c["M"], c["C"] // c["group"]] + c["ks"]
        out, pb, pe = _resolved(x_shape, w_shape, c["strides"], c["dil"], c["mode"], c["pads"])
        x, w, _, _ = random_tensors([6, nsp, trial], "f16", x_shape, w_shape)
        got = oracle.fusedconv(x, w, group=c["group"], strides=c["strides"], dilations=c["dil"],
                               auto_pad=c["mode"], pads=c["pads"])
        ref = _im2col_matmul(x.astype(np.float64), w, c["group"], c["strides"], c["dil"], pb, out)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_identity_1x1_kernel():
    """W[m, c] = delta(m, c): Y = act(X subsampled by the stride + B + Z)."""
    x, _, b, _ = random_tensors([7, 0], "f32", [2, 5, 9, 11], [5, 5, 1, 1], [5])
    w = np.eye(5, dtype=np.float32).reshape(5, 5, 1, 1)
    for s in ([1, 1], [2, 3]):
        y_sub = x[:, :, ::s[0], ::s[1]].astype(np.float64)
        z = np.random.default_rng(8).uniform(-1, 1, y_sub.shape).astype(np.float32)
        got = oracle.fusedconv(x, w, b, z, strides=s, activation="Tanh")
        np.testing.assert_allclose(got, np.tanh(y_sub + b.reshape(1, 5, 1, 1) + z), rtol=1e-14)


@pytest.mark.parametrize("mode,pads", [("NOTSET", [2, 1, 0, 3]), ("SAME_UPPER", None),
                                       ("SAME_LOWER", None), ("VALID", None)])
def test_single_tap_depthwise_is_shifted_copy(mode, pads):
    """group = C = M, one nonzero tap t per channel: Y[n,m,o] = X[n,m,o*s - p + t*d] (0 outside)."""
    C, k, s, d = 4, [3, 4], [2, 1], [2, 3]
    x, _, _, _ = random_tensors([9, 0], "f32", [2, C, 10, 13], [C, 1] + k)
    for tap in [(0, 0), (2, 3), (1, 2)]:
        w = np.zeros([C, 1] + k, np.float32)
        w[:, 0, tap[0], tap[1]] = 1.0
        got = oracle.fusedconv(x, w, group=C, strides=s, dilations=d, auto_pad=mode, pads=pads)
        out, pb = oracle.output_dims([10, 13], k, s, d, mode, pads)
        ref = np.zeros([2, C] + out)
        for oh in range(out[0]):
            for ow in range(out[1]):
                ih = oh * s[0] - pb[0] + tap[0] * d[0]
                iw = ow * s[1] - pb[1] + tap[1] * d[1]
                if 0 <= ih < 10 and 0 <= iw < 13:
                    ref[:, :, oh, ow] = x[:, :, ih, iw]
        np.testing.assert_array_equal(got, ref)


def _box_sum_sat(x, k, s, d, pb, out):
    """All-ones kernel over all channels, by summed-area tables per dilation residue."""
    n, C, H, W = x.shape
    xc = x.astype(np.float64).sum(axis=1)  # sum over channels first
    Hp = max(pb[0] + H, (out[0] - 1) * s[0] + (k[0] - 1) * d[0] + 1)
    Wp = max(pb[1] + W, (out[1] - 1) * s[1] + (k[1] - 1) * d[1] + 1)
    xp = np.zeros([n, Hp, Wp])
    xp[:, pb[0]:pb[0] + H, pb[1]:pb[1] + W] = xc
    y = np.zeros([n, out[0], out[1]])
    for oh in range(out[0]):
        for ow in range(out[1]):
            h0, w0 = oh * s[0], ow * s[1]
            sub = xp[:, h0 % d[0]::d[0], w0 % d[1]::d[1]]
            sat = np.zeros([n, sub.shape[1] + 1, sub.shape[2] + 1])
            sat[:, 1:, 1:] = sub.cumsum(1).cumsum(2)
            a, c = h0 // d[0], w0 // d[1]
            y[:, oh, ow] = sat[:, a + k[0], c + k[1]] - sat[:, a, c + k[1]] - sat[:, a + k[0], c] + sat[:, a, c]
    return y


@pytest.mark.parametrize("mode,pads,s,d", [("NOTSET", [1, 2, 3, 0], [1, 1], [1, 1]),
                                           ("SAME_UPPER", None, [2, 1], [1, 2]),
                                           ("SAME_LOWER", None, [1, 3], [3, 1]),
                                           ("VALID", None, [2, 2], [2, 2])])
def test_all_ones_kernel_is_box_sum(mode, pads, s, d):
    k = [3, 4]
    x, _, _, _ = random_tensors([10, 0], "f32", [2, 3, 12, 14], [2, 3] + k)
    w = np.ones([2, 3] + k, np.float32)
    got = oracle.fusedconv(x, w, strides=s, dilations=d, auto_pad=mode, pads=pads)
    out, pb = oracle.output_dims([12, 14], k, s, d, mode, pads)
    ref = _box_sum_sat(x, k, s, d, pb, out)
    for m in range(2):
        np.testing.assert_allclose(got[:, m], ref, rtol=1e-12, atol=1e-12)


def test_delta_input_reads_out_the_kernel():
    """X = e(n0, c0, p0): each output is one kernel weight or 0 (no flip, group mapping, pads)."""
    group, cg, mg = 2, 3, 2
    C, M, k, s, d = cg * group, mg * group, [3, 2], [2, 1], [1, 2]
    pads = [1, 2, 0, 1]
    _, w, _, _ = random_tensors([11, 0], "f32", [1, C, 7, 6], [M, cg] + k)
    out, pb = oracle.output_dims([7, 6], k, s, d, "NOTSET", pads)
    for n0, c0, p0 in [(1, 4, (3, 2)), (0, 0, (0, 0)), (1, 2, (6, 5))]:
        x = np.zeros([2, C, 7, 6], np.float32)
        x[n0, c0, p0[0], p0[1]] = 1.0
        got = oracle.fusedconv(x, w, group=group, strides=s, dilations=d, pads=pads)
        ref = np.zeros([2, M] + out)
        g = c0 // cg
        for m in range(g * mg, (g + 1) * mg):
            for oh in range(out[0]):
                for ow in range(out[1]):
                    th, tw = p0[0] + pb[0] - oh * s[0], p0[1] + pb[1] - ow * s[1]
                    if th % d[0] == 0 and tw % d[1] == 0 and 0 <= th // d[0] < k[0] \
                            and 0 <= tw // d[1] < k[1]:
                        ref[n0, m, oh, ow] = w[m, c0 - g * cg, th // d[0], tw // d[1]]
        np.testing.assert_array_equal(got, ref)


def test_zero_weights_isolate_epilogue():
    x, _, b, z = random_tensors([12, 0], "f16", [2, 4, 6, 5], [6, 2, 3, 3], [6], [2, 6, 6, 5])
    w = np.zeros([6, 2, 3, 3], np.float16)
    pre = b.astype(np.float64).reshape(1, 6, 1, 1) + z.astype(np.float64)
    for act, params, fn in [("Relu", None, torch.relu), ("Softplus", None, F.softplus),
                            ("Elu", [0.5], lambda t: F.elu(t, 0.5)), (None, None, lambda t: t)]:
        got = oracle.fusedconv(x, w, b, z, group=2, auto_pad="SAME_LOWER", activation=act,
                               activation_params=params)
        np.testing.assert_allclose(got, fn(torch.tensor(pre)).numpy(), rtol=1e-12, atol=1e-14)
    # bias alone and residual alone
    got = oracle.fusedconv(x, w, b, None, group=2, auto_pad="SAME_LOWER")
    np.testing.assert_array_equal(got, np.broadcast_to(b.astype(np.float64).reshape(1, 6, 1, 1), got.shape))
    got = oracle.fusedconv(x, w, None, z, group=2, auto_pad="SAME_LOWER")
    np.testing.assert_array_equal(got, z.astype(np.float64))


def test_points_match_full_output():
    x, w, b, z = random_tensors([13, 0], "f32", [2, 4, 5, 6, 7], [4, 2, 2, 3, 2], [4], [2, 4, 3, 3, 7])
    kw = dict(group=2, strides=[2, 2, 1], pads=[1, 0, 1, 0, 1, 0], activation="Gelu")
    full = oracle.fusedconv(x, w, b, z, **kw)
    assert list(full.shape) == [2, 4, 3, 3, 7]
    idx = np.random.default_rng(1).integers(0, full.size, 300)
    np.testing.assert_array_equal(oracle.fusedconv_at(x, w, b, z, idx=idx, **kw), full.ravel()[idx])
    part = oracle.fusedconv(x, w, b, z, batches=(1, 2), **kw)
    np.testing.assert_array_equal(part, full[1:2])


# ---- transposed convolution (oracle.conv_transpose) ------------------------

CONVT_CASES = [
    # (x shape, w shape [C, M/group, k...], attrs)
    ([2, 4, 5, 6], [4, 3, 3, 2], dict(strides=[2, 3], pads=[1, 0, 2, 1], dilations=[1, 2],
                                      output_padding=[1, 2])),
    ([1, 6, 7], [6, 2, 4], dict(group=3, strides=[2], pads=[1, 2])),
    ([2, 4, 3, 4, 3], [4, 2, 2, 3, 2], dict(group=2, strides=[1, 2, 2], pads=[0, 1, 0, 1, 0, 1],
                                           output_padding=[0, 1, 1])),
    ([1, 3, 4, 4], [3, 5, 2, 2], dict(strides=[2, 2])),                     # patch upsampling
    ([2, 2, 6], [2, 3, 3], dict(dilations=[3], pads=[2, 1])),
]


def _torch_convt(x, w, group=1, strides=None, dilations=None, pads=None, output_padding=None):
    """torch's CPU conv_transpose in float64 (symmetric-pad API): run it without
    padding, then cut [pad_begin, full - pad_end + output_padding), zero past
    the full extent (where output padding reaches beyond every tap)."""
    nsp = x.ndim - 2
    f = {1: F.conv_transpose1d, 2: F.conv_transpose2d, 3: F.conv_transpose3d}[nsp]
    full = f(torch.from_numpy(x), torch.from_numpy(w), stride=strides or [1] * nsp,
             dilation=dilations or [1] * nsp, groups=group).numpy()
    p = pads or [0] * (2 * nsp)
    op = output_padding or [0] * nsp
    out = [full.shape[2 + i] - p[i] - p[nsp + i] + op[i] for i in range(nsp)]
    y = np.zeros(list(full.shape[:2]) + out)
    src = tuple(slice(p[i], min(full.shape[2 + i], p[i] + out[i])) for i in range(nsp))
    cut = full[(slice(None), slice(None)) + src]
    y[(slice(None), slice(None)) + tuple(slice(0, c) for c in cut.shape[2:])] = cut
    return y


@pytest.mark.parametrize("ci", range(len(CONVT_CASES)))
def test_conv_transpose_matches_torch_fp64(ci):
    xs, ws, kw = CONVT_CASES[ci]
    rng = np.random.default_rng([700, ci])
    x, w = rng.standard_normal(xs), rng.standard_normal(ws)
    np.testing.assert_allclose(oracle.conv_transpose(x, w, **kw), _torch_convt(x, w, **kw),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("ci", range(len(CONVT_CASES)))
def test_conv_transpose_is_the_adjoint_of_the_conv(ci):
    # <convT(x; W), y> = <x, conv(y; W)> with W read as a [C, M/group, k] conv weight
    xs, ws, kw = CONVT_CASES[ci]
    rng = np.random.default_rng([701, ci])
    x, w = rng.standard_normal(xs), rng.standard_normal(ws)
    yt = oracle.conv_transpose(x, w, **kw)
    y = rng.standard_normal(yt.shape)
    fw = {k: v for k, v in kw.items() if k in ("group", "strides", "dilations", "pads")}
    back = oracle.fusedconv(y, w, **fw)
    assert back.shape == x.shape
    lhs, rhs = float(np.sum(yt * y)), float(np.sum(x * back))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_conv_transpose_1x1_is_zero_insertion_upsampling():
    rng = np.random.default_rng(702)
    x, w = rng.standard_normal([2, 5, 3, 4]), rng.standard_normal([5, 6, 1, 1])
    y = oracle.conv_transpose(x, w, strides=[3, 2], output_padding=[1, 1])
    assert y.shape == (2, 6, 8, 8)
    ref = np.zeros(y.shape)
    ref[:, :, ::3, ::2][:, :, :3, :4] = np.einsum("ncij,cm->nmij", x, w[:, :, 0, 0])
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


def test_conv_transpose_epilogue():
    rng = np.random.default_rng(703)
    x, w = rng.standard_normal([1, 4, 3, 3]), rng.standard_normal([4, 2, 2, 2])
    b = rng.standard_normal([2])
    core = oracle.conv_transpose(x, w, strides=[2, 2])
    z = rng.standard_normal(core.shape)
    y = oracle.conv_transpose(x, w, b, z, strides=[2, 2], activation="LeakyRelu",
                              activation_params=[0.1])
    pre = core + b.reshape(1, 2, 1, 1) + z
    np.testing.assert_allclose(y, np.where(pre >= 0, pre, 0.1 * pre), rtol=0, atol=1e-13)
