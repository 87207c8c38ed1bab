"""Randomized GPU parity of the specialised routes against the oracle.

Seeded random problems for each route a planner may pick or a caller may
force: the fp16 and fp32 halo kernels (1-3-D, groups, strides, dilations,
every padding mode), SMALLC (few input channels, kernels 3-8, strides 1-4),
POINTWISE (1x1 and 2x2 stride-2, groups), the banded-MFMA depthwise kernel
(3x3 / 5x5 / 7x7, dilation 1-2), the explicit im2col route, and the
planner's own choice for fp16 and fp32.  A drawn problem that the forced
route does not take is skipped (its handle is refused on the host, before any
device call).  Every output is compared with the oracle by the parity
suite's rule (tests/test_parity_gpu.py: relative to max |Y_ref|, 1e-4 for
fp32 and 2e-2 for fp16; ThresholdedRelu outputs within the fp32 summation
bound of alpha may take either side).
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as fc
from convolution_implicit_gemm_amd import _binding as B
from oracle import oracle
from workloads import random_tensors

import test_parity_gpu as P

pytestmark = pytest.mark.gpu

KINDS = [("f32_halo", "f32", "igemm_halo"), ("f16_halo", "f16", "igemm_halo"),
         ("smallc", "f16", "smallc"), ("pointwise", "f16", "pointwise"),
         ("depthwise", "f16", "depthwise"), ("im2col", "f16", "im2col"),
         ("auto16", "f16", "auto"), ("auto32", "f32", "auto")]


def draw_problem(rng, kind):
    nsp = int(rng.integers(1, 4)) if kind in ("f32_halo", "f16_halo", "im2col", "auto16", "auto32") else 2
    g = int(rng.choice([1, 1, 2, 4]))
    if kind == "smallc":
        g, cg, mg = 1, int(rng.integers(1, 16)), int(rng.integers(8, 200))
    elif kind == "pointwise":
        g, cg, mg = int(rng.choice([1, 2])), 8 * int(rng.integers(2, 20)), int(rng.integers(8, 300))
    elif kind == "depthwise":
        g, cg, mg = int(rng.integers(1, 40)), 1, 1
    else:
        cg, mg = int(rng.integers(3, 70)), int(rng.integers(5, 150))
    if kind == "pointwise":
        ks = [1, 1] if rng.random() < 0.5 else [2, 2]
        ss = [1, 1] if ks[0] == 1 else [2, 2]
        ins = [2 * int(rng.integers(2, 20)), 8 * int(rng.integers(1, 12))]
        ds, mode, pads = [1, 1], "NOTSET", [0, 0, 0, 0]
    elif kind == "depthwise":
        k = int(rng.choice([3, 5, 7]))
        ks, ss = [k, k], [1, 1]
        ins = [int(rng.integers(5, 40)), 8 * int(rng.integers(1, 9))]
        ds, mode, pads = [int(rng.choice([1, 2]))] * 2, "SAME_UPPER", None
    elif kind == "smallc":
        k, s = int(rng.choice([3, 4, 7, 8])), int(rng.choice([1, 2, 4]))
        ks, ss = [k, k], [s, s]
        ins = [int(rng.integers(k, 70)), 8 * int(rng.integers(1, 12))]
        ds, mode, pads = [1, 1], "NOTSET", [int(v) for v in rng.integers(0, 4, 4)]
    else:
        ks = [int(v) for v in rng.integers(1, 4 if nsp > 1 else 10, nsp)]
        ins = [int(v) for v in rng.integers(4, 12 if nsp == 3 else (48 if nsp == 2 else 700), nsp)]
        if rng.random() < 0.5:
            ins[-1] = 4 * max(1, ins[-1] // 4)
        ss = [int(v) for v in rng.integers(1, 3, nsp)]
        ds = [int(v) for v in rng.integers(1, 3, nsp)]
        mode = str(rng.choice(["NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID"]))
        pads = [int(v) for v in rng.integers(0, 3, 2 * nsp)] if mode == "NOTSET" else None
        for i in range(nsp):
            ins[i] = max(ins[i], (ks[i] - 1) * ds[i] + 1)
    return dict(n=int(rng.integers(1, 4)), C=cg * g, M=mg * g, group=g, ks=ks, ins=ins,
                strides=ss, dilations=ds, auto_pad=mode, pads=pads)


@pytest.mark.parametrize("kind,dtype,route", KINDS, ids=[k[0] for k in KINDS])
def test_random_problems_on_route(kind, dtype, route):
    rng = np.random.default_rng([8800, len(kind), sum(map(ord, kind))])
    ran = 0
    for trial in range(60):
        c = draw_problem(rng, kind)
        act = P.ACTS[int(rng.integers(0, len(P.ACTS)))]
        bias, resid = bool(rng.random() < 0.7), bool(rng.random() < 0.5)
        xs = [c["n"], c["C"]] + c["ins"]
        ws = [c["M"], c["C"] // c["group"]] + c["ks"]
        attrs = dict(group=c["group"], strides=c["strides"], dilations=c["dilations"],
                     auto_pad=c["auto_pad"], pads=c["pads"], activation=act[0],
                     activation_params=P.f32params(act[1]))
        out = oracle.output_dims(c["ins"], c["ks"], c["strides"], c["dilations"], c["auto_pad"],
                                 c["pads"])
        if min(out[0]) <= 0:
            continue
        ys = [c["n"], c["M"]] + list(out[0])
        try:  # host only: the forced route may refuse the problem
            h = B.Handle(dtype, xs, ws, [c["M"]] if bias else None, ys if resid else None,
                         route=route, **attrs)
        except fc.FusedConvError:
            continue
        x, w, b, z = random_tensors([8801, len(kind), trial], dtype, xs, ws,
                                    [c["M"]] if bias else None, ys if resid else None,
                                    dist="normal" if dtype == "f16" else "uniform",
                                    w_std=1.0 / np.sqrt(int(np.prod(ws[1:]))) if dtype == "f16" else 1.0)
        what = f"{kind} {h.kernel_name} x={xs} w={ws} {attrs} bias={bias} z={resid}"
        P.log("CASE " + what)
        got = P.run_gpu(x, w, b, z, route=route, **attrs)
        P.check(got, P.reference(x, w, b, z, **attrs), dtype, what)
        ran += 1
    assert ran >= 10, f"{kind}: only {ran} problems ran"
