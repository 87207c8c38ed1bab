"""Error bounds of the kernels' fast activation forms (CPU, no GPU).

The epilogues evaluate erf (Erf, and Gelu's erf form) with Abramowitz &
Stegun, Handbook of Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7),
tanh (FastGelu, Tanh) as 1 - 2 / (1 + e^(2x)), and the SMALLC kernel Gelu /
Erf by linear interpolation in a table of the normal CDF.  These tests take
the constants from the kernel sources themselves (csrc/epilogue.h,
csrc/kernels_smallc.hip), evaluate the same forms in float32 with numpy, and
check them against the true functions in float64 (math.erf, math.tanh) over
dense grids, against the bounds the sources state:

* A&S 7.1.26: |erf error| <= 1.5e-7 plus float32 rounding of the evaluation
  (6e-7 in all);
* the tanh form: |error| <= 1e-6 (absolute);
* the normal-CDF table (step 1/64 on [-6, 6]): |Gelu error| <= 4.4e-5 on
  [-6, 6], and the table's end values beyond.

A mistyped coefficient, a wrong table step or origin, or an index/fraction
mix-up in the table lookup fails here.
"""
import math
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_implicit_gemm_amd", "csrc")


def _src(name):
    return open(os.path.join(CSRC, name)).read()


def _erfc_as_constants():
    """p and the five polynomial coefficients of erfc_as() in epilogue.h."""
    s = _src("epilogue.h")
    body = s[s.index("float erfc_as(float u)"):]
    body = body[:body.index("}")]
    p = float(re.search(r"1\.0f \+ ([0-9.]+)f \* u", body).group(1))
    coef = [float(c) for c in re.findall(r"(-?[0-9]+\.[0-9]+)f", body.split("poly")[1])]
    assert len(coef) == 5, coef
    return p, coef


def _erfc_as(u, p, a):
    u = u.astype(np.float32)
    t = (np.float32(1.0) / (np.float32(1.0) + np.float32(p) * u)).astype(np.float32)
    poly = np.zeros_like(t)
    for c in reversed(a):
        poly = (np.float32(c) + t * poly).astype(np.float32)
    poly = (t * poly).astype(np.float32)
    return (poly * np.exp(-(u * u)).astype(np.float32)).astype(np.float32)


def test_erf_form_within_abramowitz_stegun_bound():
    p, a = _erfc_as_constants()
    assert abs(p - 0.3275911) < 1e-12
    x = np.linspace(-8.0, 8.0, 400001)
    c = _erfc_as(np.abs(x), p, a)
    got = np.where(x < 0, -(1.0 - c.astype(np.float64)), 1.0 - c.astype(np.float64))
    ref = np.array([math.erf(v) for v in x])
    err = np.max(np.abs(got - ref))
    # the formula's bound, plus the float32 evaluation: t, five Horner steps and
    # the exponential each round a value near 1 (about 7 roundings of 6e-8)
    assert err <= 1.5e-7 + 4.5e-7, err


def test_gelu_erf_form_error():
    # 0.5 v (1 + erf(v / sqrt 2)) with 1 + erf = erfc(|v|/sqrt 2) for v < 0
    p, a = _erfc_as_constants()
    v = np.linspace(-10.0, 10.0, 200001).astype(np.float32)
    c = _erfc_as(np.abs(v) * np.float32(0.70710678118654752), p, a).astype(np.float64)
    got = 0.5 * v * np.where(v < 0, c, 2.0 - c)
    ref = np.array([0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0))) for t in v.astype(np.float64)])
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    assert np.max(err) <= 1e-6, np.max(err)


def test_tanh_form_error():
    x = np.linspace(-12.0, 12.0, 240001).astype(np.float32)
    got = (np.float32(1.0) - np.float32(2.0) / (np.float32(1.0) + np.exp(np.float32(2.0) * x))).astype(np.float64)
    ref = np.tanh(x.astype(np.float64))
    assert np.max(np.abs(got - ref)) <= 1e-6


def _phi_table_constants():
    s = _src("kernels_smallc.hip")
    n = int(re.search(r"constexpr int kPhiN = (\d+);", s).group(1))
    scale, origin = re.search(r"constexpr float kPhiScale = ([0-9.]+)f, kPhiOrigin = ([0-9.]+)f;", s).groups()
    top = float(re.search(r"constexpr float kPhiTop = ([0-9.]+)f;", s).group(1))
    return n, float(scale), float(origin), top


def test_smallc_phi_table_gelu_bound():
    n, scale, origin, top = _phi_table_constants()
    assert np.float32(top) < np.float32(n) and np.floor(np.float32(top)) == n - 1
    # the table as the kernel writes it: Phi at x_i = (i - origin) / scale, in
    # double, stored as float32 pairs (Phi_i, Phi_{i+1} - Phi_i)
    xi = (np.arange(n + 1) - origin) / scale
    phi = np.array([0.5 * math.erfc(-t / math.sqrt(2.0)) for t in xi])
    p0 = phi.astype(np.float32)
    d = np.append(phi[1:] - phi[:-1], 0.0).astype(np.float32)
    v = np.linspace(-9.0, 9.0, 360001).astype(np.float32)
    u = np.clip((v * np.float32(scale) + np.float32(origin)).astype(np.float32), np.float32(0.0), np.float32(top))
    i = np.floor(u).astype(np.int64)                  # (int)u, u >= 0
    f = (u - np.floor(u)).astype(np.float32)          # v_fract
    got = (v * (f * d[i] + p0[i]).astype(np.float32)).astype(np.float64)
    ref = np.array([0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0))) for t in v.astype(np.float64)])
    inside = np.abs(v) <= 6.0
    assert np.max(np.abs(got - ref)[inside]) <= 4.4e-5
    # beyond +-6 the end values: |Gelu(x) - x * Phi(+-6)| stays below 1e-8 * |x|
    assert np.max(np.abs(got - ref)[~inside] / np.abs(v[~inside])) <= 1e-8
