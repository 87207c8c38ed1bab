"""Python face of the FusedConv oracle (fusedconv_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and
the CPU-baseline leg of the benchmark, never by the product package.  It
shares no code with the HIP library (see the header of fusedconv_oracle.c).

All inputs are converted to float64 exactly (float16 and float32 values are
representable in double), and results come back as float64 arrays.
conv_transpose() (the transposed convolution) is written here in numpy,
float64, and pinned in the tests against torch's CPU routine, the adjoint
identity with fusedconv() and a closed form.
Attribute conventions follow the FusedConv README "Attributes" table:
``pads`` in ONNX order [begins..., ends...], ``strides``/``dilations`` one
entry per spatial axis, ``auto_pad`` one of NOTSET/SAME_UPPER/SAME_LOWER/VALID.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fusedconv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# Position in the manifest's activation list, plus one (0 = none).
ACTIVATIONS = ["Relu", "LeakyRelu", "Sigmoid", "Tanh", "HardSigmoid", "HardSwish", "Clip",
               "QuickGelu", "Elu", "Gelu", "FastGelu", "Softplus", "ThresholdedRelu", "Erf"]
PAD_MODES = {"NOTSET": 0, "SAME_UPPER": 1, "SAME_LOWER": 2, "VALID": 3}

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc: plain C, -O2, OpenMP, no intrinsics."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        lib = ctypes.CDLL(LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_output_dims.argtypes = [ctypes.c_int, i64p, i64p, i64p, i64p, ctypes.c_int,
                                           i64p, i64p, i64p]
        lib.oracle_output_dims.restype = ctypes.c_int
        common = [ctypes.c_int, i64p, i64p, dp, dp, dp, dp, ctypes.c_int64, i64p, i64p,
                  ctypes.c_int, i64p, ctypes.c_int, dp, ctypes.c_int]
        lib.oracle_fusedconv.argtypes = common + [ctypes.c_int64, ctypes.c_int64, dp]
        lib.oracle_fusedconv.restype = ctypes.c_int
        lib.oracle_fusedconv_at.argtypes = common + [i64p, ctypes.c_int64, dp]
        lib.oracle_fusedconv_at.restype = ctypes.c_int
        lib.oracle_activation_array.argtypes = [ctypes.c_int, dp, ctypes.c_int, dp,
                                                ctypes.c_int64, dp]
        lib.oracle_activation_array.restype = None
        _lib = lib
    return _lib


def _i64(seq):
    if seq is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(seq, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _f64(arr):
    if arr is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(arr).astype(np.float64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def act_id(name):
    return 0 if name is None else ACTIVATIONS.index(name) + 1


def output_dims(in_sp, k_sp, strides=None, dilations=None, auto_pad="NOTSET", pads=None):
    """(out_sp, pad_begin) per axis, or None when an output size is not positive."""
    lib = _load()
    nsp = len(in_sp)
    keep = []
    args = []
    for seq in (in_sp, k_sp, strides, dilations):
        a, p = _i64(seq)
        keep.append(a)
        args.append(p)
    pa, pp = _i64(pads)
    out = np.zeros(nsp, np.int64)
    pb = np.zeros(nsp, np.int64)
    rc = lib.oracle_output_dims(nsp, args[0], args[1], args[2], args[3], PAD_MODES[auto_pad], pp,
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                pb.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    if rc != 0:
        return None
    return [int(v) for v in out], [int(v) for v in pb]


def _prep(x, w, b, z, group, strides, dilations, auto_pad, pads, activation, activation_params):
    nsp = x.ndim - 2
    keep = []
    xs, xsp = _i64(x.shape)
    ws, wsp = _i64(w.shape)
    xa, xp = _f64(x)
    wa, wp = _f64(w)
    ba, bp = _f64(b)
    za, zp = _f64(z)
    sa, sp = _i64(strides)
    da, dp_ = _i64(dilations)
    pa, pp = _i64(pads)
    prm = list(activation_params) if activation_params is not None else []
    ra, rp = _f64(np.asarray(prm if prm else [0.0], dtype=np.float64))
    keep += [xs, ws, xa, wa, ba, za, sa, da, pa, ra]
    args = [nsp, xsp, wsp, xp, wp, bp, zp, int(group), sp, dp_, PAD_MODES[auto_pad], pp,
            act_id(activation), rp, len(prm)]
    return keep, args


def fusedconv(x, w, b=None, z=None, *, group=1, strides=None, dilations=None,
              auto_pad="NOTSET", pads=None, activation=None, activation_params=None,
              batches=None):
    """Y as float64 for all images, or for images [batches[0], batches[1])."""
    lib = _load()
    out = output_dims(list(x.shape[2:]), list(w.shape[2:]), strides, dilations, auto_pad, pads)
    if out is None:
        raise ValueError("oracle: output size not positive")
    n0, n1 = (0, x.shape[0]) if batches is None else batches
    y = np.zeros([n1 - n0, w.shape[0]] + out[0], np.float64)
    keep, args = _prep(x, w, b, z, group, strides, dilations, auto_pad, pads, activation,
                       activation_params)
    rc = lib.oracle_fusedconv(*args, n0, n1, y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    del keep
    if rc != 0:
        raise ValueError("oracle: invalid problem")
    return y


def fusedconv_at(x, w, b=None, z=None, *, idx, group=1, strides=None, dilations=None,
                 auto_pad="NOTSET", pads=None, activation=None, activation_params=None):
    """Y at the given flat output indices (NC(D)(H)W order), as float64."""
    lib = _load()
    ia, ip = _i64(np.asarray(idx, dtype=np.int64).ravel())
    out = np.zeros(ia.size, np.float64)
    keep, args = _prep(x, w, b, z, group, strides, dilations, auto_pad, pads, activation,
                       activation_params)
    rc = lib.oracle_fusedconv_at(*args, ip, ia.size,
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    del keep
    if rc != 0:
        raise ValueError("oracle: invalid problem")
    return out


def activation(name, v, params=None):
    """The oracle's activation applied elementwise to v (float64)."""
    lib = _load()
    va, vp = _f64(np.asarray(v, dtype=np.float64).ravel())
    prm = list(params) if params is not None else []
    ra, rp = _f64(np.asarray(prm if prm else [0.0], dtype=np.float64))
    out = np.zeros(va.size, np.float64)
    lib.oracle_activation_array(act_id(name), rp, len(prm), vp, va.size,
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out.reshape(np.shape(v))


def conv_transpose(x, w, b=None, z=None, *, group=1, strides=None, dilations=None, pads=None,
                   output_padding=None, activation=None, activation_params=None):
    """Transposed convolution with the FusedConv epilogue, as float64.

    The reading (the pages name the transposed form of aten.convolution, the
    ExecuTorch conv page's entry point, without writing it out): the adjoint
    of the cross-correlation that fusedconv() computes.  X is [n, C, in...],
    W is [C, M/group, k...] (for input channel c of group g = c // (C/group)
    and output channel g*(M/group) + m), and every input element scatters
        Y[n, g*(M/group) + m, i*s - pad_begin + k*d] += X[n, c, i] * W[c, m, k]
    for all kernel taps k; positions outside the output are dropped.  Output
    size per axis: s*(in - 1) + output_padding + (k - 1)*d + 1 - pad_begin
    - pad_end.  Then Y = act(Y + B[m] + Z), as in fusedconv().

    Plain loops over groups and taps; each tap is one channel contraction
    (numpy einsum over the group's input channels) added into the strided
    output positions it reaches.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    nsp = x.ndim - 2
    n, C = x.shape[:2]
    insp = list(x.shape[2:])
    ksp = list(w.shape[2:])
    Cg, Mg = C // group, w.shape[1]
    M = Mg * group
    s = list(strides) if strides is not None else [1] * nsp
    d = list(dilations) if dilations is not None else [1] * nsp
    p = list(pads) if pads is not None else [0] * (2 * nsp)
    op = list(output_padding) if output_padding is not None else [0] * nsp
    out = [s[i] * (insp[i] - 1) + op[i] + (ksp[i] - 1) * d[i] + 1 - p[i] - p[nsp + i]
           for i in range(nsp)]
    if min(out) < 1:
        raise ValueError("oracle: output size not positive")
    # scatter into a buffer that also holds the positions before pad_begin and
    # past the end, then cut the output window out of it
    full = [s[i] * (insp[i] - 1) + (ksp[i] - 1) * d[i] + 1 + op[i] for i in range(nsp)]
    buf = np.zeros([n, M] + full, np.float64)
    for g in range(group):
        xg = x[:, g * Cg:(g + 1) * Cg]
        wg = w[g * Cg:(g + 1) * Cg]
        for tap in np.ndindex(*ksp):
            contrib = np.einsum("nc...,cm->nm...", xg, wg[(slice(None), slice(None)) + tap])
            sl = tuple(slice(tap[i] * d[i], tap[i] * d[i] + s[i] * (insp[i] - 1) + 1, s[i])
                       for i in range(nsp))
            buf[(slice(None), slice(g * Mg, (g + 1) * Mg)) + sl] += contrib
    win = tuple(slice(p[i], p[i] + out[i]) for i in range(nsp))
    y = buf[(slice(None), slice(None)) + win].copy()
    if b is not None:
        y += np.asarray(b, dtype=np.float64).reshape([1, M] + [1] * nsp)
    if z is not None:
        y += np.asarray(z, dtype=np.float64)
    if activation is not None:
        y = activation_fn(activation, y, activation_params)
    return y


def activation_fn(name, v, params=None):
    """activation() under a name that conv_transpose's argument does not shadow."""
    return activation(name, v, params)
