"""fusedconv_run_noalloc (the library's own fixed scratch array as the
workspace) against fusedconv_run with a caller workspace: the same kernels on
the same data, so the outputs must be identical bit for bit, and both within
tolerance of the oracle.  Two calls in a row, the second on a smaller problem,
so the second reads scratch the first left behind."""
import sys

import numpy as np
import pytest
import torch

import convolution_implicit_gemm_amd as fc
from convolution_implicit_gemm_amd import _binding as B
from oracle import oracle
from workloads import random_tensors

pytestmark = pytest.mark.gpu
TAU = {"f32": 1e-4, "f16": 2e-2}
SCRATCH_BYTES = 8 << 20


def log(msg):
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def ptr(t):
    return None if t is None else t.data_ptr()


def run_both(dtype, xs, ws, attrs, seed):
    """(noalloc output, fusedconv_run output, oracle) for one problem."""
    y_shape = B.Handle(dtype, xs, ws, [ws[0]], None, **attrs).y_shape
    hz = B.Handle(dtype, xs, ws, [ws[0]], y_shape, **attrs)
    assert 0 < hz.workspace_bytes <= SCRATCH_BYTES, (hz.kernel_name, hz.workspace_bytes)
    x, w, b, z = random_tensors(seed, dtype, xs, ws, [ws[0]], y_shape, dist="normal",
                                w_std=1.0 / np.sqrt(np.prod(ws[1:])))
    dx, dw, db, dz = dev(x), dev(w), dev(b), dev(z)
    tdt = torch.float16 if dtype == "f16" else torch.float32
    y_na = torch.full(hz.y_shape, 7.0, dtype=tdt, device="cuda")
    y_ws = torch.full(hz.y_shape, -7.0, dtype=tdt, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    log(f"CASE noalloc {hz.kernel_name} x={xs} w={ws} ws={hz.workspace_bytes}")
    hz.run_noalloc(ptr(dx), ptr(dw), ptr(db), ptr(dz), ptr(y_na), st)
    wsb = torch.empty(hz.workspace_bytes, dtype=torch.uint8, device="cuda")
    hz.run(ptr(dx), ptr(dw), ptr(db), ptr(dz), ptr(y_ws), ptr(wsb), hz.workspace_bytes, st)
    torch.cuda.synchronize()
    ref = oracle.fusedconv(x, w, b, z, **attrs)
    return y_na, y_ws, ref, dtype


def check(y_na, y_ws, ref, dtype):
    assert torch.equal(y_na, y_ws), "noalloc and workspace runs differ"
    g = y_na.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-30)
    assert err <= TAU[dtype], err


# (dtype, x, w, attrs): larger first, then smaller, per route with a workspace
SEQUENCES = [
    [("f16", [4, 96, 20, 20], [160, 96, 3, 3], dict(pads=[1, 1, 1, 1], activation="Relu")),  # halo
     ("f16", [2, 64, 12, 16], [96, 64, 3, 3], dict(pads=[1, 1, 1, 1], activation="Relu"))],
    [("f32", [1, 512, 8, 8], [64, 512, 3, 3], dict(pads=[1, 1, 1, 1])),               # split-K
     ("f32", [1, 256, 6, 6], [32, 256, 3, 3], dict(pads=[1, 1, 1, 1]))],
    [("f16", [2, 128, 16, 16], [128, 128, 1, 1], {}),                                 # pointwise
     ("f16", [1, 64, 8, 8], [32, 64, 1, 1], {})],
    [("f16", [2, 3, 64, 64], [64, 3, 7, 7], dict(strides=[4, 4], pads=[3, 3, 3, 3])),  # smallc
     ("f16", [1, 3, 64, 64], [32, 3, 7, 7], dict(strides=[4, 4], pads=[3, 3, 3, 3]))],
]


@pytest.mark.parametrize("si", range(len(SEQUENCES)))
def test_noalloc_matches_workspace_run_twice(si):
    for k, (dtype, xs, ws, attrs) in enumerate(SEQUENCES[si]):
        out = run_both(dtype, xs, ws, attrs, [9900, si, k])
        check(*out)


def test_noalloc_refuses_plans_beyond_the_scratch():
    xs, ws = [1, 1024, 8, 8], [1024, 1024, 3, 3]
    h = B.Handle("f16", xs, ws, None, None, pads=[1, 1, 1, 1], route="igemm_halo")
    assert h.workspace_bytes > SCRATCH_BYTES
    x = torch.zeros(xs, dtype=torch.float16, device="cuda")
    w = torch.zeros(ws, dtype=torch.float16, device="cuda")
    y = torch.zeros(h.y_shape, dtype=torch.float16, device="cuda")
    with pytest.raises(B.FusedConvError) as e:
        h.run_noalloc(x.data_ptr(), w.data_ptr(), None, None, y.data_ptr(), 0)
    assert e.value.status == "FUSEDCONV_ERR_WORKSPACE"
    assert "noalloc" in str(e.value)
    torch.cuda.synchronize()
