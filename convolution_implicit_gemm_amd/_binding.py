"""ctypes binding of libfusedconv.so (include/fusedconv.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  If the library is not built the import of the package still works,
but every call raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfusedconv.so")

MAX_RANK = 8
F32, F16 = 0, 1
ROUTES = {"auto": 0, "direct": 1, "igemm": 2, "depthwise": 3, "igemm_halo": 4, "smallc": 5,
          "pointwise": 6, "transposed": 7, "im2col": 8}
ROUTE_NAMES = {v: k for k, v in ROUTES.items()}

STATUS = {
    0: "FUSEDCONV_OK", -1: "FUSEDCONV_ERR_NULL_ARG", -2: "FUSEDCONV_ERR_DTYPE",
    -3: "FUSEDCONV_ERR_RANK", -4: "FUSEDCONV_ERR_ATTR_LENGTH", -5: "FUSEDCONV_ERR_ATTR_VALUE",
    -6: "FUSEDCONV_ERR_PADS_WITH_AUTO_PAD", -7: "FUSEDCONV_ERR_KERNEL_SHAPE",
    -8: "FUSEDCONV_ERR_GROUP", -9: "FUSEDCONV_ERR_BIAS_SHAPE", -10: "FUSEDCONV_ERR_Z_SHAPE",
    -11: "FUSEDCONV_ERR_ACTIVATION", -12: "FUSEDCONV_ERR_ACTIVATION_PARAMS",
    -13: "FUSEDCONV_ERR_OUTPUT_SHAPE", -14: "FUSEDCONV_ERR_WORKSPACE",
    -15: "FUSEDCONV_ERR_ALIGNMENT", -16: "FUSEDCONV_ERR_ROUTE", -17: "FUSEDCONV_ERR_LAUNCH",
    -18: "FUSEDCONV_ERR_DEVICE", -19: "FUSEDCONV_ERR_ALLOC", -20: "FUSEDCONV_ERR_TOO_LARGE",
}

# Every symbol include/fusedconv.h declares.
EXPORTS = ["fusedconv_desc_init", "fusedconv_create", "fusedconv_create_transposed",
           "fusedconv_output_shape",
           "fusedconv_workspace_size", "fusedconv_plan_info", "fusedconv_run",
           "fusedconv_prepare_weights", "fusedconv_run_ex", "fusedconv_run_timed",
           "fusedconv_run_noalloc", "fusedconv_create_backward_data",
           "fusedconv_backward_data", "fusedconv_create_backward_weight",
           "fusedconv_backward_weight", "fusedconv_destroy",
           "fusedconv_status_string", "fusedconv_last_error"]
RUN_WEIGHTS_PREPARED = 1


class Tensor(ctypes.Structure):
    _fields_ = [("present", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("dims", ctypes.c_int64 * MAX_RANK)]


class Desc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("x", Tensor), ("w", Tensor), ("bias", Tensor), ("z", Tensor),
        ("auto_pad", ctypes.c_char_p),
        ("group", ctypes.c_int64),
        ("kernel_shape", ctypes.POINTER(ctypes.c_int64)), ("n_kernel_shape", ctypes.c_int32),
        ("strides", ctypes.POINTER(ctypes.c_int64)), ("n_strides", ctypes.c_int32),
        ("dilations", ctypes.POINTER(ctypes.c_int64)), ("n_dilations", ctypes.c_int32),
        ("pads", ctypes.POINTER(ctypes.c_int64)), ("n_pads", ctypes.c_int32),
        ("activation", ctypes.c_char_p),
        ("activation_params", ctypes.POINTER(ctypes.c_float)),
        ("n_activation_params", ctypes.c_int32),
        ("route", ctypes.c_int32),
        ("split_k", ctypes.c_int32),
    ]


class FusedConvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


_lib = None


def load():
    """Load the in-tree library; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m convolution_implicit_gemm_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        lib.fusedconv_desc_init.argtypes = [ctypes.POINTER(Desc)]
        lib.fusedconv_desc_init.restype = None
        lib.fusedconv_create.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(vp)]
        lib.fusedconv_create.restype = ctypes.c_int
        lib.fusedconv_create_transposed.argtypes = [ctypes.POINTER(Desc),
                                                    ctypes.POINTER(ctypes.c_int64), ctypes.c_int32,
                                                    ctypes.POINTER(vp)]
        lib.fusedconv_create_transposed.restype = ctypes.c_int
        lib.fusedconv_output_shape.argtypes = [vp, ctypes.POINTER(ctypes.c_int64),
                                               ctypes.POINTER(ctypes.c_int32)]
        lib.fusedconv_output_shape.restype = ctypes.c_int
        lib.fusedconv_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
        lib.fusedconv_workspace_size.restype = ctypes.c_int
        lib.fusedconv_plan_info.argtypes = [vp, ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_int32), ctypes.c_char_p,
                                            ctypes.c_size_t]
        lib.fusedconv_plan_info.restype = ctypes.c_int
        lib.fusedconv_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.fusedconv_run.restype = ctypes.c_int
        lib.fusedconv_prepare_weights.argtypes = [vp, vp, vp, ctypes.c_size_t, vp]
        lib.fusedconv_prepare_weights.restype = ctypes.c_int
        lib.fusedconv_run_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                         ctypes.c_uint, vp]
        lib.fusedconv_run_ex.restype = ctypes.c_int
        lib.fusedconv_run_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                            ctypes.c_uint, vp, vp, vp]
        lib.fusedconv_run_timed.restype = ctypes.c_int
        lib.fusedconv_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        lib.fusedconv_run_noalloc.restype = ctypes.c_int
        for fn in ("fusedconv_create_backward_data", "fusedconv_create_backward_weight"):
            getattr(lib, fn).argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(vp)]
            getattr(lib, fn).restype = ctypes.c_int
        lib.fusedconv_backward_data.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.fusedconv_backward_data.restype = ctypes.c_int
        lib.fusedconv_backward_weight.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.fusedconv_backward_weight.restype = ctypes.c_int
        lib.fusedconv_destroy.argtypes = [vp]
        lib.fusedconv_destroy.restype = None
        lib.fusedconv_status_string.argtypes = [ctypes.c_int]
        lib.fusedconv_status_string.restype = ctypes.c_char_p
        lib.fusedconv_last_error.argtypes = []
        lib.fusedconv_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _tensor(shape):
    t = Tensor()
    if shape is None:
        return t
    shape = list(shape)
    if len(shape) > MAX_RANK:
        raise ValueError("rank above %d" % MAX_RANK)
    t.present = 1
    t.rank = len(shape)
    for i, v in enumerate(shape):
        t.dims[i] = int(v)
    return t


def _i64list(vals, keep):
    if vals is None:
        return None, 0
    arr = (ctypes.c_int64 * max(1, len(vals)))(*[int(v) for v in vals])
    keep.append(arr)
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), len(vals)


class Handle:
    """An immutable FusedConv problem: resolved shapes, attributes and plan.

    kind: "forward" (fusedconv_create, or fusedconv_create_transposed with
    transposed=True), "backward_data" (fusedconv_create_backward_data: the
    activation names the one that produced X, z_shape declares a residual
    gradient of X's shape) or "backward_weight"
    (fusedconv_create_backward_weight: bias_shape requests the bias gradient).
    """

    def __init__(self, dtype, x_shape, w_shape, bias_shape=None, z_shape=None, *,
                 auto_pad=None, group=1, kernel_shape=None, strides=None, dilations=None,
                 pads=None, activation=None, activation_params=None, route="auto", split_k=0,
                 transposed=False, output_padding=None, kind="forward"):
        lib = load()
        d = Desc()
        lib.fusedconv_desc_init(ctypes.byref(d))
        keep = []
        d.dtype = {"f32": F32, "f16": F16}[dtype] if isinstance(dtype, str) else int(dtype)
        d.x, d.w = _tensor(x_shape), _tensor(w_shape)
        d.bias, d.z = _tensor(bias_shape), _tensor(z_shape)
        if auto_pad is not None:
            b = auto_pad.encode()
            keep.append(b)
            d.auto_pad = b
        d.group = int(group)
        d.kernel_shape, d.n_kernel_shape = _i64list(kernel_shape, keep)
        d.strides, d.n_strides = _i64list(strides, keep)
        d.dilations, d.n_dilations = _i64list(dilations, keep)
        d.pads, d.n_pads = _i64list(pads, keep)
        if activation is not None:
            b = activation.encode()
            keep.append(b)
            d.activation = b
        if activation_params is not None:
            arr = (ctypes.c_float * max(1, len(activation_params)))(
                *[float(v) for v in activation_params])
            keep.append(arr)
            d.activation_params = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
            d.n_activation_params = len(activation_params)
        d.route = ROUTES[route] if isinstance(route, str) else int(route)
        d.split_k = int(split_k)
        h = ctypes.c_void_p()
        if kind == "backward_data":
            rc = lib.fusedconv_create_backward_data(ctypes.byref(d), ctypes.byref(h))
        elif kind == "backward_weight":
            rc = lib.fusedconv_create_backward_weight(ctypes.byref(d), ctypes.byref(h))
        elif kind != "forward":
            raise ValueError(f"unknown handle kind {kind!r}")
        elif transposed:
            op, nop = _i64list(output_padding, keep)
            rc = lib.fusedconv_create_transposed(ctypes.byref(d), op, nop, ctypes.byref(h))
        else:
            rc = lib.fusedconv_create(ctypes.byref(d), ctypes.byref(h))
        if rc != 0:
            raise FusedConvError(rc, lib.fusedconv_last_error().decode())
        self._lib = lib
        self._h = h
        self.kind = kind
        dims = (ctypes.c_int64 * MAX_RANK)()
        rank = ctypes.c_int32()
        lib.fusedconv_output_shape(h, dims, ctypes.byref(rank))
        self.y_shape = [dims[i] for i in range(rank.value)]
        ws = ctypes.c_size_t()
        lib.fusedconv_workspace_size(h, ctypes.byref(ws))
        self.workspace_bytes = ws.value
        r, s = ctypes.c_int32(), ctypes.c_int32()
        name = ctypes.create_string_buffer(64)
        lib.fusedconv_plan_info(h, ctypes.byref(r), ctypes.byref(s), name, 64)
        self.route = ROUTE_NAMES.get(r.value, str(r.value))
        self.split_k = s.value
        self.kernel_name = name.value.decode()

    def run(self, x, w, bias, z, y, workspace, workspace_bytes, stream, flags=0, events=None):
        """Raw device pointers (ints or None); stream is a hipStream_t as int (0 = default).
        events: optional (start, stop) hipEvent_t handles recorded by the convolution
        kernels' dispatches (fusedconv_run_timed)."""
        if events is not None:
            rc = self._lib.fusedconv_run_timed(self._h, x, w, bias, z, y, workspace,
                                               workspace_bytes, flags, stream, events[0],
                                               events[1])
        else:
            rc = self._lib.fusedconv_run_ex(self._h, x, w, bias, z, y, workspace,
                                            workspace_bytes, flags, stream)
        if rc != 0:
            raise FusedConvError(rc, self._lib.fusedconv_last_error().decode())

    def run_noalloc(self, x, w, bias, z, y, stream):
        """fusedconv_run_noalloc: the workspace is the library's own fixed array."""
        rc = self._lib.fusedconv_run_noalloc(self._h, x, w, bias, z, y, stream)
        if rc != 0:
            raise FusedConvError(rc, self._lib.fusedconv_last_error().decode())

    def backward_data(self, dy, w, pre, dres, dx, workspace, workspace_bytes, stream):
        """fusedconv_backward_data on raw device pointers (ints or None)."""
        rc = self._lib.fusedconv_backward_data(self._h, dy, w, pre, dres, dx, workspace,
                                               workspace_bytes, stream)
        if rc != 0:
            raise FusedConvError(rc, self._lib.fusedconv_last_error().decode())

    def backward_weight(self, x, dy, dw, db, workspace, workspace_bytes, stream):
        """fusedconv_backward_weight on raw device pointers (ints or None)."""
        rc = self._lib.fusedconv_backward_weight(self._h, x, dy, dw, db, workspace,
                                                 workspace_bytes, stream)
        if rc != 0:
            raise FusedConvError(rc, self._lib.fusedconv_last_error().decode())

    def prepare_weights(self, w, workspace, workspace_bytes, stream):
        rc = self._lib.fusedconv_prepare_weights(self._h, w, workspace, workspace_bytes, stream)
        if rc != 0:
            raise FusedConvError(rc, self._lib.fusedconv_last_error().decode())

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.fusedconv_destroy(h)
            self._h = None
