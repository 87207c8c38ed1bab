"""FusedConv for MI355X (gfx950): Y = act(conv(X, W) + B + Z) in hand-written HIP.

The computation lives in libfusedconv.so behind the C ABI of
include/fusedconv.h.  This package marshals arguments: torch tensors supply
device memory and the current HIP stream, nothing else.  Semantics follow the
FusedConv README ("Description", "Inputs", "Outputs", "Attributes").
"""
from __future__ import annotations

from ._binding import EXPORTS, FusedConvError, Handle, LIB_PATH, load

__all__ = ["fused_conv", "FusedConv", "Handle", "FusedConvError", "load", "LIB_PATH", "EXPORTS",
           "ConvBackwardData", "ConvBackwardWeight", "conv_backward_data", "conv_backward_weight"]

_cache: dict = {}


def _dtype_name(t):
    import torch
    if t.dtype == torch.float32:
        return "f32"
    if t.dtype == torch.float16:
        return "f16"
    raise FusedConvError(-2, f"dtype {t.dtype} is not float32 or float16")


class FusedConv:
    """A planned FusedConv for fixed shapes and attributes, run on torch tensors."""

    def __init__(self, x_shape, w_shape, dtype, has_bias=False, has_z=False, **attrs):
        self.attrs = attrs
        self.x_shape = [int(v) for v in x_shape]
        self.w_shape = [int(v) for v in w_shape]
        self.dtype = dtype
        self.has_bias = bool(has_bias)
        self.has_z = bool(has_z)
        # B has M entries: W.shape[0], or W.shape[1] * group for a transposed conv
        m = w_shape[1] * attrs.get("group", 1) if attrs.get("transposed") else w_shape[0]
        z_shape = None
        if has_z:
            # Z must have Y's shape; resolve Y first with a probe handle.
            z_shape = Handle(dtype, x_shape, w_shape, [m] if has_bias else None,
                             None, **attrs).y_shape
        self.m = int(m)
        self.handle = Handle(dtype, x_shape, w_shape, [m] if has_bias else None,
                             z_shape, **attrs)
        self.y_shape = self.handle.y_shape
        self.workspace_bytes = self.handle.workspace_bytes

    def prepare_weights(self, w, workspace, stream=None):
        """Enqueue only the weight preparation of this plan into `workspace`."""
        import torch
        if not w.is_cuda or list(w.shape) != self.w_shape or not w.is_contiguous():
            raise ValueError(f"w must be a contiguous device tensor of shape {self.w_shape}")
        if self.workspace_bytes and (workspace is None or not workspace.is_cuda or
                                     workspace.numel() * workspace.element_size()
                                     < self.workspace_bytes):
            raise FusedConvError(-14, f"prepare_weights needs a device workspace of "
                                      f"{self.workspace_bytes} bytes")
        st = stream if stream is not None else torch.cuda.current_stream(w.device).cuda_stream
        self.handle.prepare_weights(w.data_ptr(), workspace.data_ptr() if workspace is not None
                                    else None, self.workspace_bytes, st)

    def _check(self, x, w, bias, z, out, workspace, weights_prepared):
        """Raise unless every tensor has the planned shape, dtype and device: the
        library receives bare pointers and trusts the sizes it planned."""
        import torch
        want = torch.float16 if self.dtype == "f16" else torch.float32
        shapes = (("x", x, self.x_shape), ("w", w, self.w_shape),
                  ("bias", bias, [self.m] if self.has_bias else None),
                  ("z", z, self.y_shape if self.has_z else None), ("out", out, self.y_shape))
        for name, t, shape in shapes:
            if t is None:
                if shape is not None and name != "out":
                    raise ValueError(f"{name} was planned but not given")
                continue
            if name in ("bias", "z") and shape is None:
                raise ValueError(f"{name} given but not planned")
            if not t.is_cuda:
                raise FusedConvError(-1, f"{name} must be a device tensor (no CPU path)")
            if not t.is_contiguous():
                raise FusedConvError(-1, f"{name} must be contiguous")
            if t.dtype != want:
                raise ValueError(f"{name} is {t.dtype}, the plan is {want}")
            if list(t.shape) != list(shape):
                raise ValueError(f"{name} has shape {list(t.shape)}, the plan expects "
                                 f"{list(shape)}")
            if t.device != x.device:
                raise ValueError(f"{name} is on {t.device}, x on {x.device}")
        if workspace is not None:
            if not workspace.is_cuda or workspace.device != x.device:
                raise FusedConvError(-14, "workspace must be device memory on x's device")
            if workspace.numel() * workspace.element_size() < self.workspace_bytes:
                raise FusedConvError(-14, f"workspace holds fewer than {self.workspace_bytes} bytes")
        elif weights_prepared and self.workspace_bytes:
            raise FusedConvError(-14, "weights_prepared needs the workspace that "
                                      "prepare_weights filled")

    def __call__(self, x, w, bias=None, z=None, out=None, workspace=None, stream=None,
                 weights_prepared=False, events=None):
        """events: optional (start, stop) torch.cuda.Event pair (timing enabled, each
        recorded once beforehand so that it exists); the convolution kernels' own
        dispatches record them (fusedconv_run_timed)."""
        import torch
        self._check(x, w, bias, z, out, workspace, weights_prepared)
        y = out if out is not None else torch.empty(self.y_shape, dtype=x.dtype, device=x.device)
        ws = workspace
        if self.workspace_bytes and ws is None:
            ws = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=x.device)
        st = stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
        self.handle.run(x.data_ptr(), w.data_ptr(),
                        bias.data_ptr() if bias is not None else None,
                        z.data_ptr() if z is not None else None, y.data_ptr(),
                        ws.data_ptr() if ws is not None else None,
                        self.workspace_bytes if ws is not None else 0, st,
                        1 if weights_prepared else 0,
                        None if events is None else (events[0].cuda_event, events[1].cuda_event))
        return y


def fused_conv(x, w, bias=None, z=None, *, auto_pad=None, group=1, kernel_shape=None,
               strides=None, dilations=None, pads=None, activation=None,
               activation_params=None, route="auto", split_k=0, transposed=False,
               output_padding=None):
    """Y = act(conv(x, w) + bias + z) on the current stream; Y is allocated with torch.
    transposed=True: the transposed conv (W as [C, M/group, k...], output_padding)."""
    attrs = dict(auto_pad=auto_pad, group=group, kernel_shape=kernel_shape, strides=strides,
                 dilations=dilations, pads=pads, activation=activation,
                 activation_params=activation_params, route=route, split_k=split_k)
    if transposed:
        attrs.update(transposed=True, output_padding=output_padding)
    key = (tuple(x.shape), tuple(w.shape), x.dtype, bias is not None, z is not None,
           tuple((k, tuple(v) if isinstance(v, (list, tuple)) else v)
                 for k, v in sorted(attrs.items())))
    op = _cache.get(key)
    if op is None:
        op = FusedConv(list(x.shape), list(w.shape), _dtype_name(x), bias is not None,
                       z is not None, **attrs)
        _cache[key] = op
    return op(x, w, bias, z)


def _device_checks(named, want, device):
    """Each (name, tensor, shape) must be a contiguous device tensor of dtype
    `want` (None: any) and the given shape on `device`."""
    for name, t, shape in named:
        if not t.is_cuda:
            raise FusedConvError(-1, f"{name} must be a device tensor (no CPU path)")
        if not t.is_contiguous():
            raise FusedConvError(-1, f"{name} must be contiguous")
        if want is not None and t.dtype != want:
            raise ValueError(f"{name} is {t.dtype}, the plan is {want}")
        if list(t.shape) != list(shape):
            raise ValueError(f"{name} has shape {list(t.shape)}, the plan expects {list(shape)}")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


class ConvBackwardData:
    """The input gradient of a planned convolution (fusedconv_create_backward_data):
    dP = (conv^T(G, W) + R) * act_in'(P), G the gradient of the convolution's
    pre-activation output, act_in the activation that produced X from P."""

    def __init__(self, x_shape, w_shape, dtype, has_residual=False, input_activation=None,
                 input_activation_params=None, **attrs):
        self.x_shape = [int(v) for v in x_shape]
        self.w_shape = [int(v) for v in w_shape]
        self.dtype = dtype
        self.has_residual = bool(has_residual)
        self.has_pre = input_activation is not None
        fwd = {k: v for k, v in attrs.items() if k not in ("route", "split_k")}
        self.y_shape = Handle(dtype, x_shape, w_shape, None, None, **fwd).y_shape
        self.handle = Handle(dtype, x_shape, w_shape, None,
                             self.x_shape if has_residual else None, activation=input_activation,
                             activation_params=input_activation_params, kind="backward_data",
                             **attrs)
        self.workspace_bytes = self.handle.workspace_bytes

    def __call__(self, dy, w, pre=None, residual=None, out=None, workspace=None, stream=None):
        import torch
        want = torch.float16 if self.dtype == "f16" else torch.float32
        named = [("dy", dy, self.y_shape), ("w", w, self.w_shape)]
        if self.has_pre:
            if pre is None:
                raise ValueError("pre (the input pre-activation) was planned but not given")
            named.append(("pre", pre, self.x_shape))
        elif pre is not None:
            raise ValueError("pre given but no input activation was planned")
        if self.has_residual != (residual is not None):
            raise ValueError("residual given / planned mismatch")
        if residual is not None:
            named.append(("residual", residual, self.x_shape))
        if out is not None:
            named.append(("out", out, self.x_shape))
        _device_checks(named, want, dy.device)
        dx = out if out is not None else torch.empty(self.x_shape, dtype=dy.dtype, device=dy.device)
        ws = workspace
        if self.workspace_bytes and ws is None:
            ws = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=dy.device)
        if ws is not None and ws.numel() * ws.element_size() < self.workspace_bytes:
            raise FusedConvError(-14, f"workspace holds fewer than {self.workspace_bytes} bytes")
        st = stream if stream is not None else torch.cuda.current_stream(dy.device).cuda_stream
        self.handle.backward_data(dy.data_ptr(), w.data_ptr(),
                                  pre.data_ptr() if pre is not None else None,
                                  residual.data_ptr() if residual is not None else None,
                                  dx.data_ptr(), ws.data_ptr() if ws is not None else None,
                                  self.workspace_bytes if ws is not None else 0, st)
        return dx


class ConvBackwardWeight:
    """The weight (and optionally bias) gradient of a planned convolution
    (fusedconv_create_backward_weight), in float32."""

    def __init__(self, x_shape, w_shape, dtype, bias_grad=False, **attrs):
        self.x_shape = [int(v) for v in x_shape]
        self.w_shape = [int(v) for v in w_shape]
        self.dtype = dtype
        self.bias_grad = bool(bias_grad)
        fwd = {k: v for k, v in attrs.items() if k not in ("route", "split_k")}
        self.y_shape = Handle(dtype, x_shape, w_shape, None, None, **fwd).y_shape
        self.handle = Handle(dtype, x_shape, w_shape, [w_shape[0]] if bias_grad else None,
                             None, kind="backward_weight", **attrs)
        self.workspace_bytes = self.handle.workspace_bytes

    def __call__(self, x, dy, dw=None, db=None, workspace=None, stream=None):
        import torch
        want = torch.float16 if self.dtype == "f16" else torch.float32
        _device_checks([("x", x, self.x_shape), ("dy", dy, self.y_shape)], want, x.device)
        if dw is None:
            dw = torch.empty(self.w_shape, dtype=torch.float32, device=x.device)
        if self.bias_grad and db is None:
            db = torch.empty([self.w_shape[0]], dtype=torch.float32, device=x.device)
        if not self.bias_grad and db is not None:
            raise ValueError("db given but the bias gradient was not planned")
        named = [("dw", dw, self.w_shape)] + ([("db", db, [self.w_shape[0]])] if db is not None else [])
        _device_checks(named, torch.float32, x.device)
        ws = workspace
        if self.workspace_bytes and ws is None:
            ws = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=x.device)
        if ws is not None and ws.numel() * ws.element_size() < self.workspace_bytes:
            raise FusedConvError(-14, f"workspace holds fewer than {self.workspace_bytes} bytes")
        st = stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
        self.handle.backward_weight(x.data_ptr(), dy.data_ptr(), dw.data_ptr(),
                                    db.data_ptr() if db is not None else None,
                                    ws.data_ptr() if ws is not None else None,
                                    self.workspace_bytes if ws is not None else 0, st)
        return (dw, db) if self.bias_grad else dw


def conv_backward_data(dy, w, x_shape, pre=None, residual=None, *, input_activation=None,
                       input_activation_params=None, **attrs):
    """dP = (conv^T(dy, w) + residual) * act_in'(pre) on the current stream."""
    op = ConvBackwardData(x_shape, list(w.shape), _dtype_name(dy), residual is not None,
                          input_activation, input_activation_params, **attrs)
    return op(dy, w, pre, residual)


def conv_backward_weight(x, dy, w_shape, *, bias_grad=False, **attrs):
    """dW (and dB with bias_grad=True), float32, on the current stream."""
    op = ConvBackwardWeight(list(x.shape), w_shape, _dtype_name(x), bias_grad, **attrs)
    return op(x, dy)
