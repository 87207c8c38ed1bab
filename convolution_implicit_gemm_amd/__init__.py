"""FusedConv for MI355X (gfx950): Y = act(conv(X, W) + B + Z) in hand-written HIP.

The computation lives in libfusedconv.so behind the C ABI of
include/fusedconv.h.  This package marshals arguments: torch tensors supply
device memory and the current HIP stream, nothing else.  Semantics follow the
FusedConv README ("Description", "Inputs", "Outputs", "Attributes").
"""
from __future__ import annotations

from ._binding import EXPORTS, FusedConvError, Handle, LIB_PATH, load

__all__ = ["fused_conv", "FusedConv", "Handle", "FusedConvError", "load", "LIB_PATH", "EXPORTS"]

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
