"""Seeded synthetic inputs for FusedConv.

This module only draws random tensors of given shapes and holds the
workload descriptions; it contains none of the convolution arithmetic
(no output-size or padding rules).  Output shapes listed here are stated
facts about each workload; the tests check them against both the oracle's
and the library's own shape arithmetic.

Workloads are shaped like the pages' layers: a small fp32 conv2d, the
CIFAR-ResNet 3x3 conv with residual and QuickGelu (tinygrad hlb-CIFAR10
ConvGroup), a vision-encoder patch-embed stem and strided downsample
(ExecuTorch conv2d PR, DaViT / SigLIP stems), a depthwise 7x7 layer
(FusedConv manifest grouped_large_kernel variants), grouped 1-D and 3-D
convs, the 1x1 reduce conv of a ResNet-50 stage-3 bottleneck (the FusedConv
README's usage example is a 1x1 conv), and a 2x2 stride-2 transposed conv (the
decoder-side inverse of the downsample).  Three more compare the explicit
im2col route with the implicit ones: a CIFAR-sized 3x3 pad-1 conv with few
input channels (12: a reduction of 108, not a multiple of 16; the tinygrad
page's MatmulConv2d runs the CIFAR net's 3x3 convs as an explicit patch
matrix times the weights), a non-overlapping 4x4 stride-4
patch embedding and a SigLIP-style 16x16 stride-16 patch embedding (a 14x14
patch grid).  "compare_routes" lists the routes each is timed on: the
implicit routes against the explicit im2col one, and for the fp32 1-D and
3-D convs the channel-last halo kernel (where it fits) against the gathered
implicit GEMM and the direct one-output-per-lane kernel.  No dataset, image
or trained weight is used.

Draw rule: numpy.random.default_rng([workload_index, sub]); tensors are
drawn in the order X, W, B, Z in float64 (standard normal times a standard
deviation, or uniform(-1, 1)), cast to float32 and then, for fp16
workloads, to float16 (round to nearest even).
"""
from __future__ import annotations

import math

import numpy as np


def draw(rng, shape, dist, std=1.0):
    """float64 sample: 'normal' (N(0, std^2)) or 'uniform' (U(-1, 1))."""
    if dist == "normal":
        return rng.standard_normal(size=shape) * std
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape)
    raise ValueError(dist)


def cast(a, dtype):
    a32 = np.asarray(a, dtype=np.float32)
    return a32.astype(np.float16) if dtype == "f16" else a32


# name -> description.  "seed" is the [workload_index, sub] pair of the draw rule.
WORKLOADS = {
    "conv2d_f32_3to16_32x32": dict(
        seed=[0, 0], dtype="f32", x=[1, 3, 32, 32], w=[16, 3, 3, 3], b=[16], z=None,
        y=[1, 16, 32, 32], dist="uniform", w_std=1.0,
        attrs=dict(pads=[1, 1, 1, 1], activation="Relu")),
    "cifar_resnet_conv3x3_f16": dict(
        seed=[1, 0], dtype="f16", x=[512, 128, 16, 16], w=[256, 128, 3, 3], b=None,
        z=[512, 256, 16, 16], y=[512, 256, 16, 16], dist="normal",
        w_std=1.0 / math.sqrt(128 * 9),
        attrs=dict(pads=[1, 1, 1, 1], activation="QuickGelu", activation_params=[1.702]),
        compare_routes=["igemm_halo", "im2col"]),
    "cifar_conv3x3_12to64_f16": dict(
        seed=[1, 1], dtype="f16", x=[512, 12, 32, 32], w=[64, 12, 3, 3], b=None, z=None,
        y=[512, 64, 32, 32], dist="normal", w_std=1.0 / math.sqrt(12 * 9),
        attrs=dict(pads=[1, 1, 1, 1]),
        compare_routes=["igemm", "im2col"]),
    "vision_stem_7x7s4_f16": dict(
        seed=[2, 0], dtype="f16", x=[32, 3, 768, 768], w=[128, 3, 7, 7], b=[128], z=None,
        y=[32, 128, 192, 192], dist="normal", w_std=1.0 / math.sqrt(147),
        attrs=dict(strides=[4, 4], pads=[3, 3, 3, 3], activation="Gelu"),
        compare_routes=["smallc", "im2col"]),
    "patch_embed_4x4s4_f16": dict(
        seed=[2, 2], dtype="f16", x=[32, 3, 768, 768], w=[128, 3, 4, 4], b=[128], z=None,
        y=[32, 128, 192, 192], dist="normal", w_std=1.0 / math.sqrt(48),
        attrs=dict(strides=[4, 4]),
        compare_routes=["smallc", "im2col", "igemm"]),
    "siglip_patch_embed_16x16s16_f16": dict(
        seed=[7, 0], dtype="f16", x=[256, 3, 224, 224], w=[768, 3, 16, 16], b=[768], z=None,
        y=[256, 768, 14, 14], dist="normal", w_std=1.0 / math.sqrt(768),
        attrs=dict(strides=[16, 16]),
        compare_routes=["im2col", "igemm"]),
    "downsample_2x2s2_f16": dict(
        seed=[2, 1], dtype="f16", x=[32, 128, 192, 192], w=[256, 128, 2, 2], b=None, z=None,
        y=[32, 256, 96, 96], dist="normal", w_std=1.0 / math.sqrt(512),
        attrs=dict(strides=[2, 2])),
    "depthwise_7x7_f16": dict(
        seed=[3, 0], dtype="f16", x=[64, 384, 56, 56], w=[384, 1, 7, 7], b=[384], z=None,
        y=[64, 384, 56, 56], dist="normal", w_std=1.0,
        attrs=dict(group=384, auto_pad="SAME_UPPER", activation="HardSwish")),
    "depthwise_7x7_dil2_f16": dict(
        seed=[3, 0], dtype="f16", x=[64, 384, 56, 56], w=[384, 1, 7, 7], b=[384], z=None,
        y=[64, 384, 56, 56], dist="normal", w_std=1.0,
        attrs=dict(group=384, auto_pad="SAME_UPPER", dilations=[2, 2], activation="HardSwish")),
    "conv1d_grouped_dil3_f32": dict(
        seed=[4, 0], dtype="f32", x=[16, 512, 4096], w=[512, 64, 9], b=None, z=None,
        y=[16, 512, 4096], dist="uniform", w_std=1.0,
        attrs=dict(group=8, dilations=[3], auto_pad="SAME_LOWER", activation="LeakyRelu",
                   activation_params=[0.1]),
        compare_routes=["igemm_halo", "igemm", "direct"]),
    "conv3d_s122_f32": dict(
        seed=[4, 1], dtype="f32", x=[4, 64, 32, 64, 64], w=[128, 64, 3, 3, 3], b=[128],
        z=[4, 128, 32, 32, 32], y=[4, 128, 32, 32, 32], dist="uniform", w_std=1.0,
        attrs=dict(strides=[1, 2, 2], pads=[1, 1, 1, 1, 1, 1], activation="Clip",
                   activation_params=[0.0, 6.0]),
        compare_routes=["igemm", "direct"]),
    "conv_transpose_2x2s2_f16": dict(
        seed=[6, 0], dtype="f16", x=[8, 256, 96, 96], w=[256, 128, 2, 2], b=[128], z=None,
        y=[8, 128, 192, 192], dist="normal", w_std=1.0 / math.sqrt(256),
        attrs=dict(transposed=True, strides=[2, 2], activation="Relu")),
    "pointwise_1x1_512to128_f16": dict(
        seed=[5, 0], dtype="f16", x=[256, 512, 28, 28], w=[128, 512, 1, 1], b=[128], z=None,
        y=[256, 128, 28, 28], dist="normal", w_std=1.0 / math.sqrt(512),
        attrs=dict(activation="Relu")),
}

# The workload the headline throughput is quoted on.
HEADLINE = "cifar_resnet_conv3x3_f16"


def make_inputs(name):
    """dict with numpy x, w, b (or None), z (or None) in the workload's dtype."""
    wl = WORKLOADS[name]
    rng = np.random.default_rng(wl["seed"])
    dt = wl["dtype"]
    x = cast(draw(rng, wl["x"], wl["dist"]), dt)
    w = cast(draw(rng, wl["w"], wl["dist"], wl["w_std"]), dt)
    b = cast(draw(rng, wl["b"], wl["dist"]), dt) if wl["b"] else None
    z = cast(draw(rng, wl["z"], wl["dist"]), dt) if wl["z"] else None
    return dict(x=x, w=w, b=b, z=z)


def random_tensors(seed, dtype, x_shape, w_shape, b_shape=None, z_shape=None,
                   dist="uniform", w_std=1.0):
    """Seeded X, W, B, Z of the given shapes (same draw rule as make_inputs)."""
    rng = np.random.default_rng(seed)
    x = cast(draw(rng, x_shape, dist), dtype)
    w = cast(draw(rng, w_shape, dist, w_std), dtype)
    b = cast(draw(rng, b_shape, dist), dtype) if b_shape is not None else None
    z = cast(draw(rng, z_shape, dist), dtype) if z_shape is not None else None
    return x, w, b, z
