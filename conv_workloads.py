"""Seeded synthetic workloads for the channels-last convolution forward pass.

This module is the one piece that both sides of a parity check share: it
names the problem shapes and draws the seeded random inputs.  It holds none
of the convolution's arithmetic (no output extents, no index mapping, no
sums); the CPU oracle and the HIP library each compute those on their own.

Shapes follow the pages: the tutorial's worked 3x3 256->256 56x56 layer and
the ResNet-50 first layer ("Convolutions", sections 4 and 5), and the
benchmark shapes of the MLX pull request "Add implicit matmul pathway for
mx.conv3d" (its fp16/fp32 tables).  No dataset is involved; every tensor is
drawn here from a fixed seed.

Distributions: x ~ U[-1, 1) (``rand * 2 - 1``) or N(0, 1); w ~ N(0, 1) scaled
by 1/sqrt(fan_in), fan_in = C_in * KD * KH * KW (the second parameter of
"N(0, 1/sqrt(fan_in))" read as a standard deviation).  Draws are made in fp32
on the CPU with ``torch.Generator`` and then rounded to the workload's dtype
(round-to-nearest-even).  Seeds: 1000*cfg + 10*sub + 1 for x and + 2 for w.
"""
from dataclasses import dataclass, replace
import hashlib
import math

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "fp32" | "fp16" | "bf16"
    x_shape: tuple             # (N, H, W, C_in) or (N, D, H, W, C_in)
    w_shape: tuple             # (C_out, KH, KW, C_in) or (C_out, KD, KH, KW, C_in)
    stride: tuple
    padding: tuple
    x_dist: str = "uniform"    # "uniform" -> U[-1, 1); "normal" -> N(0, 1)
    seed_x: int = 1
    seed_w: int = 2
    dilation: tuple = None     # per dimension, None = 1 (the variants only)
    groups: int = 1            # channel groups (the variants only); w holds C_in/groups channels
    dx_shape: tuple = None     # backward-data workloads: x_shape is dy's shape, dx_shape the result's

    @property
    def dims(self) -> int:
        return len(self.x_shape) - 2

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def scaled(self, name=None, **changes):
        """A copy with some fields replaced (used for reduced-size parity cases)."""
        return replace(self, name=name or self.name, **changes)


def _wl(cfg, sub, name, dtype, x_shape, w_shape, stride, padding, x_dist="uniform"):
    return Workload(name, dtype, tuple(x_shape), tuple(w_shape), tuple(stride), tuple(padding),
                    x_dist, 1000 * cfg + 10 * sub + 1, 1000 * cfg + 10 * sub + 2)


# The five workload groups at full size.
WORKLOADS = {
    w.name: w for w in [
        _wl(1, 0, "c1_conv3d_fp32_n1_8c16_o32", "fp32", (1, 8, 8, 8, 16), (32, 3, 3, 3, 16),
            (1, 1, 1), (1, 1, 1)),
        _wl(2, 0, "c2_conv2d_fp16_n32_56c256_o256", "fp16", (32, 56, 56, 256), (256, 3, 3, 256),
            (1, 1), (1, 1)),
        _wl(3, 0, "c3_conv2d_fp16_stem_n64_224c3_o64_k7s2", "fp16", (64, 224, 224, 3),
            (64, 7, 7, 3), (2, 2), (3, 3), x_dist="normal"),
        _wl(4, 0, "c4a_conv3d_fp16_n4_32c128_o128", "fp16", (4, 32, 32, 32, 128),
            (128, 3, 3, 3, 128), (1, 1, 1), (1, 1, 1)),
        _wl(4, 1, "c4b_conv3d_fp16_n1_64c64_o128", "fp16", (1, 64, 64, 64, 64),
            (128, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1)),
        _wl(4, 2, "c4c_conv3d_fp16_n4_32c64_o128_s2", "fp16", (4, 32, 32, 32, 64),
            (128, 3, 3, 3, 64), (2, 2, 2), (1, 1, 1)),
        _wl(5, 0, "c5a_conv3d_bf16_n4_32c65_o65", "bf16", (4, 32, 32, 32, 65),
            (65, 3, 3, 3, 65), (1, 1, 1), (1, 1, 1)),
        _wl(5, 1, "c5b_conv3d_bf16_n4_16c21_o21", "bf16", (4, 16, 16, 16, 21),
            (21, 3, 3, 3, 21), (1, 1, 1), (1, 1, 1)),
        _wl(5, 2, "c5c_conv3d_bf16_n4_32c64_o128_k311", "bf16", (4, 32, 32, 32, 64),
            (128, 3, 1, 1, 64), (1, 1, 1), (1, 0, 0)),
        _wl(5, 3, "c5d_conv3d_bf16_n4_32c64_o128_k133", "bf16", (4, 32, 32, 32, 64),
            (128, 1, 3, 3, 64), (1, 1, 1), (0, 1, 1)),
    ]
}

# The variants the tutorial lists beside the plain convolution ("Convolution
# variants worth knowing": grouped as in ResNeXt, dilated), plus padding that
# differs between the two sides of a dimension.  The pages print no shapes for
# them; these are synthetic layers of the same families at the scale of the
# plain workloads: a ResNeXt-style grouped 3x3 (32 groups of 4 channels), a
# dilated 3x3 at 256 channels, a 3D grouped 3x3x3 (2 groups of 64), and a 4x4
# stride-2 layer padded (1, 2) per side as "same" padding of an even filter
# needs.  Padding is given as (low, high) per dimension.
VARIANT_WORKLOADS = {
    w.name: w for w in [
        replace(_wl(6, 0, "v1_conv2d_fp16_resnext_n32_56c128_g32", "fp16", (32, 56, 56, 128),
                    (128, 3, 3, 4), (1, 1), ((1, 1), (1, 1))), groups=32),
        replace(_wl(6, 1, "v2_conv2d_fp16_dilated2_n8_64c256", "fp16", (8, 64, 64, 256),
                    (256, 3, 3, 256), (1, 1), ((2, 2), (2, 2))), dilation=(2, 2)),
        replace(_wl(6, 2, "v3_conv3d_fp16_grouped2_n4_32c128", "fp16", (4, 32, 32, 32, 128),
                    (128, 3, 3, 3, 64), (1, 1, 1), ((1, 1), (1, 1), (1, 1))), groups=2),
        _wl(6, 3, "v4_conv2d_fp16_k4s2_asympad_n32_56c64_o128", "fp16", (32, 56, 56, 64),
            (128, 4, 4, 64), (2, 2), ((1, 2), (1, 2))),
        replace(_wl(6, 4, "v5_conv3d_fp16_depthwise_n4_32c128", "fp16", (4, 32, 32, 32, 128),
                    (128, 3, 3, 3, 1), (1, 1, 1), ((1, 1), (1, 1), (1, 1))), groups=128),
    ]
}

# Backward-data (the transposed convolution, "Transposed" in the tutorial's
# variant list) of two headline layers: x_shape is dy's shape (the forward
# output's, written out here), dx_shape the forward input's, w the forward
# filter; stride and padding are the forward layer's.
BWD_WORKLOADS = {
    w.name: w for w in [
        replace(_wl(7, 0, "d1_dgrad_conv3d_fp16_n4_32c128_o128", "fp16", (4, 32, 32, 32, 128),
                    (128, 3, 3, 3, 128), (1, 1, 1), (1, 1, 1)), dx_shape=(4, 32, 32, 32, 128)),
        replace(_wl(7, 1, "d2_dgrad_conv3d_fp16_n4_32c64_o128_s2", "fp16", (4, 16, 16, 16, 128),
                    (128, 3, 3, 3, 64), (2, 2, 2), (1, 1, 1)), dx_shape=(4, 32, 32, 32, 64)),
    ]
}

# The fp16 3x3x3 channels-last sweep that the headline throughput is quoted on.
HEADLINE = ["c4a_conv3d_fp16_n4_32c128_o128", "c4b_conv3d_fp16_n1_64c64_o128",
            "c4c_conv3d_fp16_n4_32c64_o128_s2"]


def make_inputs(wl: Workload, device="cpu"):
    """Seeded (x, w) for a workload, in its dtype, contiguous, on ``device``."""
    gx = torch.Generator("cpu").manual_seed(wl.seed_x)
    gw = torch.Generator("cpu").manual_seed(wl.seed_w)
    if wl.x_dist == "uniform":
        x = torch.rand(wl.x_shape, generator=gx, dtype=torch.float32) * 2.0 - 1.0
    elif wl.x_dist == "normal":
        x = torch.randn(wl.x_shape, generator=gx, dtype=torch.float32)
    else:
        raise ValueError(wl.x_dist)
    fan_in = 1
    for e in wl.w_shape[1:]:
        fan_in *= e
    w = torch.randn(wl.w_shape, generator=gw, dtype=torch.float32) * (1.0 / math.sqrt(fan_in))
    x = x.to(wl.torch_dtype).contiguous()
    w = w.to(wl.torch_dtype).contiguous()
    return x.to(device), w.to(device)


def digest(t) -> str:
    """SHA-256 of a tensor's bytes (first 16 hex digits), to log what was generated."""
    raw = t.detach().to("cpu").contiguous().view(torch.uint8).numpy().tobytes()
    return hashlib.sha256(raw).hexdigest()[:16]
