"""GPU parity at the size limit: the largest problems the library accepts (a tensor just under
2^31 bytes), on each kernel family that takes them, checked against the float64 oracle at the
first and the last outputs of the tensors (the last ones read and write bytes just below the
limit, where 32-bit buffer offsets end).

The oracle cannot hold these tensors in float64, so each checked corner is its own small
problem: the input region the corner's windows cover, with the padding that falls inside the
corner given as explicit (low, high) pads.  Output j of that problem is output o0 + j of the
full one (its windows start at (o0 + j) * s - p in both), so the comparison is element by
element.
"""
import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
import oracle
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LIMIT = 1 << 31


def _dt(name):
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[name]


def _corner(x, ks, st, pads, dil, ranges):
    """The input region and the (low, high) pads of the sub-problem whose outputs are
    `ranges` (one [o0, o1) per spatial dimension) of the full problem, on image range 0."""
    sl, sub_pads = [], []
    for dim, (o0, o1) in enumerate(ranges):
        n = x.shape[1 + dim]
        k, s, e, p = ks[dim], st[dim], dil[dim], pads[dim][0]
        i0 = o0 * s - p                       # first input index of the first window
        i1 = (o1 - 1) * s - p + e * (k - 1) + 1   # one past the last index of the last window
        sl.append(slice(max(i0, 0), min(i1, n)))
        sub_pads.append((max(0, -i0), max(0, i1 - n)))
    return sl, tuple(sub_pads)


def _check_corners(name, dtype, x, w, y, st, pads, dil, groups, depth=3, width=40):
    """Compare y with the oracle on the first `depth` outputs of every spatial dimension but
    the last, and the first `width` along the last (more than one 32-output block), of image 0;
    and on the last ones of the last image."""
    nsp = x.dim() - 2
    ks = tuple(w.shape[1:-1])
    wf = oracle.to_float64(w)
    for which in ("first", "last"):
        img = 0 if which == "first" else x.shape[0] - 1
        ranges = []
        for dim in range(nsp):
            o = y.shape[1 + dim]
            r = min(width if dim == nsp - 1 else depth, o)
            ranges.append((0, r) if which == "first" else (o - r, o))
        sl, sub_pads = _corner(x, ks, st, pads, dil, ranges)
        xs = x[(slice(img, img + 1), *sl)].contiguous()
        ref = oracle.conv_fwd(oracle.to_float64(xs), wf, st, sub_pads, dilation=dil, groups=groups)
        got = y[(slice(img, img + 1), *[slice(a, b) for a, b in ranges])]
        assert ref.shape == tuple(got.shape), (ref.shape, got.shape)
        assert_parity(oracle.to_float64(got), ref, dtype, f"{name} {which}")


# name, dtype, x shape, w shape (C_in/G last), stride, (low, high) pads, dilation, groups, path
CASES = [
    # x and y 2,146,435,072 bytes each; the last 16-row block is ragged (2047 = 127 * 16 + 15)
    ("slab_2d_c256", "fp16", (1, 2047, 2048, 256), (256, 3, 3, 256), (1, 1), ((1, 1), (1, 1)),
     (1, 1), 1, "slab"),
    # 3D: 2,130,706,432 bytes each, the depth offsets reach the limit too
    ("slab_3d_c128", "bf16", (1, 127, 128, 512, 128), (128, 3, 3, 3, 128), (1, 1, 1),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 1, "slab"),
    ("strip_2d_k5_c256", "fp16", (1, 2047, 2048, 256), (64, 5, 5, 256), (1, 1), ((2, 2), (2, 2)),
     (1, 1), 1, "strip"),
    ("main_2d_c256_s12", "bf16", (1, 2047, 2048, 256), (128, 3, 3, 256), (1, 2), ((1, 1), (1, 1)),
     (1, 1), 1, "main"),
    ("phase_2d_c256_s2", "fp16", (1, 2047, 2048, 256), (128, 3, 3, 256), (2, 2), ((1, 1), (1, 1)),
     (1, 1), 1, "phase"),
    # unaligned channels: 2,138,046,464 bytes of input
    ("runs_2d_c255", "fp16", (1, 2047, 2048, 255), (8, 3, 3, 255), (1, 1), ((1, 1), (1, 1)),
     (1, 1), 1, "runs"),
    ("grouped_depthwise_c256", "fp16", (1, 2047, 2048, 256), (256, 3, 3, 1), (1, 1),
     ((1, 1), (1, 1)), (1, 1), 256, "grouped"),
    # C_in = 3 stem: here the output is the largest tensor (4 x 2047 x 2048 x 64 x 2 bytes)
    ("rows_stem_c3", "fp16", (4, 4094, 4096, 3), (64, 7, 7, 3), (2, 2), ((3, 3), (3, 3)),
     (1, 1), 1, "rows"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_largest_problem_corners(case):
    name, dtype, xs, ws, st, pads, dil, g, path = case
    ys = igc.out_shape(xs, ws, st, pads, dilation=dil, groups=g)
    esz = torch.tensor([], dtype=_dt(dtype)).element_size()
    biggest = max(np.prod(xs), np.prod(ys)) * esz
    assert LIMIT // 2 < biggest < LIMIT, biggest
    assert igc.select_path(xs, ws, st, pads, _dt(dtype), dilation=dil, groups=g) == path
    print(f"[limit] {name} x={xs} y={ys} path={path}", flush=True)
    gen = torch.Generator(DEV).manual_seed(2024)
    x = torch.rand(xs, generator=gen, device=DEV, dtype=torch.float32).mul_(2).sub_(1).to(_dt(dtype))
    w = (torch.randn(ws, generator=gen, device=DEV) / np.sqrt(np.prod(ws[1:]))).to(_dt(dtype))
    y = igc.conv_fwd(x, w, st, pads, dilation=dil, groups=g, path=path)
    torch.cuda.synchronize()
    _check_corners(name, dtype, x, w, y, st, pads, dil, g)
    del x, y
    torch.cuda.empty_cache()
