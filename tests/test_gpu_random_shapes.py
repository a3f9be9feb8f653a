"""Randomised parity: many small problems drawn over the whole descriptor (2D and 3D, strides,
low and high pads, dilation, groups, odd channel counts, all dtypes), each run on the automatic
choice and on every path that accepts it, forward and backward-data, against the oracle.

The problems come from a fixed seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
import oracle
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
FWD_PATHS = ["auto", "main", "slab", "phase", "staged", "strip", "runs", "rows", "grouped", "flatk", "brick",
             "direct"]


def _macs(xs, ws, st, pads, dil, g):
    outs = [oracle.out_extent_ex(xs[1 + d], ws[1 + d], st[d], pads[d][0], pads[d][1], dil[d])
            for d in range(len(xs) - 2)]
    return xs[0] * int(np.prod(outs)) * ws[0] * int(np.prod(ws[1:]))


def _problem(i):
    rng = np.random.default_rng(1000 + i)
    while True:                                   # redraw until the oracle's work is small
        p = _draw(rng)
        if _macs(*p[1:]) <= 2e7:
            return p


def _draw(rng):
    dims = int(rng.integers(2, 4))
    dtype = ["fp32", "fp16", "bf16"][int(rng.integers(0, 3))]
    g = int(rng.choice([1, 1, 1, 2, 3, 4]))
    cin_g = int(rng.choice([1, 2, 3, 5, 8, 16, 21, 32, 64]))
    cout_g = int(rng.choice([1, 2, 4, 7, 8, 16, 32, 36, 64]))
    if g > 1 and rng.random() < 0.3:
        cin_g = cout_g = 1                      # depthwise
    ks = tuple(int(rng.integers(1, 6)) for _ in range(dims))
    st = tuple(int(rng.integers(1, 4)) for _ in range(dims))
    dil = tuple(int(rng.choice([1, 1, 2, 3])) for _ in range(dims))
    pads = tuple((int(rng.integers(0, 4)), int(rng.integers(0, 4))) for _ in range(dims))
    sp = []
    for d in range(dims):
        span = dil[d] * (ks[d] - 1) + 1
        lo = max(1, span - pads[d][0] - pads[d][1])
        sp.append(int(rng.integers(lo, lo + (6 if dims == 3 else 12))))
    n = int(rng.integers(1, 3))
    xs = (n, *sp, g * cin_g)
    ws = (g * cout_g, *ks, cin_g)
    return dtype, xs, ws, st, pads, dil, g


PROBLEMS = [_problem(i) for i in range(48)]


def _inputs(p, seed):
    dtype, xs, ws, st, pads, dil, g = p
    gen = torch.Generator("cpu").manual_seed(seed)
    x = (torch.rand(xs, generator=gen) * 2 - 1).to(DT[dtype])
    w = (torch.randn(ws, generator=gen) / np.sqrt(np.prod(ws[1:]))).to(DT[dtype])
    return x.to(DEV), w.to(DEV)


@pytest.mark.parametrize("i", range(len(PROBLEMS)))
def test_random_forward_every_accepting_path(i):
    dtype, xs, ws, st, pads, dil, g = PROBLEMS[i]
    x, w = _inputs(PROBLEMS[i], 7 + i)
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pads, dilation=dil, groups=g)
    ran = 0
    for path in FWD_PATHS:
        try:
            y = igc.conv_fwd(x, w, st, pads, path=path, dilation=dil, groups=g)
        except igc.ConvError as e:
            assert e.code == -3, (path, e)     # the path does not take the problem
            continue
        torch.cuda.synchronize()
        assert_parity(oracle.to_float64(y), ref, dtype, f"problem {i} {PROBLEMS[i]} path {path}")
        ran += 1
    assert ran >= 2                              # auto and at least the direct path


@pytest.mark.parametrize("i", range(0, len(PROBLEMS), 2))
def test_random_backward_data(i):
    dtype, xs, ws, st, pads, dil, g = PROBLEMS[i]
    _, w = _inputs(PROBLEMS[i], 11 + i)
    ys = igc.out_shape(xs, ws, st, pads, dilation=dil, groups=g)
    gen = torch.Generator("cpu").manual_seed(13 + i)
    dy = (torch.rand(ys, generator=gen) * 2 - 1).to(DT[dtype]).to(DEV)
    ref = oracle.conv_bwd_data(oracle.to_float64(dy), oracle.to_float64(w), xs, st, pads,
                               dilation=dil, groups=g)
    for path in ("auto", "runs", "direct"):
        dx = igc.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g, path=path)
        torch.cuda.synchronize()
        assert_parity(oracle.to_float64(dx), ref, dtype, f"problem {i} {PROBLEMS[i]} bwd {path}")
