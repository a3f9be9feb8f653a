"""GPU parity of backward-data (the transposed convolution) against the float64 oracle.

The library computes dx from dy and the rearranged filter as one forward
convolution per stride phase; these tests compare it with the oracle's direct
definition (the adjoint of the forward pass) element by element, on every
phase kernel, and bit for bit on integer-valued cases.
"""
import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
import oracle
from conv_workloads import BWD_WORKLOADS, make_inputs
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name, dtype, x shape, w shape (C_in/G last), stride, (low, high) pads, dilation, groups
CASES = [
    ("c4a_like_fp16_s1", "fp16", (2, 6, 7, 9, 128), (128, 3, 3, 3, 128), (1, 1, 1),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 1),
    ("strip_like_fp16_s1_w32", "fp16", (2, 5, 6, 32, 64), (64, 3, 3, 3, 64), (1, 1, 1),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 1),
    ("c4c_like_fp16_s2", "fp16", (2, 11, 12, 13, 64), (128, 3, 3, 3, 64), (2, 2, 2),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 1),
    ("bf16_2d_k4_s2_asym", "bf16", (3, 14, 15, 64), (96, 4, 4, 64), (2, 2), ((1, 2), (2, 1)), (1, 1), 1),
    ("bf16_s3_k2_gaps", "bf16", (1, 7, 8, 10, 32), (64, 2, 2, 2, 32), (3, 3, 3),
     ((0, 0), (1, 0), (0, 1)), (1, 1, 1), 1),
    ("fp16_pad_past_span", "fp16", (1, 5, 6, 7, 32), (64, 3, 3, 3, 32), (1, 1, 1),
     ((3, 3), (2, 2), (3, 0)), (1, 1, 1), 1),
    ("fp16_dilated_strided", "fp16", (2, 9, 10, 11, 64), (64, 3, 3, 3, 64), (2, 1, 2),
     ((2, 2), (1, 1), (2, 1)), (2, 1, 2), 1),
    ("bf16_grouped_g2", "bf16", (2, 6, 7, 8, 64), (128, 3, 3, 3, 32), (2, 2, 1),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 2),
    ("fp16_depthwise_s1", "fp16", (2, 8, 9, 24), (24, 3, 3, 1), (1, 1), ((1, 1), (1, 1)), (1, 1), 24),
    ("fp16_depthwise_s2", "fp16", (2, 9, 10, 24), (24, 3, 3, 1), (2, 2), ((1, 1), (1, 1)), (1, 1), 24),
    ("fp32_odd_channels", "fp32", (2, 5, 6, 7, 5), (7, 3, 2, 3, 5), (1, 2, 1), ((1, 1), (0, 1), (2, 0)),
     (1, 1, 1), 1),
    ("bf16_c65_s2", "bf16", (1, 7, 8, 9, 21), (65, 3, 3, 3, 21), (2, 2, 2), ((1, 1), (1, 1), (1, 1)),
     (1, 1, 1), 1),
    ("fp16_1x1_s2", "fp16", (2, 6, 7, 8, 64), (32, 1, 1, 1, 64), (2, 2, 2), ((0, 0), (0, 0), (0, 0)),
     (1, 1, 1), 1),
]
PATHS = ["auto", "main", "runs", "direct"]


def _dt(name):
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[name]


def _accepts(case, path):
    name, dtype, xs, ws, st, pads, dil, g = case
    if path == "main":
        return dtype in ("fp16", "bf16") and (ws[0] // g) % 32 == 0 and (xs[-1] // g) % 4 == 0
    return True


def _inputs(case):
    name, dtype, xs, ws, st, pads, dil, g = case
    gen = torch.Generator("cpu").manual_seed(sum(map(ord, name)))
    ys = igc.out_shape(xs, ws, st, pads, dilation=dil, groups=g)
    dy = (torch.rand(ys, generator=gen) * 2 - 1).to(_dt(dtype))
    fan_in = int(np.prod(ws[1:]))
    w = (torch.randn(ws, generator=gen) / np.sqrt(fan_in)).to(_dt(dtype))
    return dy.to(DEV), w.to(DEV)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_data_parity(case, path):
    if not _accepts(case, path):
        pytest.skip(f"{path} does not take {case[0]}")
    name, dtype, xs, ws, st, pads, dil, g = case
    print(f"[bwd] {name} path={path}", flush=True)
    dy, w = _inputs(case)
    dx = igc.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g, path=path)
    torch.cuda.synchronize()
    ref = oracle.conv_bwd_data(oracle.to_float64(dy), oracle.to_float64(w), xs, st, pads,
                               dilation=dil, groups=g)
    assert_parity(oracle.to_float64(dx), ref, dtype, f"{name}/{path}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_data_tap_counts_bit_exact(case):
    """dy = 1 and w = 1 only from output channel 0 to input channel 0: dx at channel 0 counts
    the (output, tap) pairs that reach each position (at most the tap count, exact in every
    dtype), every other channel is 0; bit-exact on every phase kernel."""
    name, dtype, xs, ws, st, pads, dil, g = case
    ys = igc.out_shape(xs, ws, st, pads, dilation=dil, groups=g)
    dy = torch.ones(ys, dtype=_dt(dtype), device=DEV)
    w = torch.zeros(ws, dtype=_dt(dtype))
    w[0, ..., 0] = 1
    w = w.to(DEV)
    ref = oracle.conv_bwd_data(oracle.to_float64(dy), oracle.to_float64(w), xs, st, pads,
                               dilation=dil, groups=g)
    for path in PATHS:
        if _accepts(case, path):
            dx = igc.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g, path=path)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(oracle.to_float64(dx), ref, err_msg=f"{name}/{path}")


def test_bwd_data_prepared_filter_is_reusable():
    """The rearranged filter depends only on w and the problem: one preparation serves
    repeated gradients, identical to the one-call form."""
    name, dtype, xs, ws, st, pads, dil, g = CASES[2]
    dy, w = _inputs(CASES[2])
    wt = igc.bwd_data_filter(w, xs, st, pads, dilation=dil, groups=g)
    a = igc.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g, wt=wt)
    b = igc.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g, wt=wt)
    c = igc.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_bwd_data_writes_every_position_and_nothing_else():
    """dx is filled with a marker first: every element must be overwritten (phases no tap
    reaches get zeros), and a guard band after dx must stay untouched."""
    name, dtype, xs, ws, st, pads, dil, g = CASES[4]   # stride 3 > filter 2: phases without taps
    dy, w = _inputs(CASES[4])
    n = int(np.prod(xs))
    buf = torch.full((n + 4096,), 7.0, dtype=_dt(dtype), device=DEV)
    dx = buf[:n].view(xs)
    igc.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g, out=dx)
    torch.cuda.synchronize()
    ref = oracle.conv_bwd_data(oracle.to_float64(dy), oracle.to_float64(w), xs, st, pads,
                               dilation=dil, groups=g)
    assert_parity(oracle.to_float64(dx), ref, dtype, name)
    assert (ref == 0).any()
    assert torch.all(buf[n:] == 7.0)


@pytest.mark.parametrize("name", sorted(BWD_WORKLOADS))
def test_bwd_data_workloads_full_size(name):
    """The backward-data workloads at full size, as bench.py --sweep runs them, every input
    position compared with the oracle."""
    wl = BWD_WORKLOADS[name]
    print(f"[bwd full] {name}", flush=True)
    x, w = make_inputs(wl, DEV)          # x here is dy: the shapes come from the workload
    dx = igc.conv_bwd_data(x, w, wl.dx_shape, wl.stride, wl.padding)
    torch.cuda.synchronize()
    ref = oracle.conv_bwd_data(oracle.to_float64(x), oracle.to_float64(w), wl.dx_shape, wl.stride,
                               wl.padding)
    e = assert_parity(oracle.to_float64(dx), ref, wl.dtype, name)
    print(f"[bwd full] {name} outputs={ref.size} l2_rel={e['l2_rel']:.2e} max_rel={e['max_rel']:.2e}",
          flush=True)
