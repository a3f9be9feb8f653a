"""GPU tests of the boundary rules: no workspace and no writes outside y on every path,
tensors that are not 16-byte aligned, and the plain ``conv_fwd(desc, x, w, y, stream)``
entry point.

The implicit GEMM needs no memory beyond x, w and y (the "Convolutions" tutorial,
section 5, the implicit-GEMM entry of its list of alternatives); every path is run
here with y inside a larger buffer whose guard bands on both sides must come back
untouched.  A tensor that is only element-aligned (a view at an element offset) must
not reach the kernels that move 16-byte pieces: AUTO falls back to the tail path
instead (the dispatch rule of the MLX pull request "Add implicit matmul pathway for
mx.conv3d", section "What changed"), and a forced 16-byte path is refused.
"""
import ctypes
import zlib

import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
import oracle
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def _inputs(name, dtype, xs, ws):
    gen = torch.Generator("cpu").manual_seed(zlib.crc32(name.encode()))
    x = (torch.rand(xs, generator=gen) * 2 - 1).to(DT[dtype])
    w = (torch.randn(ws, generator=gen) / np.sqrt(int(np.prod(ws[1:])))).to(DT[dtype])
    return x.to(DEV), w.to(DEV)


def _ref(x, w, st, pd, dil=1, groups=1):
    return oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pd, dilation=dil, groups=groups)


# One problem per path, each with ragged tiles along M (and N where the path allows it).
CANARY = [
    # path, dtype, x shape, w shape, stride, pad, groups
    ("slab", "fp16", (1, 3, 19, 37, 64), (68, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1), 1),
    ("slab", "bf16", (1, 2, 21, 40, 128), (256, 3, 3, 3, 128), (1, 1, 1), (1, 1, 1), 1),
    ("strip", "fp16", (1, 3, 5, 32, 64), (72, 3, 3, 3, 64), (1, 2, 1), (1, 1, 1), 1),
    ("phase", "fp16", (1, 3, 19, 37, 64), (68, 3, 3, 3, 64), (1, 2, 2), (1, 1, 1), 1),
    ("phase", "bf16", (2, 21, 34, 128), (256, 3, 2, 128), (2, 2), (1, 0), 1),
    ("main", "fp16", (2, 5, 6, 7, 64), (68, 3, 3, 3, 64), (2, 2, 2), (1, 1, 1), 1),
    ("main", "bf16", (3, 7, 9, 11, 64), (132, 3, 1, 1, 64), (1, 1, 1), (1, 0, 0), 1),
    ("brick", "fp16", (2, 5, 6, 7, 32), (36, 3, 3, 3, 32), (1, 1, 1), (1, 1, 1), 1),
    ("rows", "fp16", (1, 9, 16, 3), (20, 3, 3, 3), (1, 1), (1, 1), 1),
    ("rows", "bf16", (2, 23, 40, 3), (64, 7, 7, 3), (2, 2), (3, 3), 1),
    ("runs", "bf16", (2, 5, 6, 7, 21), (21, 3, 3, 3, 21), (1, 1, 1), (1, 1, 1), 1),
    ("runs", "fp32", (1, 5, 6, 7, 5), (7, 3, 3, 3, 5), (1, 1, 1), (1, 1, 1), 1),
    ("flatk", "bf16", (2, 5, 6, 7, 5), (7, 3, 3, 3, 5), (1, 1, 1), (1, 1, 1), 1),
    ("direct", "fp16", (1, 5, 6, 7, 3), (5, 3, 3, 3, 3), (2, 1, 2), (1, 1, 1), 1),
    ("grouped", "fp16", (2, 9, 10, 32), (32, 3, 3, 1), (1, 1), (1, 1), 32),
    ("grouped", "bf16", (2, 9, 10, 12), (18, 3, 3, 2), (1, 1), (1, 1), 6),
    ("staged", "bf16", (1, 3, 19, 37, 65), (65, 3, 3, 3, 65), (1, 1, 1), (1, 1, 1), 1),
    ("staged", "fp16", (2, 18, 40, 33), (130, 3, 2, 33), (1, 1), (1, 1), 1),
    ("staged", "fp16", (1, 4, 16, 32, 9), (24, 3, 3, 3, 9), (1, 1, 1), (1, 1, 1), 1),
]


@pytest.mark.parametrize("case", CANARY, ids=[f"{c[0]}_{c[1]}_{i}" for i, c in enumerate(CANARY)])
def test_no_workspace_and_no_out_of_bounds_writes(case):
    """The call allocates nothing and writes only inside y: guard bands on both sides of y
    keep their values; y itself matches the oracle."""
    path, dtype, xs, ws, st, pd, g = case
    print(f"[canary] {path} {dtype} {xs} {ws}", flush=True)
    x, w = _inputs(f"canary{xs}{ws}", dtype, xs, ws)
    shape = igc.out_shape(xs, ws, st, pd, groups=g)
    n = int(np.prod(shape))
    guard = 4096
    buf = torch.full((n + 2 * guard,), 1234.0, dtype=DT[dtype], device=DEV)
    y = buf[guard:guard + n].view(shape)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    igc.conv_fwd(x, w, st, pd, out=y, path=path, groups=g)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.all(buf[:guard] == 1234.0) and torch.all(buf[guard + n:] == 1234.0)
    assert_parity(oracle.to_float64(y), _ref(x, w, st, pd, groups=g), dtype, f"canary {path}")


@pytest.mark.parametrize("path", ["auto", "main", "runs", "direct"])
def test_bwd_data_phases_write_only_inside_dx(path):
    """Backward-data of a stride-2 layer (eight stride phases; on main they share one phased
    launch): guard bands on both sides of dx keep their values, dx matches the oracle."""
    dtype, xs, ws, st, pd = "fp16", (2, 9, 10, 11, 64), (128, 3, 3, 3, 64), (2, 2, 2), (1, 1, 1)
    print(f"[canary bwd] {path}", flush=True)
    ys = igc.out_shape(xs, ws, st, pd)
    dy, w = _inputs("canary_bwd", dtype, ys, ws)
    n = int(np.prod(xs))
    guard = 4096
    buf = torch.full((n + 2 * guard,), 1234.0, dtype=DT[dtype], device=DEV)
    dx = buf[guard:guard + n].view(xs)
    wt = igc.bwd_data_filter(w, xs, st, pd)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    igc.conv_bwd_data(dy, w, xs, st, pd, out=dx, path=path, wt=wt)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.all(buf[:guard] == 1234.0) and torch.all(buf[guard + n:] == 1234.0)
    ref = oracle.conv_bwd_data(oracle.to_float64(dy), oracle.to_float64(w), xs, st, pd)
    assert_parity(oracle.to_float64(dx), ref, dtype, f"bwd canary {path}")


# ---- tensors that are only element-aligned -------------------------------------------------

def _offset_view(t, elems):
    """A contiguous copy of t that starts `elems` elements into a fresh allocation, so its
    address is element-aligned but (for elems * itemsize not a multiple of 16) not 16-byte
    aligned."""
    buf = torch.empty(t.numel() + elems + 64, dtype=t.dtype, device=t.device)
    v = buf[elems:elems + t.numel()].view(t.shape)
    v.copy_(t)
    return v


MISALIGNED = [
    # name, dtype, x shape, w shape, stride, pad, groups, which tensors are offset
    ("slab_shape_x", "fp16", (1, 4, 9, 33, 64), (64, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1), 1, "x"),
    ("slab_shape_w", "fp16", (1, 4, 9, 33, 64), (64, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1), 1, "w"),
    ("slab_shape_y", "bf16", (1, 4, 9, 33, 64), (68, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1), 1, "y"),
    ("main_shape_s2_xwy", "fp16", (2, 9, 10, 11, 64), (128, 3, 3, 3, 64), (2, 2, 2), (1, 1, 1), 1, "xwy"),
    ("rows_shape_x", "fp16", (2, 30, 32, 3), (64, 7, 7, 3), (2, 2), (3, 3), 1, "x"),
    ("tail_c21_y", "bf16", (2, 6, 7, 8, 21), (21, 3, 3, 3, 21), (1, 1, 1), (1, 1, 1), 1, "y"),
    ("fp32_x", "fp32", (1, 6, 6, 6, 16), (32, 3, 3, 3, 16), (1, 1, 1), (1, 1, 1), 1, "xy"),
    ("depthwise_x", "fp16", (2, 9, 10, 32), (32, 3, 3, 1), (1, 1), (1, 1), 32, "x"),
    ("staged_c65_xwy", "bf16", (1, 3, 16, 32, 65), (65, 3, 3, 3, 65), (1, 1, 1), (1, 1, 1), 1, "xwy"),
    ("staged_shape_c64_x", "fp16", (1, 3, 16, 32, 64), (64, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1), 1, "x"),
]


@pytest.mark.parametrize("case", MISALIGNED, ids=[c[0] for c in MISALIGNED])
def test_element_aligned_tensors_fall_back(case):
    """x, w or y at an odd element offset (element-aligned, not 16-byte aligned): AUTO runs
    the problem on a path that needs element alignment only and matches the oracle; on the
    fall-back path (staged or runs) the result equals that path's result on aligned copies bit for bit (the same
    kernel and summation order; the grouped path switches from its 16-byte kernel to its
    general one); a forced 16-byte path is refused before any launch."""
    name, dtype, xs, ws, st, pd, g, which = case
    print(f"[misaligned] {name}", flush=True)
    x, w = _inputs(name, dtype, xs, ws)
    shape = igc.out_shape(xs, ws, st, pd, groups=g)
    xm = _offset_view(x, 1) if "x" in which else x
    wm = _offset_view(w, 1) if "w" in which else w
    ym = _offset_view(torch.zeros(shape, dtype=x.dtype, device=DEV), 1) if "y" in which \
        else torch.empty(shape, dtype=x.dtype, device=DEV)
    for t, tag in ((xm, "x"), (wm, "w"), (ym, "y")):
        if tag in which:
            assert t.data_ptr() % 16 != 0 and t.data_ptr() % t.element_size() == 0
    igc.conv_fwd(xm, wm, st, pd, out=ym, groups=g)
    torch.cuda.synchronize()
    assert_parity(oracle.to_float64(ym), _ref(x, w, st, pd, groups=g), dtype, name)
    if g == 1:
        # the element-aligned paths AUTO may fall back to: staged, else runs
        bits = (lambda t: t.view(torch.uint8) if dtype != "fp32" else t.view(torch.int32))
        same = []
        for p in ("staged", "runs"):
            try:
                ya = igc.conv_fwd(x, w, st, pd, path=p)
            except igc.ConvError:
                continue
            torch.cuda.synchronize()
            same.append(torch.equal(bits(ym), bits(ya)))
        assert any(same), same
    aligned_path = igc.select_path(xs, ws, st, pd, DT[dtype], groups=g)
    if aligned_path in ("slab", "phase", "strip", "main", "rows"):
        with pytest.raises(igc.ConvError) as err:
            igc.conv_fwd(xm, wm, st, pd, out=ym, path=aligned_path, groups=g)
        assert err.value.code == -3


def test_bwd_data_element_aligned_dy_falls_back():
    """Backward-data with dy at an odd element offset: every phase runs on an
    element-aligned path and dx matches the oracle; forced main is refused."""
    dtype, xs, ws, st, pd = "fp16", (2, 9, 10, 11, 64), (128, 3, 3, 3, 64), (2, 2, 2), (1, 1, 1)
    ys = igc.out_shape(xs, ws, st, pd)
    dy, w = _inputs("misaligned_bwd", dtype, ys, ws)
    dym = _offset_view(dy, 3)
    dx = igc.conv_bwd_data(dym, w, xs, st, pd)
    torch.cuda.synchronize()
    ref = oracle.conv_bwd_data(oracle.to_float64(dy), oracle.to_float64(w), xs, st, pd)
    assert_parity(oracle.to_float64(dx), ref, dtype, "bwd misaligned dy")
    with pytest.raises(igc.ConvError) as err:
        igc.conv_bwd_data(dym, w, xs, st, pd, path="main")
    assert err.value.code == -3


# ---- the plain entry point: conv_fwd(desc, x, w, y, stream) ---------------------------------

PLAIN = [
    # name, dtype, x shape, w shape, stride, pad, groups, the path AUTO takes
    ("slab_c64", "fp16", (2, 4, 16, 30, 64), (128, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1), 1, "slab"),
    ("phase_s2", "fp16", (2, 11, 12, 13, 64), (128, 3, 3, 3, 64), (2, 2, 2), (1, 1, 1), 1, "phase"),
    ("main_s221", "fp16", (2, 11, 12, 13, 64), (128, 3, 3, 3, 64), (2, 2, 1), (1, 1, 1), 1, "main"),
    ("runs_c21", "bf16", (3, 6, 7, 8, 21), (21, 3, 3, 3, 21), (1, 1, 1), (1, 1, 1), 1, "runs"),
    ("rows_stem", "fp16", (2, 30, 32, 3), (64, 7, 7, 3), (2, 2), (3, 3), 1, "rows"),
    ("runs_fp32", "fp32", (1, 8, 8, 8, 16), (32, 3, 3, 3, 16), (1, 1, 1), (1, 1, 1), 1, "runs"),
    ("grouped_depthwise", "bf16", (2, 6, 7, 9, 32), (32, 3, 3, 3, 1), (1, 1, 1), (1, 1, 1), 32, "grouped"),
    ("staged_c65", "bf16", (1, 4, 16, 32, 65), (65, 3, 3, 3, 65), (1, 1, 1), (1, 1, 1), 1, "staged"),
]


@pytest.mark.parametrize("case", PLAIN, ids=[c[0] for c in PLAIN])
def test_plain_conv_fwd_entry_point(case):
    """The plain descriptor through conv_fwd itself (the route a C caller takes: the
    descriptor widened to the extended one, then AUTO and any recorded choice)."""
    name, dtype, xs, ws, st, pd, g, expect = case
    print(f"[plain] {name}", flush=True)
    igc.tune_clear()
    x, w = _inputs(name, dtype, xs, ws)
    d = igc.make_desc(xs, ws, st, pd, DT[dtype], groups=g)
    assert igc.lib().conv_select_path(ctypes.byref(d)) == igc.PATHS[expect]
    shape = igc.out_shape(xs, ws, st, pd, groups=g)
    y = torch.empty(shape, dtype=x.dtype, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    rc = igc.lib().conv_fwd(ctypes.byref(d), x.data_ptr(), w.data_ptr(), y.data_ptr(), stream)
    assert rc == 0, igc.lib().conv_strerror(rc)
    torch.cuda.synchronize()
    assert_parity(oracle.to_float64(y), _ref(x, w, st, pd, groups=g), dtype, name)


@pytest.mark.parametrize("case", CANARY, ids=[f"{c[0]}_{c[1]}_{i}" for i, c in enumerate(CANARY)])
def test_repeated_launches_are_bit_identical(case):
    """Three launches of the same path on the same inputs, each preceded by a different
    unrelated launch (so the machine state and the order of work around them differ), give
    bit-identical results: a race on a staged LDS buffer would show as a difference."""
    path, dtype, xs, ws, st, pd, g = case
    x, w = _inputs(f"repeat{xs}{ws}", dtype, xs, ws)
    other_x, other_w = _inputs("repeat_other", "fp16", (2, 6, 7, 9, 64), (64, 3, 3, 3, 64))
    outs = []
    for i in range(3):
        for _ in range(i):
            igc.conv_fwd(other_x, other_w, 1, 1, path=("main", "slab", "runs")[i])
        outs.append(igc.conv_fwd(x, w, st, pd, path=path, groups=g))
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "fp32" else torch.int16
    for o in outs[1:]:
        assert torch.equal(o.view(view), outs[0].view(view))
