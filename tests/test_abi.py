"""Host-side tests of the C ABI (no GPU needed): symbols, shapes, validation, path choice.

Every call made here returns before the library touches the GPU: descriptor
validation, output extents, path selection, the empty-batch no-op and the
pointer checks all run on the host first.
"""
import ctypes
import os
import re

import pytest
import torch

import implicit_gemm_conv_amd as igc
import oracle
from conv_workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convfwd.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(conv_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert names == sorted(n for n, _, _ in igc.EXPORTS)
    lib = igc.lib()
    for n in names:
        assert hasattr(lib, n), n


def _desc(**kw):
    base = dict(n=2, d=4, h=5, w=6, c_in=8, c_out=4, k_d=3, k_h=3, k_w=3, s_d=1, s_h=1, s_w=1,
                p_d=1, p_h=1, p_w=1, groups=1, dtype=1)
    base.update(kw)
    return igc.Desc(**base)


def _out_shape(d):
    out = (ctypes.c_int64 * 5)()
    rc = igc.lib().conv_out_shape(ctypes.byref(d), out)
    return rc, tuple(out)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_out_shape_matches_oracle_extents(name):
    wl = WORKLOADS[name]
    got = igc.out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.padding)
    sp = wl.x_shape[1:-1]
    ks = wl.w_shape[1:-1]
    expect = (wl.x_shape[0], *[oracle.out_extent(sp[i], ks[i], wl.stride[i], wl.padding[i])
                               for i in range(wl.dims)], wl.w_shape[0])
    assert got == expect


def test_out_shape_table_from_pages():
    assert igc.out_shape((64, 224, 224, 3), (64, 7, 7, 3), 2, 3) == (64, 112, 112, 64)
    assert igc.out_shape((4, 32, 32, 32, 64), (128, 3, 3, 3, 64), 2, 1) == (4, 16, 16, 16, 128)
    assert igc.out_shape((1, 3, 3, 1), (1, 2, 2, 1), 1, 0) == (1, 2, 2, 1)
    assert igc.out_shape((1, 5, 5, 1), (1, 3, 3, 1), 1, 0) == (1, 3, 3, 1)


@pytest.mark.parametrize("field,value,code", [
    ("d", 0, -2), ("h", -1, -2), ("c_in", 0, -2), ("c_out", 0, -2), ("k_w", 0, -2),
    ("s_h", 0, -2), ("p_d", -1, -2), ("n", -1, -2),
    ("k_h", 12, -2),            # 5 + 2 < 12: empty output
    ("groups", 0, -2), ("groups", 3, -2),   # groups must be >= 1 and divide C_in and C_out
    ("dtype", 7, -3),
])
def test_validation_codes(field, value, code):
    rc, _ = _out_shape(_desc(**{field: value}))
    assert rc == code
    assert igc.lib().conv_fwd(ctypes.byref(_desc(**{field: value})), 16, 4096, 1 << 20, None) == code


def test_null_arguments():
    lib = igc.lib()
    assert lib.conv_out_shape(None, (ctypes.c_int64 * 5)()) == -1
    assert lib.conv_out_shape(ctypes.byref(_desc()), None) == -1
    assert lib.conv_fwd(None, 16, 16, 16, None) == -1
    assert lib.conv_fwd(ctypes.byref(_desc()), None, 4096, 1 << 20, None) == -1
    assert lib.conv_fwd(ctypes.byref(_desc()), 16, 4096, None, None) == -1


def test_too_large():
    # 2^31 bytes of fp16 input
    d = _desc(n=1, d=1, h=1 << 15, w=1 << 15, c_in=1, c_out=1, k_d=1, k_h=1, k_w=1, p_d=0, p_h=0, p_w=0)
    assert _out_shape(d)[0] == -4
    d = _desc(n=1, d=1, h=1 << 14, w=1 << 15, c_in=1, c_out=1, k_d=1, k_h=1, k_w=1, p_d=0, p_h=0, p_w=0)
    assert _out_shape(d)[0] == 0


def test_alias_rejected_before_launch():
    lib = igc.lib()
    d = _desc()
    xb = 2 * 4 * 5 * 6 * 8 * 2
    base = 1 << 24
    # y starting inside x
    assert lib.conv_fwd(ctypes.byref(d), base, base + (1 << 20), base + xb - 2, None) == -5
    # y covering w
    assert lib.conv_fwd(ctypes.byref(d), base, base + (1 << 20), base + (1 << 20) - 64, None) == -5


def test_empty_batch_is_a_no_op():
    lib = igc.lib()
    d = _desc(n=0)
    rc, shape = _out_shape(d)
    assert rc == 0 and shape[0] == 0
    assert lib.conv_fwd(ctypes.byref(d), None, None, None, None) == 0


def test_forced_path_rules():
    lib = igc.lib()
    # main path needs C_in % 32 == 0 and fp16/bf16
    d = _desc(c_in=65, n=0)
    assert lib.conv_fwd_path(ctypes.byref(d), 1, None, None, None, None) == -3
    d = _desc(c_in=64, dtype=0, n=0)
    assert lib.conv_fwd_path(ctypes.byref(d), 1, None, None, None, None) == -3
    d = _desc(c_in=64, n=0)
    assert lib.conv_fwd_path(ctypes.byref(d), 1, None, None, None, None) == 0
    assert lib.conv_fwd_path(ctypes.byref(d), 99, None, None, None, None) == -3
    # filters wider than 16 only on the direct path
    d = _desc(n=0, w=40, k_w=17)
    assert lib.conv_fwd_path(ctypes.byref(d), 2, None, None, None, None) == -3
    assert lib.conv_fwd_path(ctypes.byref(d), 7, None, None, None, None) == -3
    assert lib.conv_fwd_path(ctypes.byref(d), 4, None, None, None, None) == 0


def test_strerror_and_path_names():
    lib = igc.lib()
    for code in range(-7, 1):
        assert lib.conv_strerror(code)
    assert [lib.conv_path_name(i).decode() for i in range(12)] == ["auto", "main", "flatk", "rows",
                                                                   "direct", "brick", "strip", "runs",
                                                                   "grouped", "slab", "phase", "staged"]


EXPECTED_PATHS = {
    "c1_conv3d_fp32_n1_8c16_o32": "runs",
    "c2_conv2d_fp16_n32_56c256_o256": "slab",
    "c4a_conv3d_fp16_n4_32c128_o128": "slab",
    "c4b_conv3d_fp16_n1_64c64_o128": "slab",
    "c4c_conv3d_fp16_n4_32c64_o128_s2": "phase",
    "c5a_conv3d_bf16_n4_32c65_o65": "staged",
    "c5b_conv3d_bf16_n4_16c21_o21": "runs",
    "c5c_conv3d_bf16_n4_32c64_o128_k311": "main",
    "c5d_conv3d_bf16_n4_32c64_o128_k133": "slab",
    "c3_conv2d_fp16_stem_n64_224c3_o64_k7s2": "rows",
}


@pytest.mark.parametrize("name", sorted(EXPECTED_PATHS))
def test_auto_path_choice(name):
    wl = WORKLOADS[name]
    assert igc.select_path(wl.x_shape, wl.w_shape, wl.stride, wl.padding,
                           wl.torch_dtype) == EXPECTED_PATHS[name]


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(1, 4, 4, 4, dtype=torch.float16)
    w = torch.zeros(4, 3, 3, 4, dtype=torch.float16)
    with pytest.raises(ValueError):
        igc.conv_fwd(x, w, 1, 1)



# ---- the extended descriptor: low / high pads, dilation, groups ---------------------------

def _desc_ex(**kw):
    base = dict(n=2, d=4, h=5, w=6, c_in=8, c_out=4, k_d=3, k_h=3, k_w=3, s_d=1, s_h=1, s_w=1,
                p_d=1, p_h=1, p_w=1, q_d=1, q_h=1, q_w=1, e_d=1, e_h=1, e_w=1, groups=1, dtype=1)
    base.update(kw)
    return igc.DescEx(**base)


def _out_shape_ex(d):
    out = (ctypes.c_int64 * 5)()
    rc = igc.lib().conv_out_shape_ex(ctypes.byref(d), out)
    return rc, tuple(out)


@pytest.mark.parametrize("field,value,code", [
    ("e_d", 0, -2), ("e_w", -1, -2), ("q_h", -1, -2), ("groups", 0, -2), ("groups", 3, -2),
    ("e_h", 4, -2),             # 5 + 2 < 4*(3-1)+1: empty output
    ("dtype", 9, -3),
])
def test_validation_codes_ex(field, value, code):
    rc, _ = _out_shape_ex(_desc_ex(**{field: value}))
    assert rc == code
    assert igc.lib().conv_fwd_ex(ctypes.byref(_desc_ex(**{field: value})), 16, 4096, 1 << 20, None) == code


@pytest.mark.parametrize("dims,pads,dil", [
    ((4, 5, 6), ((1, 0), (0, 2), (2, 1)), (1, 2, 1)),
    ((7, 9, 8), ((0, 0), (1, 1), (3, 0)), (2, 1, 3)),
    ((1, 11, 13), ((0, 0), (2, 3), (1, 4)), (1, 3, 2)),
])
def test_out_shape_ex_matches_oracle(dims, pads, dil):
    x_shape, w_shape, st = (2, *dims, 6), (4, 1 if dims[0] == 1 else 3, 3, 3, 3), (1, 2, 2)
    got = igc.out_shape(x_shape, w_shape, st, pads, dil, groups=2)
    expect = (2, *[oracle.out_extent_ex(dims[i], w_shape[1 + i], st[i], pads[i][0], pads[i][1], dil[i])
                   for i in range(3)], 4)
    assert got == expect


def test_plain_descriptor_equals_extended_with_symmetric_pads():
    """conv_out_shape / conv_select_path of a convfwd_desc agree with the extended calls
    for q = p and e = 1, for every workload shape."""
    for wl in WORKLOADS.values():
        assert igc.out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.padding) == \
            igc.out_shape(wl.x_shape, wl.w_shape, wl.stride, [(q, q) for q in wl.padding], 1, 1)
        d = igc.make_desc(wl.x_shape, wl.w_shape, wl.stride, wl.padding, wl.torch_dtype)
        assert igc.lib().conv_select_path(ctypes.byref(d)) == \
            igc.lib().conv_select_path_ex(ctypes.byref(igc.make_desc_ex(
                wl.x_shape, wl.w_shape, wl.stride, wl.padding, 1, 1, wl.torch_dtype)))


@pytest.mark.parametrize("path,ok", [(1, True), (7, True), (4, True), (2, False), (3, False), (5, False), (6, False)])
def test_grouped_problem_path_acceptance(path, ok):
    """Grouped problems (here C_in/G = 64): main, runs and direct take them; flat-K, rows, brick
    and strip do not (the last returns UNSUPPORTED instead of computing something else)."""
    d = _desc_ex(n=0, c_in=128, c_out=64, groups=2, w=32, p_w=1, q_w=1)
    assert igc.lib().conv_fwd_path_ex(ctypes.byref(d), path, None, None, None, None) == (0 if ok else -3)


# The slab path: fp16/bf16, C_in/G % 32 == 0, C_out % 4 == 0 and (G = 1 or C_out/G % 64 == 0),
# unit stride along h and w, K_h in {2, 3}, K_w <= 3, dilation 1 along h and w or 2 along both
# with a 3 x 3 plane (n = 0: only the rules run).
_SLAB_OK = dict(n=0, c_in=64, c_out=68, h=9, w=32)
@pytest.mark.parametrize("change,ok", [
    ({}, True), ({"k_h": 2, "p_h": 0, "q_h": 0}, True), ({"k_w": 1, "p_w": 0, "q_w": 0}, True),
    ({"dtype": 2}, True), ({"s_d": 2}, True), ({"e_d": 2}, True),
    ({"k_h": 1, "p_h": 0, "q_h": 0}, False), ({"k_h": 4, "p_h": 2}, False), ({"k_w": 4, "p_w": 2}, False),
    ({"s_h": 2}, False), ({"e_h": 2, "p_h": 2, "q_h": 2}, False), ({"s_w": 2, "w": 63}, False),
    ({"w": 33}, True), ({"w": 7}, True), ({"c_in": 48}, False), ({"c_out": 66}, False), ({"dtype": 0}, False),
    ({"groups": 2, "c_out": 64}, False),                     # 32 outputs per group
    ({"groups": 2, "c_out": 128}, True),                     # 64 outputs per group: 64-wide tiles
    ({"e_h": 2, "e_w": 2, "p_h": 2, "q_h": 2, "p_w": 2, "q_w": 2}, True),                  # dilated 3 x 3
    ({"e_h": 2, "e_w": 2, "p_h": 2, "q_h": 2, "p_w": 2, "q_w": 2, "groups": 2, "c_out": 128}, True),
    ({"e_h": 2, "e_w": 2, "k_w": 2, "p_h": 2, "q_h": 2, "p_w": 1, "q_w": 1}, False),     # dilated 3 x 2
    ({"e_h": 2, "e_w": 2, "k_h": 2, "p_h": 1, "q_h": 1, "p_w": 2, "q_w": 2}, False),     # dilated 2 x 3
    ({"e_h": 3, "e_w": 3, "p_h": 3, "q_h": 3, "p_w": 3, "q_w": 3}, False),
    ({"e_w": 2, "p_w": 2, "q_w": 2}, False),                 # dilated along w only
])
def test_slab_path_acceptance(change, ok):
    d = _desc_ex(**{**_SLAB_OK, **change})
    assert _out_shape_ex(d)[0] == 0
    assert igc.lib().conv_fwd_path_ex(ctypes.byref(d), 9, None, None, None, None) == (0 if ok else -3)


@pytest.mark.parametrize("path,ok", [(1, True), (7, True), (4, True), (6, False), (2, False)])
def test_w_dilated_problem_path_acceptance(path, ok):
    d = _desc_ex(n=0, c_in=64, c_out=64, w=40, e_w=2, p_w=2, q_w=2)
    assert igc.lib().conv_fwd_path_ex(ctypes.byref(d), path, None, None, None, None) == (0 if ok else -3)


def test_auto_path_for_variants():
    assert igc.select_path((2, 8, 8, 8, 128), (64, 3, 3, 3, 64), 1, 1, torch.float16, groups=2) == "main"
    assert igc.select_path((2, 8, 8, 8, 32), (32, 3, 3, 3, 1), 1, 1, torch.float16, groups=32) == "grouped"
    assert igc.select_path((2, 8, 8, 8, 96), (96, 3, 3, 3, 3), 1, 1, torch.float16, groups=32) == "runs"
    assert igc.select_path((2, 16, 16, 64), (64, 3, 3, 64), 1, 2, torch.float16, dilation=2) == "main"
    assert igc.select_path((8, 64, 64, 256), (256, 3, 3, 256), 1, 2, torch.float16, dilation=2) == "slab"
    assert igc.select_path((2, 8, 8, 32, 64), (64, 3, 3, 3, 64), 1, 1, torch.float16, dilation=(2, 2, 1)) == "strip"


# ---- backward-data entry points (host-side checks only) ---------------------------

def test_bwd_data_validation_and_pointer_rules():
    lib = igc.lib()
    d = _desc()
    xb, wb = 2 * 4 * 5 * 6 * 8 * 2, 4 * 27 * 8 * 2
    base = 1 << 24
    # the descriptor is validated first
    assert lib.conv_bwd_data(ctypes.byref(_desc(s_h=0)), base, base, base, None) == -2
    assert lib.conv_bwd_data_filter(ctypes.byref(_desc(k_w=0)), base, base, None) == -2
    assert lib.conv_bwd_data(None, base, base, base, None) == -1
    # NULL tensors
    assert lib.conv_bwd_data(ctypes.byref(d), None, base, base + (1 << 22), None) == -1
    assert lib.conv_bwd_data_filter(ctypes.byref(d), base, None, None) == -1
    # dx overlapping dy or wt, wt overlapping w
    assert lib.conv_bwd_data(ctypes.byref(d), base, base + (1 << 22), base + 64, None) == -5
    assert lib.conv_bwd_data(ctypes.byref(d), base, base + (1 << 22), base + (1 << 22) - xb + 2, None) == -5
    assert lib.conv_bwd_data_filter(ctypes.byref(d), base, base + wb - 2, None) == -5
    # empty batch: nothing launched, pointers not read
    assert lib.conv_bwd_data(ctypes.byref(_desc(n=0)), None, None, None, None) == 0


def test_bwd_data_stride_limit_and_forced_paths():
    lib = igc.lib()
    ex = _desc_ex(n=0, w=40, s_w=17, k_w=3)
    assert lib.conv_bwd_data_path_ex(ctypes.byref(ex), 0, None, None, None, None) == -3
    assert lib.conv_bwd_data_filter_ex(ctypes.byref(ex), 16, 4096, None) == -3
    ex = _desc_ex(n=0, w=40, s_w=16, k_w=3)
    assert lib.conv_bwd_data_path_ex(ctypes.byref(ex), 0, None, None, None, None) == 0
    # phases run on main, runs or direct only; main needs C_out % 32 == 0 (dy channels)
    ex = _desc_ex(n=0, c_in=8, c_out=64, s_d=2, s_h=2, s_w=2)
    for path, rc in ((1, 0), (7, 0), (4, 0), (2, -3), (6, -3), (3, -3), (5, -3), (8, -3)):
        assert lib.conv_bwd_data_path_ex(ctypes.byref(ex), path, None, None, None, None) == rc, path
    ex = _desc_ex(n=0, c_in=8, c_out=65)
    assert lib.conv_bwd_data_path_ex(ctypes.byref(ex), 1, None, None, None, None) == -3


# ---- measured selection table (host-side checks only) -------------------------------

def test_tune_table_host_rules():
    lib = igc.lib()
    assert lib.conv_tune_clear() == 0
    ex = _desc_ex()
    assert lib.conv_tuned_path_ex(ctypes.byref(ex)) == 0            # nothing recorded
    assert lib.conv_tuned_path_ex(ctypes.byref(_desc_ex(k_h=0))) == -2
    us = ctypes.c_float(0)
    base = 1 << 24
    assert lib.conv_tune_ex(None, base, base, base, None, 5, ctypes.byref(us)) == -1
    assert lib.conv_tune_ex(ctypes.byref(ex), base, base + (1 << 20), base + (1 << 21), None, 0, None) == -2
    assert lib.conv_tune_ex(ctypes.byref(ex), None, base, base + (1 << 21), None, 5, None) == -1
    assert lib.conv_tune_ex(ctypes.byref(ex), base, base + (1 << 20), base + 64, None, 5, None) == -5
    # an empty batch times nothing and records nothing
    empty = _desc_ex(n=0)
    assert lib.conv_tune_ex(ctypes.byref(empty), None, None, None, None, 5, None) == \
        lib.conv_select_path_ex(ctypes.byref(empty))
    assert lib.conv_tuned_path_ex(ctypes.byref(empty)) == 0
    assert igc.tuned_path((2, 4, 5, 6, 8), (4, 3, 3, 3, 8), 1, 1) is None


# ---- pointer alignment (host-side checks only: every call below returns before a launch) ----

def test_forced_16_byte_paths_refuse_tensors_not_16_byte_aligned():
    """The slab, strip and main kernels move 16-byte pieces counted from the base pointers:
    forced onto them, an element-aligned but not 16-byte-aligned x, w or y is refused with
    UNSUPPORTED before any launch (AUTO would take the tail path instead)."""
    lib = igc.lib()
    d = _desc(n=1, d=4, h=6, w=32, c_in=64, c_out=64)     # slab, strip and main all take it
    base = 1 << 24
    x, w, y = base, base + (1 << 22), base + (1 << 23)
    for path in (1, 6, 9):
        for dx, dw, dy in ((2, 0, 0), (0, 2, 0), (0, 0, 2), (8, 8, 8)):
            assert lib.conv_fwd_path(ctypes.byref(d), path, x + dx, w + dw, y + dy, None) == -3, (path, dx, dw, dy)
    # the same pointers aligned pass every host check (a forced path with n = 0 launches nothing)
    d0 = _desc(n=0, d=4, h=6, w=32, c_in=64, c_out=64)
    for path in (1, 6, 9):
        assert lib.conv_fwd_path(ctypes.byref(d0), path, x, w, y, None) == 0
    # the descriptor-only choice assumes aligned tensors
    assert lib.conv_select_path(ctypes.byref(d)) == 6   # strip: 6 of 16 slab rows would be used
    # the stride-2 path likewise
    d2 = _desc(n=1, d=4, h=12, w=32, c_in=64, c_out=64, s_h=2, s_w=2)
    assert lib.conv_select_path(ctypes.byref(d2)) == 10
    assert lib.conv_fwd_path(ctypes.byref(d2), 10, x, w + 2, y, None) == -3
    assert lib.conv_fwd_path(ctypes.byref(_desc(n=0, d=4, h=12, w=32, c_in=64, c_out=64, s_h=2, s_w=2)),
                             10, x, w, y, None) == 0


def test_pointers_not_aligned_to_their_element_are_rejected():
    lib = igc.lib()
    base = 1 << 24
    x, w, y = base, base + (1 << 22), base + (1 << 23)
    d16 = _desc(n=1, d=4, h=6, w=32, c_in=64, c_out=64)
    assert lib.conv_fwd(ctypes.byref(d16), x + 1, w, y, None) == -7
    assert lib.conv_fwd_path(ctypes.byref(d16), 7, x, w + 1, y, None) == -7   # runs
    assert lib.conv_fwd_path(ctypes.byref(d16), 4, x, w, y + 3, None) == -7   # direct
    d32 = _desc(n=1, d=4, h=6, w=8, c_in=16, c_out=32, dtype=0)
    assert lib.conv_fwd(ctypes.byref(d32), x + 2, w, y, None) == -7
    assert lib.conv_tune(ctypes.byref(d16), x, w, y + 1, None, 5, None) == -7
    assert lib.conv_strerror(-7).decode().startswith("a tensor pointer")


def test_bwd_data_alignment_rules():
    lib = igc.lib()
    base = 1 << 24
    dy, wt, dx = base, base + (1 << 22), base + (1 << 23)
    ex = _desc_ex(n=1, c_in=8, c_out=64, s_d=2, s_h=2, s_w=2)
    # forced main needs every phase's tensors 16-byte aligned
    assert lib.conv_bwd_data_path_ex(ctypes.byref(ex), 1, dy + 2, wt, dx, None) == -3
    assert lib.conv_bwd_data_path_ex(ctypes.byref(ex), 1, dy, wt, dx + 8, None) == -3
    # not even element-aligned: rejected on every path, before any launch
    assert lib.conv_bwd_data_ex(ctypes.byref(ex), dy + 1, wt, dx, None) == -7
    assert lib.conv_bwd_data_path_ex(ctypes.byref(ex), 4, dy, wt + 1, dx, None) == -7
    assert lib.conv_bwd_data_filter_ex(ctypes.byref(ex), dy + 1, wt, None) == -7


def test_binding_checks_filter_and_buffers_before_any_launch():
    """The binding compares w with x (rank, C_in/groups channels) and a caller's out / wt
    buffers with the shape, dtype and device the call will write or read: the library sizes
    every access from the descriptor, so a mismatch must be caught before the call."""
    igc._check_filter((1, 4, 4, 4, 64), (8, 3, 3, 3, 64), 1)
    igc._check_filter((1, 4, 4, 4, 64), (8, 3, 3, 3, 32), 2)
    with pytest.raises(ValueError):
        igc._check_filter((1, 4, 4, 4, 64), (8, 3, 3, 3, 32), 1)       # half the channels
    with pytest.raises(ValueError):
        igc._check_filter((1, 4, 4, 4, 64), (8, 3, 3, 3, 128), 1)      # twice the channels
    with pytest.raises(ValueError):
        igc._check_filter((1, 4, 4, 64), (8, 3, 3, 3, 64), 1)          # rank
    like = torch.zeros(2, 3, dtype=torch.float16)
    igc._check_out(torch.zeros(4, 5, dtype=torch.float16), (4, 5), like)
    for bad in (torch.zeros(4, 6, dtype=torch.float16), torch.zeros(4, 5, dtype=torch.bfloat16),
                torch.zeros(5, 4, dtype=torch.float16).t()):
        with pytest.raises(ValueError):
            igc._check_out(bad, (4, 5), like)
