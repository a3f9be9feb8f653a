"""GPU parity: the HIP library against the float64 oracle, element by element.

Every case draws seeded inputs from conv_workloads, runs the library through
the C ABI (via the thin Python binding) on one forced path or on the path the
library picks, and compares with the oracle under the tolerances in
tests/parity.py.  Integer-valued cases (tap counts, one-hot gathers) are
compared bit for bit.  Full-size workloads run in the launch configuration the
bench times and every output element is compared with the oracle.
"""
import zlib

import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
import oracle
from conv_workloads import VARIANT_WORKLOADS, WORKLOADS, Workload, make_inputs
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(name, dtype, xs, ws, st, pd, x_dist="uniform", seed=7):
    return Workload(name, dtype, tuple(xs), tuple(ws), tuple(st), tuple(pd), x_dist,
                    seed * 10 + 1, seed * 10 + 2)


# Reduced shapes: several tiles plus ragged M (and N) tails, same channel and
# filter structure as the full workloads, plus the degenerate cases.
CASES = [
    _case("c4_like_fp16_c64", "fp16", (2, 9, 10, 11, 64), (128, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1), seed=1),
    _case("c4a_like_fp16_c128", "fp16", (1, 6, 7, 9, 128), (128, 3, 3, 3, 128), (1, 1, 1), (1, 1, 1), seed=2),
    _case("c4c_like_fp16_s2", "fp16", (2, 11, 12, 13, 64), (128, 3, 3, 3, 64), (2, 2, 2), (1, 1, 1), seed=3),
    _case("c5c_like_bf16_k311", "bf16", (2, 8, 9, 10, 64), (128, 3, 1, 1, 64), (1, 1, 1), (1, 0, 0), seed=4),
    _case("c5d_like_bf16_k133", "bf16", (2, 8, 9, 10, 64), (128, 1, 3, 3, 64), (1, 1, 1), (0, 1, 1), seed=5),
    _case("c2_like_fp16_2d_c256_o96", "fp16", (3, 13, 14, 256), (96, 3, 3, 256), (1, 1), (1, 1), seed=6),
    _case("fp16_2d_o4", "fp16", (2, 9, 9, 64), (4, 3, 3, 64), (1, 1), (1, 1), seed=7),
    _case("fp16_2d_o260", "fp16", (1, 7, 9, 128), (260, 3, 3, 128), (1, 1), (1, 1), seed=8),
    _case("fp16_s3_pad3", "fp16", (1, 7, 8, 9, 64), (64, 3, 3, 3, 64), (3, 3, 3), (3, 3, 3), seed=9),
    _case("bf16_2d_k5", "bf16", (2, 12, 13, 64), (32, 5, 5, 64), (1, 1), (2, 2), seed=10),
    _case("c5a_like_bf16_c65", "bf16", (2, 7, 8, 9, 65), (65, 3, 3, 3, 65), (1, 1, 1), (1, 1, 1), seed=11),
    _case("c5b_like_bf16_c21", "bf16", (3, 6, 7, 8, 21), (21, 3, 3, 3, 21), (1, 1, 1), (1, 1, 1), seed=12),
    _case("c3_like_fp16_stem", "fp16", (2, 30, 32, 3), (64, 7, 7, 3), (2, 2), (3, 3), "normal", seed=13),
    _case("stem_wide_ragged_bf16", "bf16", (1, 11, 240, 3), (40, 7, 7, 3), (2, 2), (3, 3), "normal", seed=19),
    _case("tiny_c3_3d_fp16", "fp16", (2, 5, 9, 8, 3), (32, 3, 3, 3, 3), (1, 1, 1), (1, 1, 1), seed=20),
    _case("c1_fp32", "fp32", (1, 8, 8, 8, 16), (32, 3, 3, 3, 16), (1, 1, 1), (1, 1, 1), seed=14),
    _case("fp32_odd", "fp32", (2, 5, 6, 7, 5), (7, 3, 2, 3, 5), (1, 2, 1), (1, 0, 2), seed=15),
    _case("fp16_c16", "fp16", (2, 6, 6, 6, 16), (32, 3, 3, 3, 16), (1, 1, 1), (1, 1, 1), seed=16),
    _case("bf16_c1_single_output", "bf16", (1, 3, 3, 1), (1, 3, 3, 1), (1, 1), (0, 0), seed=17),
    _case("fp16_1x1_pointwise", "fp16", (2, 5, 7, 64), (64, 1, 1, 64), (1, 1), (0, 0), seed=18),
    _case("strip_fp16_c64_w32", "fp16", (2, 5, 6, 32, 64), (128, 3, 3, 3, 64), (1, 1, 1), (1, 1, 1), seed=21),
    _case("strip_bf16_c96_w64_o72", "bf16", (1, 4, 5, 64, 96), (72, 3, 3, 3, 96), (1, 1, 1), (1, 1, 1), seed=22),
    _case("strip_fp16_2d_k5_o132", "fp16", (3, 9, 32, 32), (132, 5, 5, 32), (1, 1), (1, 2), seed=23),
    _case("strip_fp16_hs2_w32", "fp16", (2, 7, 9, 34, 64), (64, 3, 3, 3, 64), (2, 2, 1), (1, 0, 0), seed=24),
    _case("slab_bf16_k2_o36_sd2", "bf16", (2, 3, 9, 33, 32), (36, 2, 2, 2, 32), (2, 1, 1), (0, 0, 0), seed=25),
    _case("slab_fp16_2d_k3x1_o68", "fp16", (2, 21, 32, 32), (68, 3, 1, 32), (1, 1), (1, 0), seed=26),
    _case("slab_fp16_h35_w64_two_wblocks", "fp16", (1, 2, 35, 64, 32), (64, 3, 3, 3, 32), (1, 1, 1), (1, 1, 1),
          seed=27),
    _case("slab_fp16_2d_w56_ragged", "fp16", (2, 12, 56, 64), (64, 3, 3, 64), (1, 1), (1, 1), seed=28),
    _case("slab_bf16_w9_narrow", "bf16", (1, 3, 5, 9, 32), (40, 2, 2, 3, 32), (1, 1, 1), (0, 0, 1), seed=29),
    # an odd filter element count (7 x 27): the rows path copies its filter in 16-byte pieces
    _case("rows_odd_filter_fp16", "fp16", (1, 9, 16, 3), (7, 3, 3, 3), (1, 1), (1, 1), seed=30),
    # stride 2 along h and w: ragged h, w and C_out tiles, two 64-channel chunks, 2 x 2 filters
    _case("phase_fp16_c128_o68_ragged", "fp16", (1, 5, 19, 37, 128), (68, 3, 3, 3, 128), (1, 2, 2), (1, 1, 1),
          seed=31),
    _case("phase_bf16_2d_s2", "bf16", (3, 29, 35, 64), (64, 3, 3, 64), (2, 2), (1, 1), seed=32),
    _case("phase_fp16_2d_k2", "fp16", (2, 17, 18, 64), (72, 2, 2, 64), (2, 2), (0, 0), seed=33),
    _case("phase_fp16_k233_pad0", "fp16", (1, 7, 16, 16, 64), (64, 2, 3, 3, 64), (2, 2, 2), (0, 0, 0), seed=34),
    _case("phase_bf16_k32_o200", "bf16", (1, 4, 18, 23, 192), (200, 1, 3, 2, 192), (1, 2, 2), (0, 1, 1), seed=35),
    _case("phase_fp16_2d_k23_o48", "fp16", (2, 15, 21, 64), (48, 2, 3, 64), (2, 2), (0, 1), seed=61),
    # C_in not a multiple of 8: 32-channel chunks plus the packed leftover block; ragged h and w
    # blocks, 80-, 64- and 32-channel tiles, two column tiles (element-wise stores), pack only
    _case("staged_bf16_c65_o65_ragged", "bf16", (1, 5, 19, 37, 65), (65, 3, 3, 3, 65), (1, 1, 1), (1, 1, 1),
          seed=36),
    _case("staged_fp16_c9_one_piece", "fp16", (2, 6, 20, 33, 9), (24, 3, 3, 3, 9), (1, 1, 1), (1, 1, 1), seed=37),
    _case("staged_bf16_2d_c11_o40", "bf16", (3, 21, 40, 11), (40, 3, 3, 11), (1, 1), (1, 1), seed=38),
    _case("staged_fp16_c40_partial_chunk", "fp16", (1, 4, 18, 34, 40), (33, 3, 3, 3, 40), (1, 1, 1), (1, 1, 1),
          seed=39),
    _case("staged_fp16_2d_c33_o130_kw2", "fp16", (2, 18, 35, 33), (130, 3, 2, 33), (1, 1), (1, 0), seed=40),
    _case("staged_bf16_k223_c66_o70", "bf16", (1, 3, 17, 33, 66), (70, 2, 2, 3, 66), (1, 1, 1), (0, 1, 1),
          seed=41),
    _case("staged_fp16_2d_c24_o16", "fp16", (2, 16, 64, 24), (16, 3, 3, 24), (1, 1), (1, 1), seed=42),
    _case("staged_bf16_sd2_c17_o48", "bf16", (2, 9, 16, 32, 17), (48, 3, 3, 3, 17), (2, 1, 1), (1, 1, 1), seed=43),
]
PATHS = ["slab", "phase", "staged", "strip", "main", "brick", "rows", "runs", "flatk", "direct"]


def _accepts(wl, path):
    half = wl.dtype in ("fp16", "bf16") and wl.w_shape[0] % 4 == 0
    taps = int(np.prod(wl.w_shape[1:-1]))
    if path == "main":
        return half and wl.x_shape[-1] % 32 == 0
    if path == "strip":
        ow = (wl.x_shape[-2] + 2 * wl.padding[-1] - wl.w_shape[-2]) // wl.stride[-1] + 1
        return (half and wl.x_shape[-1] % 32 == 0 and wl.stride[-1] == 1 and ow % 32 == 0
                and wl.w_shape[-2] <= 5)
    if path == "slab":
        return (half and wl.x_shape[-1] % 32 == 0 and wl.stride[-1] == 1 and wl.stride[-2] == 1
                and wl.w_shape[-2] <= 3 and wl.w_shape[-3] in (2, 3))
    if path == "phase":
        return (half and wl.x_shape[-1] % 64 == 0 and wl.stride[-1] == 2 and wl.stride[-2] == 2
                and wl.w_shape[-2] in (2, 3) and wl.w_shape[-3] in (2, 3))
    if path == "staged":
        cin = wl.x_shape[-1]
        kd = wl.w_shape[1] if len(wl.w_shape) == 5 else 1
        return (wl.dtype in ("fp16", "bf16") and wl.stride[-1] == 1 and wl.stride[-2] == 1
                and wl.w_shape[-2] in (2, 3) and wl.w_shape[-3] in (2, 3) and cin >= 8
                and (cin % 8) * taps <= 32 and (cin % 8 == 0 or kd <= 3))
    if path == "brick":
        return half and wl.x_shape[-1] % 16 == 0 and taps >= 4
    if path == "rows":
        cin, kw = wl.x_shape[-1], wl.w_shape[-2]
        return (wl.dtype in ("fp16", "bf16") and cin < 16 and cin * kw <= 32
                and wl.w_shape[0] <= 64 and (wl.x_shape[-2] * cin) % 8 == 0)
    return True


def _run(wl, path="auto", x=None, w=None):
    if x is None:
        x, w = make_inputs(wl, DEV)
    y = igc.conv_fwd(x, w, wl.stride, wl.padding, path=path)
    torch.cuda.synchronize()
    return x, w, y


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_parity_reduced(wl, path):
    if not _accepts(wl, path):
        pytest.skip(f"{path} does not take {wl.name}")
    print(f"[parity] {wl.name} path={path}", flush=True)
    x, w, y = _run(wl, path)
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), wl.stride, wl.padding)
    assert_parity(oracle.to_float64(y), ref, wl.dtype, f"{wl.name}/{path}")


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_auto_path_is_deterministic(wl):
    x, w, y1 = _run(wl)
    _, _, y2 = _run(wl, x=x, w=w)
    assert torch.equal(y1.view(torch.uint8) if y1.dtype != torch.float32 else y1.view(torch.int32),
                       y2.view(torch.uint8) if y2.dtype != torch.float32 else y2.view(torch.int32))


# The runs path picks its tile by the number of 64-row tiles: under half a tile
# per CU, 16-row tiles whose four waves split the K walk; under two per CU, the
# same with 32-row tiles; else 64-row tiles with the steps staged through LDS.
# On a 256-CU MI355X these shapes take each variant (M = 1785 and 512: 16 rows;
# 16384: 32 rows; 32768: 64 rows), with ragged row and column tails, 32- and
# 64-column tiles, bf16 with C_in = 21 (2-byte aligned rows) and fp32.
RUNS_TILE_CASES = [
    _case("runs_bf16_c21_m1785", "bf16", (1, 7, 15, 17, 21), (21, 3, 3, 3, 21), (1, 1, 1), (1, 1, 1), seed=62),
    _case("runs_fp32_c16_o40_m512", "fp32", (1, 8, 8, 8, 16), (40, 3, 3, 3, 16), (1, 1, 1), (1, 1, 1), seed=63),
    _case("runs_bf16_c21_o50_m16384", "bf16", (2, 8, 32, 32, 21), (50, 3, 3, 3, 21), (1, 1, 1), (1, 1, 1), seed=64),
    _case("runs_bf16_c21_m32768", "bf16", (2, 16, 32, 32, 21), (21, 3, 3, 3, 21), (1, 1, 1), (1, 1, 1), seed=65),
]


@pytest.mark.parametrize("wl", RUNS_TILE_CASES, ids=[c.name for c in RUNS_TILE_CASES])
def test_runs_tile_variants(wl):
    """Each runs-path tile variant against the oracle on every output element, and repeated
    launches bit-identical (the split K walk adds its partial sums in a fixed order)."""
    print(f"[runs] {wl.name}", flush=True)
    x, w, y = _run(wl, "runs")
    _, _, y2 = _run(wl, "runs", x=x, w=w)
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), wl.stride, wl.padding)
    assert_parity(oracle.to_float64(y), ref, wl.dtype, wl.name)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_parity_full_size(name):
    """Full-size workloads on the auto path (the launch the bench times), every output element
    compared with the oracle (the multithreaded float64 loop nest over the whole output)."""
    wl = WORKLOADS[name]
    print(f"[full] {name} path={igc.select_path(wl.x_shape, wl.w_shape, wl.stride, wl.padding, wl.torch_dtype)}",
          flush=True)
    x, w, y = _run(wl)
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), wl.stride, wl.padding)
    e = assert_parity(oracle.to_float64(y), ref, wl.dtype, name)
    print(f"[full] {name} outputs={ref.size} l2_rel={e['l2_rel']:.2e} max_rel={e['max_rel']:.2e}", flush=True)


@pytest.mark.parametrize("xs,ws,st,pd", [
    ((1, 17, 61, 64, 64), (132, 3, 1, 1, 64), (1, 1, 1), (1, 0, 0)),   # K = 192, ragged M and N tiles
    ((2, 130, 260, 96), (256, 1, 1, 96), (1, 1), (0, 0)),               # 1x1, K = 96
], ids=["3x1x1_c132_ragged", "1x1_2d_c256"])
def test_main_short_depth_tiles(xs, ws, st, pd):
    """Problems with a short GEMM depth and at least 512 tiles of 128x128 take the main path's
    short-depth tile (BK = 32, 32x32x16, three workgroups per CU); checked on every output."""
    wl = _case("short_k", "bf16", xs, ws, st, pd, seed=31)
    assert igc.select_path(xs, ws, st, pd, torch.bfloat16) == "main"
    print(f"[short-k] {xs} {ws}", flush=True)
    x, w, y = _run(wl)
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pd)
    assert_parity(oracle.to_float64(y), ref, "bf16", f"short-k {xs}")


@pytest.mark.parametrize("dtype,xs,ws,pd,dil", [
    ("fp16", (64, 2, 17, 33, 32), (196, 3, 3, 3, 32), ((1, 1), (1, 1), (1, 1)), (1, 1, 1)),  # ragged h, w, C_out
    ("bf16", (64, 20, 36, 64), (132, 3, 3, 64), ((2, 2), (2, 2)), (2, 2)),                   # dilated 3 x 3
], ids=["3d_c196_ragged", "2d_dilated2_c132"])
def test_slab_wide_tiles(dtype, xs, ws, pd, dil):
    """Problems with at least as many 128-channel tiles as compute units (1024 and 512 here)
    take the slab path's 128-channel tile; smaller ones take 64-channel tiles.  Every output
    is compared with the oracle."""
    st = (1,) * (len(xs) - 2)
    print(f"[slab wide] {xs} {ws} dil={dil}", flush=True)
    gen = torch.Generator("cpu").manual_seed(zlib.crc32(repr(xs).encode()))
    x = (torch.rand(xs, generator=gen) * 2 - 1).to(_dt(dtype)).to(DEV)
    w = (torch.randn(ws, generator=gen) / np.sqrt(np.prod(ws[1:]))).to(_dt(dtype)).to(DEV)
    y = igc.conv_fwd(x, w, st, pd, path="slab", dilation=dil)
    torch.cuda.synchronize()
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pd, dilation=dil)
    assert_parity(oracle.to_float64(y), ref, dtype, f"slab wide {xs}")


# ---- bit-exact index and boundary handling ----------------------------------------

EXACT = [
    ("main", "fp16", (2, 5, 6, 7, 64), (3, 3, 3), (1, 1, 1), (1, 1, 1)),
    ("strip", "fp16", (2, 5, 6, 32, 64), (3, 3, 3), (1, 1, 1), (1, 1, 1)),
    ("strip", "bf16", (1, 6, 7, 33, 32), (3, 2, 2), (2, 2, 1), (2, 1, 0)),
    ("slab", "fp16", (2, 5, 6, 32, 64), (3, 3, 3), (1, 1, 1), (1, 1, 1)),
    ("slab", "bf16", (1, 6, 19, 33, 32), (3, 2, 2), (2, 1, 1), (2, 1, 0)),
    ("slab", "fp16", (2, 3, 21, 64, 32), (1, 3, 1), (1, 1, 1), (0, 1, 0)),
    ("brick", "fp16", (2, 5, 6, 7, 64), (3, 3, 3), (1, 1, 1), (1, 1, 1)),
    ("brick", "bf16", (1, 6, 7, 9, 32), (3, 3, 3), (2, 2, 2), (2, 1, 3)),
    ("brick", "fp16", (2, 3, 9, 40, 16), (1, 5, 3), (1, 1, 2), (0, 2, 1)),
    ("main", "bf16", (1, 6, 7, 9, 64), (3, 3, 3), (2, 2, 2), (2, 1, 3)),
    ("flatk", "bf16", (2, 5, 6, 7, 5), (3, 3, 3), (1, 2, 1), (1, 1, 2)),
    ("flatk", "fp32", (1, 4, 9, 8, 3), (1, 7, 7), (1, 2, 2), (0, 3, 3)),
    ("flatk", "fp16", (2, 5, 6, 7, 65), (3, 3, 3), (3, 1, 2), (3, 1, 0)),
    ("runs", "bf16", (2, 5, 6, 7, 5), (3, 3, 3), (1, 2, 1), (1, 1, 2)),
    ("runs", "fp32", (1, 4, 9, 8, 3), (1, 7, 7), (1, 2, 2), (0, 3, 3)),
    ("runs", "fp16", (2, 5, 6, 7, 65), (3, 3, 3), (3, 1, 2), (3, 1, 0)),
    ("runs", "bf16", (1, 4, 5, 40, 21), (3, 3, 5), (1, 1, 1), (1, 1, 2)),
    ("runs", "fp32", (2, 3, 4, 5, 33), (2, 3, 3), (1, 1, 1), (1, 1, 1)),
    ("direct", "fp16", (1, 5, 6, 7, 3), (3, 3, 3), (2, 2, 2), (1, 1, 1)),
    ("rows", "fp16", (1, 1, 19, 16, 3), (1, 7, 7), (1, 2, 2), (0, 3, 3)),
    ("rows", "bf16", (2, 5, 9, 8, 3), (3, 3, 3), (1, 1, 1), (1, 1, 1)),
    ("phase", "fp16", (2, 5, 17, 18, 64), (3, 3, 3), (1, 2, 2), (1, 1, 1)),
    ("phase", "bf16", (1, 6, 19, 33, 128), (3, 2, 3), (2, 2, 2), (2, 0, 1)),
    ("phase", "fp16", (1, 4, 20, 21, 64), (2, 2, 2), (1, 2, 2), (0, 1, 0)),
    ("staged", "bf16", (1, 4, 17, 35, 65), (3, 3, 3), (1, 1, 1), (1, 1, 1)),
    ("staged", "fp16", (2, 3, 16, 33, 17), (3, 2, 3), (2, 1, 1), (1, 0, 2)),
    ("staged", "fp16", (1, 2, 18, 32, 10), (2, 3, 2), (1, 1, 1), (1, 1, 0)),
    ("staged", "bf16", (2, 17, 40, 40), (3, 3), (1, 1), (1, 1)),
]


def _dt(name):
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[name]


@pytest.mark.parametrize("path,dtype,xs,ks,st,pd", EXACT)
def test_tap_count_bit_exact(path, dtype, xs, ks, st, pd):
    """x = 1, w = 1 on input channel 0 only: every output is its number of in-bounds taps."""
    cin = xs[-1]
    cout = 8
    x = torch.ones(xs, dtype=_dt(dtype), device=DEV)
    w = torch.zeros((cout, *ks, cin), dtype=_dt(dtype), device=DEV)
    w[..., 0] = 1
    y = igc.conv_fwd(x, w, st, pd, path=path)
    torch.cuda.synchronize()
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pd)
    np.testing.assert_array_equal(oracle.to_float64(y), ref)


@pytest.mark.parametrize("path,dtype,xs,ks,st,pd", [e for e in EXACT if e[2][-1] % 8])
def test_tap_count_last_channel_bit_exact(path, dtype, xs, ks, st, pd):
    """As above on the last input channel, the one past the last 8-channel piece (on the
    staged path: packed with the other taps' leftover channels into one K block)."""
    cin = xs[-1]
    x = torch.ones(xs, dtype=_dt(dtype), device=DEV)
    w = torch.zeros((8, *ks, cin), dtype=_dt(dtype), device=DEV)
    w[..., cin - 1] = 1
    y = igc.conv_fwd(x, w, st, pd, path=path)
    torch.cuda.synchronize()
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pd)
    np.testing.assert_array_equal(oracle.to_float64(y), ref)


@pytest.mark.parametrize("path,dtype,xs,ks,st,pd", EXACT)
def test_one_hot_gather_bit_exact(path, dtype, xs, ks, st, pd):
    """w = identity on channels at one tap: y is a shifted, strided copy of x (0 in the padding)."""
    c = xs[-1]
    g = torch.Generator("cpu").manual_seed(99)
    x = (torch.rand(xs, generator=g) * 2 - 1).to(_dt(dtype)).to(DEV)
    taps = [tuple(0 for _ in ks), tuple(k - 1 for k in ks), tuple(k // 2 for k in ks)]
    for tap in taps:
        w = torch.zeros((c, *ks, c), dtype=_dt(dtype))
        w[(torch.arange(c), *[torch.full((c,), t) for t in tap], torch.arange(c))] = 1
        w = w.to(DEV)
        y = igc.conv_fwd(x, w, st, pd, path=path)
        torch.cuda.synchronize()
        ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pd)
        np.testing.assert_array_equal(oracle.to_float64(y), ref, err_msg=f"tap {tap}")


# ---- boundary behaviour -------------------------------------------------------------

def test_empty_batch_launches_nothing():
    x = torch.empty((0, 4, 4, 4, 64), dtype=torch.float16, device=DEV)
    w = torch.randn((64, 3, 3, 3, 64), device=DEV).half()
    y = igc.conv_fwd(x, w, 1, 1)
    torch.cuda.synchronize()
    assert y.shape == (0, 4, 4, 4, 64)


def test_non_contiguous_inputs_are_made_contiguous():
    wl = CASES[0]
    x, w = make_inputs(wl, DEV)
    xt = x.permute(0, 2, 1, 3, 4).contiguous().permute(0, 2, 1, 3, 4)   # same values, strided
    assert not xt.is_contiguous()
    y = igc.conv_fwd(xt, w, wl.stride, wl.padding)
    y0 = igc.conv_fwd(x, w, wl.stride, wl.padding)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


def test_no_workspace_and_no_out_of_bounds_writes():
    """The call allocates nothing and writes only inside y (canaries around it stay intact)."""
    wl = CASES[2]
    x, w = make_inputs(wl, DEV)
    shape = igc.out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.padding)
    n = int(np.prod(shape))
    guard = 4096
    buf = torch.full((n + 2 * guard,), 12345.0, dtype=torch.float16, device=DEV)
    y = buf[guard:guard + n].view(shape)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    igc.conv_fwd(x, w, wl.stride, wl.padding, out=y)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + n:] == 12345.0)
    ref = igc.conv_fwd(x, w, wl.stride, wl.padding)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


def test_wrong_out_rejected():
    x = torch.zeros((1, 4, 4, 4, 64), dtype=torch.float16, device=DEV)
    w = torch.zeros((64, 3, 3, 3, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        igc.conv_fwd(x, w, 1, 1, out=torch.empty((1, 4, 4, 4, 63), dtype=torch.float16, device=DEV))
    with pytest.raises(igc.ConvError):
        igc.conv_fwd(x, w, 1, 1, path="rows")


# ---- the variants: grouped, dilated, padded differently per side -------------------------

VARIANTS = [
    # name, dtype, x shape, w shape (C_in/G last), stride, (low, high) pads, dilation, groups
    ("grouped3d_bf16_g2_c64", "bf16", (2, 6, 7, 9, 128), (64, 3, 3, 3, 64), (1, 1, 1),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 2),
    ("resnext2d_fp16_g32_c4", "fp16", (2, 14, 15, 128), (128, 3, 3, 4), (1, 1), ((1, 1), (1, 1)), (1, 1), 32),
    ("depthwise2d_fp16_c48", "fp16", (2, 16, 17, 48), (48, 3, 3, 1), (1, 1), ((1, 1), (1, 1)), (1, 1), 48),
    ("dilated2d_fp16_e2", "fp16", (2, 20, 33, 64), (64, 3, 3, 64), (1, 1), ((2, 2), (2, 2)), (2, 2), 1),
    ("dilated3d_bf16_dh2_w32", "bf16", (1, 7, 9, 32, 64), (64, 3, 3, 3, 64), (1, 1, 1),
     ((2, 2), (2, 2), (1, 1)), (2, 2, 1), 1),
    ("asympad3d_fp16_w32", "fp16", (2, 5, 6, 32, 64), (128, 3, 3, 3, 64), (1, 1, 1),
     ((0, 2), (1, 0), (0, 2)), (1, 1, 1), 1),
    ("grouped_dilated_fp32", "fp32", (1, 5, 6, 7, 12), (6, 3, 2, 3, 4), (1, 1, 1),
     ((1, 1), (2, 0), (1, 2)), (1, 2, 2), 3),
    ("all_variants_bf16_g2", "bf16", (2, 9, 10, 11, 128), (64, 3, 3, 3, 64), (2, 1, 2),
     ((2, 1), (0, 1), (3, 2)), (2, 1, 2), 2),
    ("grouped_odd_channels_bf16", "bf16", (2, 5, 6, 7, 45), (30, 3, 3, 3, 15), (1, 1, 1),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 3),
    ("depthwise3d_bf16_mult2_s2", "bf16", (2, 7, 9, 11, 24), (48, 3, 3, 3, 1), (2, 2, 2),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 24),
    ("grouped2d_fp32_cg8_og16_dh2", "fp32", (2, 10, 13, 64), (128, 3, 3, 8), (1, 1),
     ((2, 2), (1, 1)), (2, 1), 8),
    ("grouped2d_fp16_cg16_og8_k5_s2", "fp16", (1, 12, 19, 64), (32, 5, 5, 16), (1, 2),
     ((2, 2), (2, 1)), (1, 1), 4),
    ("grouped2d_bf16_cg2_og3", "bf16", (2, 9, 10, 12), (18, 3, 3, 2), (1, 1),
     ((0, 1), (1, 1)), (1, 1), 6),
    ("depthwise2d_fp32_k5_s2_tail", "fp32", (2, 13, 23, 20), (20, 5, 5, 1), (2, 2),
     ((2, 2), (2, 2)), (1, 1), 20),
    ("depthwise3d_bf16_k7_tail", "bf16", (1, 5, 9, 19, 16), (16, 3, 3, 7, 1), (1, 1, 1),
     ((1, 1), (1, 1), (3, 3)), (1, 1, 1), 16),
    ("grouped2d_fp16_cg8_k7_s2", "fp16", (2, 9, 30, 32), (32, 7, 7, 8), (1, 2),
     ((3, 3), (3, 3)), (1, 1), 4),
    ("grouped2d_bf16_cg2_k1", "bf16", (2, 5, 11, 16), (16, 1, 1, 2), (1, 1),
     ((0, 0), (0, 0)), (1, 1), 8),
    ("depthwise3d_fp16_dil_dh_sh2", "fp16", (1, 8, 9, 10, 24), (24, 3, 3, 3, 1), (1, 2, 1),
     ((2, 2), (2, 1), (1, 1)), (2, 2, 1), 24),
    ("depthwise2d_bf16_k5_dh2_wide", "bf16", (2, 13, 70, 40), (40, 5, 5, 1), (1, 1),
     ((4, 4), (2, 2)), (2, 1), 40),
    ("depthwise3d_fp32_k3_ragged", "fp32", (2, 6, 7, 37, 12), (12, 3, 3, 3, 1), (2, 1, 1),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 12),
    ("grouped3d_fp16_g2_cg64_og64", "fp16", (1, 3, 18, 35, 128), (128, 3, 3, 3, 64), (1, 1, 1),
     ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 2),
    ("grouped2d_bf16_g4_cg32_og64", "bf16", (2, 20, 40, 128), (256, 3, 3, 32), (1, 1),
     ((1, 1), (1, 1)), (1, 1), 4),
    ("depthwise2d_fp16_k3_odd_h", "fp16", (2, 15, 21, 32), (32, 3, 3, 1), (1, 1),
     ((1, 1), (1, 1)), (1, 1), 32),
    ("depthwise2d_fp16_k7_c64", "fp16", (2, 20, 35, 64), (64, 7, 7, 1), (1, 1),
     ((3, 3), (3, 3)), (1, 1), 64),
    ("dilated2d_fp16_e2_ragged", "fp16", (2, 21, 37, 64), (64, 3, 3, 64), (1, 1),
     ((2, 2), (2, 2)), (2, 2), 1),
    ("dilated2d_bf16_e2_o136_asym", "bf16", (2, 19, 40, 64), (136, 3, 3, 64), (1, 1),
     ((1, 2), (2, 1)), (2, 2), 1),
    ("dilated3d_fp16_e2_g2_sd2", "fp16", (1, 5, 18, 34, 128), (128, 2, 3, 3, 64), (2, 1, 1),
     ((1, 0), (2, 2), (2, 2)), (2, 2, 2), 2),
    ("phase_g2_asympad_bf16", "bf16", (2, 6, 17, 19, 128), (128, 3, 3, 3, 64), (1, 2, 2),
     ((1, 1), (0, 2), (2, 1)), (1, 1, 1), 2),
    ("phase_depth_dilated_fp16", "fp16", (1, 9, 16, 18, 64), (64, 3, 3, 2, 64), (1, 2, 2),
     ((2, 2), (1, 1), (0, 1)), (2, 1, 1), 1),
    ("staged_depth_dilated_bf16_c65", "bf16", (1, 9, 16, 33, 65), (48, 3, 3, 3, 65), (1, 1, 1),
     ((2, 2), (1, 1), (1, 1)), (2, 1, 1), 1),
    ("staged_asympad_sd2_fp16_c33", "fp16", (2, 5, 17, 40, 33), (70, 3, 2, 3, 33), (2, 1, 1),
     ((1, 0), (0, 1), (2, 0)), (1, 1, 1), 1),
]
VARIANT_PATHS = ["main", "slab", "phase", "staged", "strip", "runs", "grouped", "direct"]


def _v_accepts(v, path):
    name, dtype, xs, ws, st, pads, dil, g = v
    half = dtype in ("fp16", "bf16")
    cin_g, cout_g = xs[-1] // g, ws[0] // g
    if path == "main":
        return half and cin_g % 32 == 0 and cout_g % 4 == 0
    if path == "grouped":
        return (g > 1 and cin_g in (1, 2, 4, 8, 16) and cout_g <= 16
                and ws[0] * int(np.prod(ws[1:])) <= 16384)
    if path == "strip":
        ow = (xs[-2] + pads[-1][0] + pads[-1][1] - dil[-1] * (ws[-2] - 1) - 1) // st[-1] + 1
        return (half and g == 1 and dil[-1] == 1 and xs[-1] % 32 == 0 and ws[0] % 4 == 0
                and st[-1] == 1 and ow % 32 == 0 and ws[-2] <= 5)
    if path == "phase":
        return (half and (g == 1 or cout_g % 64 == 0) and dil[-1] == 1 and dil[-2] == 1
                and cin_g % 64 == 0 and ws[0] % 4 == 0 and st[-1] == 2 and st[-2] == 2
                and ws[-2] in (2, 3) and ws[-3] in (2, 3))
    if path == "staged":
        kd = ws[1] if len(ws) == 5 else 1
        return (half and g == 1 and dil[-1] == 1 and dil[-2] == 1 and st[-1] == 1 and st[-2] == 1
                and ws[-2] in (2, 3) and ws[-3] in (2, 3) and xs[-1] >= 8
                and (xs[-1] % 8) * int(np.prod(ws[1:-1])) <= 32 and (xs[-1] % 8 == 0 or kd <= 3))
    if path == "slab":
        return (half and (g == 1 or cout_g % 64 == 0) and dil[-1] == dil[-2]
                and (dil[-1] == 1 or (dil[-1] == 2 and ws[-2] == 3 and ws[-3] == 3))
                and cin_g % 32 == 0 and ws[0] % 4 == 0 and st[-1] == 1 and st[-2] == 1
                and ws[-2] <= 3 and ws[-3] in (2, 3))
    return True


def _v_inputs(v):
    name, dtype, xs, ws, st, pads, dil, g = v
    gen = torch.Generator("cpu").manual_seed(zlib.crc32(name.encode()))
    x = (torch.rand(xs, generator=gen) * 2 - 1).to(_dt(dtype))
    fan_in = int(np.prod(ws[1:]))
    w = (torch.randn(ws, generator=gen) / np.sqrt(fan_in)).to(_dt(dtype))
    return x.to(DEV), w.to(DEV)


@pytest.mark.parametrize("path", VARIANT_PATHS)
@pytest.mark.parametrize("v", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_parity_variants(v, path):
    if not _v_accepts(v, path):
        pytest.skip(f"{path} does not take {v[0]}")
    name, dtype, xs, ws, st, pads, dil, g = v
    print(f"[parity] {name} path={path}", flush=True)
    x, w = _v_inputs(v)
    y = igc.conv_fwd(x, w, st, pads, path=path, dilation=dil, groups=g)
    torch.cuda.synchronize()
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pads, dilation=dil, groups=g)
    assert_parity(oracle.to_float64(y), ref, dtype, f"{name}/{path}")


@pytest.mark.parametrize("v", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_variant_tap_count_bit_exact(v):
    """x = 1, w = 1 on the first channel of each group: every output counts its in-bounds
    dilated taps; bit-exact on every path that takes the problem."""
    name, dtype, xs, ws, st, pads, dil, g = v
    x = torch.ones(xs, dtype=_dt(dtype), device=DEV)
    w = torch.zeros(ws, dtype=_dt(dtype), device=DEV)
    w[..., 0] = 1
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pads, dilation=dil, groups=g)
    for path in VARIANT_PATHS:
        if _v_accepts(v, path):
            y = igc.conv_fwd(x, w, st, pads, path=path, dilation=dil, groups=g)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(oracle.to_float64(y), ref, err_msg=f"{name}/{path}")


@pytest.mark.parametrize("v", [v for v in VARIANTS if v[2][-1] // v[7] == v[3][0] // v[7]],
                         ids=[v[0] for v in VARIANTS if v[2][-1] // v[7] == v[3][0] // v[7]])
def test_variant_one_hot_gather_bit_exact(v):
    """Per group, w = identity on the group's channels at one tap: y is the shifted, strided,
    dilated copy of x with channels kept in their group; bit-exact."""
    name, dtype, xs, ws, st, pads, dil, g = v
    cg = xs[-1] // g
    gen = torch.Generator("cpu").manual_seed(5)
    x = (torch.rand(xs, generator=gen) * 2 - 1).to(_dt(dtype)).to(DEV)
    ks = ws[1:-1]
    tap = tuple(k - 1 for k in ks)
    w = torch.zeros(ws, dtype=_dt(dtype))
    co = torch.arange(ws[0])
    w[(co, *[torch.full((ws[0],), t) for t in tap], co % cg)] = 1
    w = w.to(DEV)
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, pads, dilation=dil, groups=g)
    for path in VARIANT_PATHS:
        if _v_accepts(v, path):
            y = igc.conv_fwd(x, w, st, pads, path=path, dilation=dil, groups=g)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(oracle.to_float64(y), ref, err_msg=f"{name}/{path}")



@pytest.mark.parametrize("name", sorted(VARIANT_WORKLOADS))
def test_parity_variant_workloads_full_size(name):
    """The variant workloads at full size on the auto path (as bench.py --sweep runs them),
    every output element compared with the oracle."""
    wl = VARIANT_WORKLOADS[name]
    kw = dict(dilation=wl.dilation or 1, groups=wl.groups)
    print(f"[full] {name} path={igc.select_path(wl.x_shape, wl.w_shape, wl.stride, wl.padding, wl.torch_dtype, **kw)}",
          flush=True)
    x, w = make_inputs(wl, DEV)
    y = igc.conv_fwd(x, w, wl.stride, wl.padding, **kw)
    torch.cuda.synchronize()
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), wl.stride, wl.padding, **kw)
    e = assert_parity(oracle.to_float64(y), ref, wl.dtype, name)
    print(f"[full] {name} outputs={ref.size} l2_rel={e['l2_rel']:.2e} max_rel={e['max_rel']:.2e}", flush=True)
