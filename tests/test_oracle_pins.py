"""Pins the CPU oracle to facts the pages and the mathematics fix (no GPU needed).

Each test names what it pins.  Together they are chosen so that a plausible
slip in the oracle (a flipped kernel, a wrong sign or offset in the padding,
a stride applied to the wrong term, a transposed weight index, a dropped
channel or tap, a ceil instead of a floor) fails at least one of them; the
mutation tests in test_oracle_mutants.py plant such slips and check that.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from tests.im2col_ref import conv_im2col

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_matrices(path):
    mats, cur, name = {}, None, None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0].isalpha():
            name = parts[0]
            cur = mats[name] = []
        else:
            cur.append([float(v) for v in parts])
    return {k: np.array(v) for k, v in mats.items()}


def _rows(path):
    out = []
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            out.append(line.split())
    return out


# --- the pages' worked example -------------------------------------------------

def test_worked_example_2x2_on_3x3():
    """"Convolutions" section 4: [[1,2,3],[4,5,6],[7,8,9]] with [[1,0],[0,-1]] -> [[-4,-4],[-4,-4]]."""
    g = _read_matrices(os.path.join(GOLDEN, "worked_example_2x2_on_3x3.txt"))
    x = g["input"].reshape(1, 3, 3, 1)
    k = g["kernel"].reshape(1, 2, 2, 1)
    y = oracle.conv_fwd(x, k)
    assert y.shape == (1, 2, 2, 1)
    np.testing.assert_array_equal(y[0, :, :, 0], g["output"])
    # The flipped (true convolution) orientation gives +4 everywhere: the example
    # decides the orientation, so the oracle must not match the flipped kernel.
    y_flip = oracle.conv_fwd(x, k[:, ::-1, ::-1, :].copy())
    assert np.all(y_flip[0, :, :, 0] == 4.0)


def test_flop_formula_counts():
    """"Convolutions" sections 4 and 5: the oracle performs exactly the multiply-adds the FLOP
    formula 2*H_out*W_out*C_in*C_out*K_h*K_w counts, for the printed 236 MFLOPs and 3.7 GFLOP."""
    for name, h, w, cin, cout, k, s, p, printed, unit, digits in _rows(
            os.path.join(GOLDEN, "flop_counts.txt")):
        h, w, cin, cout, k, s, p, digits = map(int, (h, w, cin, cout, k, s, p, digits))
        x = np.zeros((1, h, w, cin))
        wt = np.zeros((cout, k, k, cin))
        y, macs = oracle.conv_fwd(x, wt, stride=s, padding=p, return_macs=True)
        scale = {"MFLOP": 1e6, "GFLOP": 1e9}[unit]
        assert round(2 * macs / scale, digits) == float(printed), name
        ho, wo = y.shape[1], y.shape[2]
        assert 2 * macs == 2 * ho * wo * cin * cout * k * k, name


def test_output_extents():
    """Output extents printed or implied by the pages (floor reading)."""
    for i, k, s, p, expected, *_ in _rows(os.path.join(GOLDEN, "output_extents.txt")):
        assert oracle.out_extent(int(i), int(k), int(s), int(p)) == int(expected)
    # and the oracle's output array has those extents (stem layer and the stride-2 3D row)
    y = oracle.conv_fwd(np.zeros((1, 224, 224, 3)), np.zeros((1, 7, 7, 3)), 2, 3)
    assert y.shape == (1, 112, 112, 1)
    y = oracle.conv_fwd(np.zeros((1, 32, 32, 32, 1)), np.zeros((1, 3, 3, 3, 1)), 2, 1)
    assert y.shape == (1, 16, 16, 16, 1)


def test_memory_column_matches_floor_extent():
    """MLX PR fp16 table: the implicit path's peak memory equals |x|+|w|+|y| in MiB.
    For the stride-2 row (4,32^3,64) -> 128 it prints 20.4, which only the floor
    extent (16^3 outputs) reproduces; the ceil extent (17^3) would give 21.2."""
    def mib(n_elems):
        return n_elems * 2 / 2**20
    od = oracle.out_extent(32, 3, 2, 1)
    total = mib(4 * 32**3 * 64) + mib(128 * 27 * 64) + mib(4 * od**3 * 128)
    assert round(total, 1) == 20.4
    # the unit-stride rows of the same table: (4,32^3,128->128) printed 64.8
    od = oracle.out_extent(32, 3, 1, 1)
    assert round(mib(4 * 32**3 * 128) + mib(128 * 27 * 128) + mib(4 * od**3 * 128), 1) == 64.8


# --- closed forms ----------------------------------------------------------------

def _valid_taps_1d(size, k, s, p, o):
    """Number of filter offsets t in [0, k) with 0 <= o*s - p + t < size (interval count)."""
    lo = max(0, p - o * s)
    hi = min(k, size + p - o * s)
    return max(0, hi - lo)


TAP_SHAPES = [
    # (D, H, W), (KD, KH, KW), stride, pad
    ((5, 6, 7), (3, 3, 3), (1, 1, 1), (1, 1, 1)),
    ((4, 5, 9), (3, 2, 3), (2, 1, 3), (1, 0, 2)),
    ((3, 7, 6), (1, 3, 5), (1, 2, 2), (0, 1, 2)),
    ((6, 4, 5), (3, 3, 3), (3, 3, 2), (3, 2, 3)),     # pad larger than k-1: all-padding windows
    ((1, 11, 12), (1, 7, 7), (1, 2, 2), (0, 3, 3)),   # stem-like 2D
    ((4, 4, 4), (3, 1, 1), (1, 1, 1), (1, 0, 0)),
    ((4, 4, 4), (1, 3, 3), (1, 1, 1), (0, 1, 1)),
]


@pytest.mark.parametrize("spatial,ks,st,pd", TAP_SHAPES)
def test_tap_count_closed_form(spatial, ks, st, pd):
    """x = 1 everywhere and w = 1 only on input channel 0: each output counts the
    in-bounds taps of its window, a product of per-dimension interval lengths."""
    n, cin, cout = 2, 3, 2
    x = np.ones((n, *spatial, cin))
    w = np.zeros((cout, *ks, cin))
    w[..., 0] = 1.0
    y = oracle.conv_fwd(x, w, st, pd)
    outs = [oracle.out_extent(spatial[i], ks[i], st[i], pd[i]) for i in range(3)]
    assert y.shape == (n, *outs, cout)
    for od in range(outs[0]):
        for oh in range(outs[1]):
            for ow in range(outs[2]):
                expect = (_valid_taps_1d(spatial[0], ks[0], st[0], pd[0], od)
                          * _valid_taps_1d(spatial[1], ks[1], st[1], pd[1], oh)
                          * _valid_taps_1d(spatial[2], ks[2], st[2], pd[2], ow))
                assert np.all(y[:, od, oh, ow, :] == expect)


GATHER_CASES = [((5, 6, 7), (3, 3, 3), (s, s, s), (p, p, p)) for s in (1, 2, 3) for p in (0, 1, 2, 3)]


@pytest.mark.parametrize("spatial,ks,st,pd", GATHER_CASES)
def test_one_hot_gather(spatial, ks, st, pd):
    """w = delta at one tap (kd*, kh*, kw*) with c_out = c_in: the output is the input
    shifted by that tap and subsampled by the stride, zero where it falls in the padding.
    Checked for every tap against numpy pad + strided slicing."""
    if any(oracle.out_extent(spatial[i], ks[i], st[i], pd[i]) < 1 for i in range(3)):
        pytest.skip("empty output")
    rng = np.random.default_rng(7)
    n, c = 2, 3
    x = rng.integers(-50, 50, size=(n, *spatial, c)).astype(np.float64)
    outs = [oracle.out_extent(spatial[i], ks[i], st[i], pd[i]) for i in range(3)]
    big = 16
    xp = np.pad(x, ((0, 0), (pd[0], big), (pd[1], big), (pd[2], big), (0, 0)))
    for a in range(ks[0]):
        for b in range(ks[1]):
            for e in range(ks[2]):
                w = np.zeros((c, *ks, c))
                for ch in range(c):
                    w[ch, a, b, e, ch] = 1.0
                y = oracle.conv_fwd(x, w, st, pd)
                expect = xp[:, a:a + outs[0] * st[0]:st[0], b:b + outs[1] * st[1]:st[1],
                            e:e + outs[2] * st[2]:st[2], :]
                np.testing.assert_array_equal(y, expect)


def test_pointwise_is_matmul():
    """"Convolutions" section 5, variants: a 1x1 stride-1 unpadded convolution is a GEMM
    over channels: y[M, C_out] = X[M, C_in] @ W^T."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, 5, 6, 7))
    w = rng.standard_normal((4, 1, 1, 1, 7))
    y = oracle.conv_fwd(x, w, 1, 0)
    ref = np.matmul(x.reshape(-1, 7), w.reshape(4, 7).T).reshape(2, 3, 5, 6, 4)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_linearity():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 4, 5, 6, 3))
    w1 = rng.standard_normal((5, 3, 2, 3, 3))
    w2 = rng.standard_normal((5, 3, 2, 3, 3))
    st, pd = (2, 1, 2), (1, 0, 2)
    y1 = oracle.conv_fwd(x, w1, st, pd)
    y2 = oracle.conv_fwd(x, w2, st, pd)
    np.testing.assert_allclose(oracle.conv_fwd(x, w1 + w2, st, pd), y1 + y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.conv_fwd(3.0 * x, w1, st, pd), 3.0 * y1, rtol=1e-12, atol=1e-12)


# --- independent brute force ---------------------------------------------------------

def _random_case(rng):
    dims = int(rng.integers(2, 4))
    n = int(rng.integers(1, 3))
    cin = int(rng.choice([1, 2, 3, 5, 8]))
    cout = int(rng.integers(1, 6))
    ks = [int(rng.integers(1, 4)) for _ in range(3)]
    st = [int(rng.integers(1, 4)) for _ in range(3)]
    pd = [int(rng.integers(0, 4)) for _ in range(3)]
    sp = [int(rng.integers(1, 8)) for _ in range(3)]
    if dims == 2:
        ks[0], st[0], pd[0], sp[0] = 1, 1, 0, 1
    for i in range(3):                     # keep at least one output along each dimension
        while sp[i] + 2 * pd[i] < ks[i]:
            sp[i] += 1
    return n, cin, cout, sp, ks, st, pd


def test_matches_im2col_on_random_tiny_shapes():
    """Exercise A of the tutorial: the direct loop nest equals im2col + GEMM, on 250
    random tiny 2D and 3D shapes (strides 1-3, pads 0-3, odd and unit channel counts)."""
    rng = np.random.default_rng(2024)
    for case in range(250):
        n, cin, cout, sp, ks, st, pd = _random_case(rng)
        x = rng.standard_normal((n, *sp, cin))
        w = rng.standard_normal((cout, *ks, cin))
        y = oracle.conv_fwd(x, w, st, pd)
        ref = conv_im2col(x, w, st, pd)
        assert y.shape == ref.shape, (case, sp, ks, st, pd)
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12, err_msg=str(case))


def test_rows_subset_equals_full():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 5, 6, 7, 4))
    w = rng.standard_normal((3, 3, 3, 3, 4))
    full = oracle.conv_fwd(x, w, (1, 2, 1), (1, 1, 0))
    flat = full.reshape(-1, 3)
    rows = np.array([0, 5, flat.shape[0] - 1, 17, 17])
    np.testing.assert_array_equal(oracle.conv_fwd(x, w, (1, 2, 1), (1, 1, 0), rows=rows), flat[rows])
    with pytest.raises(ValueError):
        oracle.conv_fwd(x, w, (1, 2, 1), (1, 1, 0), rows=np.array([flat.shape[0]]))


def test_empty_batch():
    y = oracle.conv_fwd(np.zeros((0, 4, 4, 4, 2)), np.zeros((3, 3, 3, 3, 2)), 1, 1)
    assert y.shape == (0, 4, 4, 4, 3)


# --- exact decoding of the input formats --------------------------------------------

def test_decode_formats_exactly():
    """fp16 / bf16 / fp32 to float64 is exact, subnormals included."""
    f16 = torch.tensor([0x3C00, 0x0001, 0x7BFF, 0x8400, 0x3555], dtype=torch.int32).to(torch.int16)
    f16 = f16.view(torch.float16)
    np.testing.assert_array_equal(oracle.to_float64(f16),
                                  [1.0, 2.0**-24, 65504.0, -2.0**-14, 0.333251953125])
    bf = torch.tensor([0x3F80, 0x0001, 0x7F7F, 0xC000], dtype=torch.int32).to(torch.int16)
    bf = bf.view(torch.bfloat16)
    np.testing.assert_array_equal(oracle.to_float64(bf),
                                  [1.0, 2.0**-133, (2 - 2.0**-7) * 2.0**127, -2.0])
    f32 = torch.tensor([1.0 + 2.0**-23, 2.0**-149], dtype=torch.float32)
    np.testing.assert_array_equal(oracle.to_float64(f32), [1.0 + 2.0**-23, 2.0**-149])


def test_fp16_decode_every_pattern():
    """All 65536 binary16 patterns against the format's definition written per class:
    zeros, subnormals m * 2^-24, normals (1024 + m) * 2^(e - 25), infinities, NaNs; and
    the sign symmetry."""
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode_fp16_bits(bits)
    e, m = (bits.astype(np.int64) >> 10) & 31, bits.astype(np.int64) & 1023
    pos = bits < 0x8000
    assert got[0x0000] == 0.0 and got[0x0001] == 2.0**-24 and got[0x03FF] == 1023 * 2.0**-24
    assert got[0x0400] == 2.0**-14 and got[0x3C00] == 1.0 and got[0x3C01] == 1.0 + 2.0**-10
    assert got[0x7BFF] == 65504.0 and got[0x7C00] == np.inf and np.isnan(got[0x7C01])
    assert np.all(np.isnan(got[(e == 31) & (m != 0)]))
    finite = e < 31
    assert np.all(got[finite & pos] * -1 == got[(bits | 0x8000)[finite & pos]])
    # strictly increasing over the positive finite patterns, and each step is the spacing
    # of the lower pattern's binade (2^-24 below 2^-14, 2^(e-25) above)
    vals = got[:0x7C00]
    steps = np.diff(vals)
    expect = np.ldexp(1.0, (np.maximum(e[:0x7C00 - 1], 1) - 25).astype(np.int32))
    np.testing.assert_array_equal(steps, expect)
    # agreement with numpy's own binary16 on every finite pattern
    np.testing.assert_array_equal(got[finite], bits[finite].view(np.float16).astype(np.float64))


def test_bf16_decode_against_fp32_fields():
    """bfloat16 patterns decode to the binary32 with the same upper 16 bits: exponent, sign
    and 7 fraction bits, spot-checked per class (subnormal, normal, infinity, NaN)."""
    bits = np.array([0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x7F7F, 0x7F80, 0xFF80, 0x7FC0,
                     0xBF80], dtype=np.uint16)
    got = oracle.decode_bf16_bits(bits)
    assert got[0] == 0.0 and got[1] == 2.0**-133 and got[2] == 127 * 2.0**-133
    assert got[3] == 2.0**-126 and got[4] == 1.0 and got[5] == 1.0 + 2.0**-7
    assert got[6] == (2 - 2.0**-7) * 2.0**127 and got[7] == np.inf and got[8] == -np.inf
    assert np.isnan(got[9]) and got[10] == -1.0


# --- the variants: grouped, dilated, asymmetric padding ("Convolution variants worth
#     knowing" on the tutorial page; pads per side as in the MLX benchmark tables) -----------

def _stuffed(w, dil):
    """The filter of taps `dil` apart as a dense filter with zeros in the gaps."""
    cout, kd, kh, kw, c = w.shape
    dd, dh, dw = dil
    ws = np.zeros((cout, dd * (kd - 1) + 1, dh * (kh - 1) + 1, dw * (kw - 1) + 1, c))
    ws[:, ::dd, ::dh, ::dw, :] = w
    return ws


DIL_CASES = [
    ((5, 7, 9), (3, 3, 3), (1, 1, 1), (2, 2, 2), (2, 2, 2)),
    ((4, 9, 8), (2, 3, 2), (1, 2, 1), (1, 3, 2), (3, 1, 2)),
    ((1, 11, 10), (1, 3, 3), (1, 1, 2), (0, 2, 1), (1, 2, 3)),
    ((6, 6, 6), (3, 2, 3), (2, 1, 1), (1, 0, 0), (2, 3, 1)),
]


@pytest.mark.parametrize("spatial,ks,st,pd,dil", DIL_CASES)
def test_dilated_filter_equals_zero_stuffed_filter(spatial, ks, st, pd, dil):
    """Taps e apart (a dilated filter) give exactly the convolution with the dense filter of
    span e*(K-1)+1 that holds the taps at multiples of e and zeros between them."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((2, *spatial, 3))
    w = rng.standard_normal((4, *ks, 3))
    y = oracle.conv_fwd(x, w, st, pd, dilation=dil)
    ref = oracle.conv_fwd(x, _stuffed(w, dil), st, pd)
    assert y.shape == ref.shape
    np.testing.assert_array_equal(y, ref)


def _valid_taps_dilated(size, k, s, p, e, o):
    """Brute force: taps t < k with 0 <= o*s - p + t*e < size."""
    return sum(1 for t in range(k) if 0 <= o * s - p + t * e < size)


@pytest.mark.parametrize("spatial,ks,st,pd,dil", DIL_CASES)
def test_dilated_tap_count_brute_force(spatial, ks, st, pd, dil):
    """x = 1, w = 1 on channel 0: every output counts its in-bounds dilated taps; output
    extents are floor((in + 2p - e*(K-1) - 1)/s) + 1."""
    x = np.ones((1, *spatial, 2))
    w = np.zeros((2, *ks, 2))
    w[..., 0] = 1.0
    y = oracle.conv_fwd(x, w, st, pd, dilation=dil)
    outs = [(spatial[i] + 2 * pd[i] - dil[i] * (ks[i] - 1) - 1) // st[i] + 1 for i in range(3)]
    assert y.shape == (1, *outs, 2)
    for od in range(outs[0]):
        for oh in range(outs[1]):
            for ow in range(outs[2]):
                expect = (_valid_taps_dilated(spatial[0], ks[0], st[0], pd[0], dil[0], od)
                          * _valid_taps_dilated(spatial[1], ks[1], st[1], pd[1], dil[1], oh)
                          * _valid_taps_dilated(spatial[2], ks[2], st[2], pd[2], dil[2], ow))
                assert np.all(y[0, od, oh, ow, :] == expect), (od, oh, ow)


@pytest.mark.parametrize("groups,cin,cout", [(2, 6, 4), (3, 9, 6), (4, 8, 8), (5, 5, 10)])
def test_groups_are_independent_convolutions_on_channel_slices(groups, cin, cout):
    """G groups: output channels [g*C_out/G, (g+1)*C_out/G) are the plain convolution of input
    channels [g*C_in/G, (g+1)*C_in/G) with their filters; the filter holds C_in/G channels."""
    rng = np.random.default_rng(groups)
    x = rng.standard_normal((2, 4, 5, 6, cin))
    w = rng.standard_normal((cout, 3, 2, 3, cin // groups))
    st, pd = (1, 2, 1), (1, 0, 2)
    y = oracle.conv_fwd(x, w, st, pd, groups=groups)
    cg, og = cin // groups, cout // groups
    parts = [oracle.conv_fwd(x[..., g * cg:(g + 1) * cg], w[g * og:(g + 1) * og], st, pd)
             for g in range(groups)]
    np.testing.assert_array_equal(y, np.concatenate(parts, axis=-1))


def test_depthwise_equals_per_channel_sums():
    """Depthwise (G = C_in = C_out): y[..., c] = sum over taps of the shifted, strided input
    channel c times w[c, tap, 0], built with numpy slicing."""
    rng = np.random.default_rng(8)
    c = 5
    x = rng.standard_normal((2, 4, 6, 7, c))
    w = rng.standard_normal((c, 3, 3, 2, 1))
    st, pd = (1, 2, 1), (1, 1, 0)
    y = oracle.conv_fwd(x, w, st, pd, groups=c)
    outs = [oracle.out_extent(x.shape[1 + i], w.shape[1 + i], st[i], pd[i]) for i in range(3)]
    xp = np.pad(x, ((0, 0), (pd[0], 8), (pd[1], 8), (pd[2], 8), (0, 0)))
    ref = np.zeros((2, *outs, c))
    for a in range(3):
        for b in range(3):
            for e in range(2):
                sl = xp[:, a:a + outs[0] * st[0]:st[0], b:b + outs[1] * st[1]:st[1],
                        e:e + outs[2] * st[2]:st[2], :]
                ref += sl * w[:, a, b, e, 0]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("pads", [((0, 2), (1, 0), (2, 1)), ((3, 0), (0, 3), (1, 2)), ((1, 1), (2, 0), (0, 0))])
def test_asymmetric_padding_equals_explicitly_padded_input(pads):
    """Low / high pads (p, q) give the unpadded convolution of the input with p zeros in
    front and q behind along each dimension."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((2, 4, 5, 6, 3))
    w = rng.standard_normal((4, 3, 3, 2, 3))
    st = (1, 2, 2)
    y = oracle.conv_fwd(x, w, st, pads)
    xp = np.pad(x, ((0, 0), *pads, (0, 0)))
    ref = oracle.conv_fwd(xp, w, st, 0)
    assert y.shape == ref.shape
    np.testing.assert_array_equal(y, ref)


def test_all_variants_together_match_im2col_of_stuffed_padded_input():
    """Groups, dilation and asymmetric pads at once against the independent im2col + GEMM
    of each group's channel slice, with the filter zero-stuffed and the input padded
    explicitly (so that path never sees a variant)."""
    rng = np.random.default_rng(99)
    for case in range(20):
        g = int(rng.choice([1, 2, 3]))
        cg, og = int(rng.integers(1, 4)), int(rng.integers(1, 3))
        ks = [int(rng.integers(1, 4)) for _ in range(3)]
        dl = [int(rng.integers(1, 3)) for _ in range(3)]
        st = [int(rng.integers(1, 3)) for _ in range(3)]
        pads = [(int(rng.integers(0, 3)), int(rng.integers(0, 3))) for _ in range(3)]
        sp = [int(rng.integers(1, 6)) for _ in range(3)]
        for i in range(3):
            while sp[i] + sum(pads[i]) < dl[i] * (ks[i] - 1) + 1:
                sp[i] += 1
        x = rng.standard_normal((2, *sp, g * cg))
        w = rng.standard_normal((g * og, *ks, cg))
        y = oracle.conv_fwd(x, w, st, pads, dilation=dl, groups=g)
        xp = np.pad(x, ((0, 0), *pads, (0, 0)))
        ws = _stuffed(w, dl)
        ref = np.concatenate([conv_im2col(xp[..., i * cg:(i + 1) * cg], ws[i * og:(i + 1) * og], st, (0, 0, 0))
                              for i in range(g)], axis=-1)
        assert y.shape == ref.shape, case
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12, err_msg=str(case))


# --- backward-data (transposed convolution) --------------------------------------
# Random problems over the whole descriptor: 2D and 3D, strides 1-3, low and high pads,
# dilation, groups.  (x shape, filter extents, stride, (low, high) pads, dilation, groups, C_out)
BWD_CASES = [
    ((2, 5, 6, 4), (3, 3), (1, 1), ((1, 1), (1, 1)), (1, 1), 1, 3),
    ((1, 7, 8, 4), (3, 2), (2, 3), ((1, 0), (0, 2)), (1, 1), 2, 6),
    ((2, 5, 6, 7, 4), (3, 3, 3), (2, 2, 2), ((1, 1), (1, 1), (1, 1)), (1, 1, 1), 1, 5),
    ((1, 6, 5, 9, 6), (2, 3, 3), (1, 2, 3), ((0, 1), (2, 0), (1, 2)), (2, 1, 2), 3, 6),
    ((2, 9, 8, 3), (3, 3), (2, 2), ((2, 2), (2, 2)), (2, 3), 1, 2),
    ((1, 4, 5, 6, 8), (3, 1, 2), (3, 1, 2), ((3, 3), (0, 0), (2, 1)), (1, 1, 2), 4, 4),
]


def _bwd_inputs(case, seed):
    xs, ks, st, pads, dil, g, cout = case
    rng = np.random.default_rng(seed)
    x = rng.normal(size=xs)
    w = rng.normal(size=(cout, *ks, xs[-1] // g))
    return x, w


@pytest.mark.parametrize("case", BWD_CASES)
def test_bwd_data_is_the_adjoint_of_the_forward_pass(case):
    """<conv(x, w), dy> = <x, dgrad(dy, w)> for all x, dy: the defining property of the
    gradient with respect to x (equal up to float64 rounding of two independent sums)."""
    xs, ks, st, pads, dil, g, cout = case
    x, w = _bwd_inputs(case, 3)
    y = oracle.conv_fwd(x, w, st, pads, dilation=dil, groups=g)
    dy = np.random.default_rng(4).normal(size=y.shape)
    dx = oracle.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g)
    assert dx.shape == tuple(xs)
    lhs, rhs = float((y * dy).sum()), float((x * dx).sum())
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + np.abs(y * dy).sum())


@pytest.mark.parametrize("case", BWD_CASES)
def test_bwd_data_is_a_forward_conv_of_zero_inserted_dy_with_the_flipped_filter(case):
    """The transposed convolution as the MLX general path builds it: dy dilated by the
    stride (zeros between neighbours), placed so that dx[i] = sum_k' B[i + k'e] wf[k'] with
    wf the spatially flipped filter with input and output channels exchanged per group."""
    xs, ks, st, pads, dil, g, cout = case
    x, w = _bwd_inputs(case, 5)
    y = oracle.conv_fwd(x, w, st, pads, dilation=dil, groups=g)
    dy = np.random.default_rng(6).normal(size=y.shape)
    dims = len(xs) - 2
    big = [xs[1 + i] + dil[i] * (ks[i] - 1) for i in range(dims)]
    B = np.zeros((xs[0], *big, cout))
    # B index t holds dy[(t - P) / s] where P = (K-1) e - p and the division is exact
    for idx in np.ndindex(*big):
        src = []
        for i in range(dims):
            u = idx[i] - (dil[i] * (ks[i] - 1) - pads[i][0])
            if u < 0 or u % st[i] != 0 or u // st[i] >= y.shape[1 + i]:
                break
            src.append(u // st[i])
        else:
            B[(slice(None), *idx)] = dy[(slice(None), *src)]
    cg, og = xs[-1] // g, cout // g
    wf = np.zeros((xs[-1], *ks, og))
    flipped = w[(slice(None),) + (slice(None, None, -1),) * dims]
    for gi in range(g):
        blk = flipped[gi * og:(gi + 1) * og]                       # (og, K..., cg)
        wf[gi * cg:(gi + 1) * cg] = np.moveaxis(blk, (0, -1), (-1, 0))
    ref = oracle.conv_fwd(B, wf, 1, 0, dilation=dil, groups=g)
    dx = oracle.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g)
    np.testing.assert_allclose(dx, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", BWD_CASES)
def test_bwd_data_tap_counts_brute_force(case):
    """dy = 1 and w = 1 only from output channel 0 to input channel 0 of group 0: dx at input
    channel 0 counts, per position, the (tap, output) pairs that read it -- counted here by
    running the forward index map over every output and tap."""
    xs, ks, st, pads, dil, g, cout = case
    y_shape = oracle.conv_fwd(np.zeros(xs), np.zeros((cout, *ks, xs[-1] // g)), st, pads,
                              dilation=dil, groups=g).shape
    dy = np.ones(y_shape)
    w = np.zeros((cout, *ks, xs[-1] // g))
    w[0, ..., 0] = 1
    dx = oracle.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g)
    dims = len(xs) - 2
    count = np.zeros(xs[1:-1])
    for o in np.ndindex(*y_shape[1:-1]):
        for k in np.ndindex(*ks):
            i = [o[j] * st[j] - pads[j][0] + k[j] * dil[j] for j in range(dims)]
            if all(0 <= i[j] < xs[1 + j] for j in range(dims)):
                count[tuple(i)] += 1
    for n in range(xs[0]):
        np.testing.assert_array_equal(dx[n, ..., 0], count)
    assert not dx[..., 1:].any()


def test_bwd_data_of_the_worked_example():
    """The tutorial's worked example (section 4): y = x * k = [[-4,-4],[-4,-4]].  With dy = 1
    the adjoint identity gives sum(x * dx) = sum(y) = -16, and dx is the kernel summed over the
    four output positions it was placed at."""
    m = _read_matrices(os.path.join(GOLDEN, "worked_example_2x2_on_3x3.txt"))
    x, k, y = m["input"], m["kernel"], m["output"]
    dx = oracle.conv_bwd_data(np.ones((1, 2, 2, 1)), k.reshape(1, 2, 2, 1), (1, 3, 3, 1))[0, ..., 0]
    assert float((x * dx).sum()) == float(y.sum()) == -16.0
    placed = np.zeros((3, 3))
    for a in range(2):
        for b in range(2):
            placed[a:a + 2, b:b + 2] += k
    np.testing.assert_array_equal(dx, placed)


def test_bwd_data_rows_subset_equals_full():
    xs, ks, st, pads, dil, g, cout = BWD_CASES[3]
    x, w = _bwd_inputs(BWD_CASES[3], 7)
    y = oracle.conv_fwd(x, w, st, pads, dilation=dil, groups=g)
    dy = np.random.default_rng(8).normal(size=y.shape)
    full = oracle.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g).reshape(-1, xs[-1])
    rows = np.array([0, 5, 17, full.shape[0] - 1])
    part = oracle.conv_bwd_data(dy, w, xs, st, pads, dilation=dil, groups=g, rows=rows)
    np.testing.assert_array_equal(part, full[rows])
