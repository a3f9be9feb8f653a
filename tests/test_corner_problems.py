"""The corner sub-problems the size-limit GPU tests compare against (CPU only): the oracle on
a corner's input region with explicit (low, high) pads must equal that corner of the oracle's
full result, for strides, asymmetric pads, dilation and both ends of every dimension."""
import numpy as np
import pytest

import oracle
from tests.test_gpu_limits import _corner


@pytest.mark.parametrize("xs,ws,st,pads,dil", [
    ((2, 11, 37, 4), (3, 3, 3, 4), (1, 1), ((1, 1), (1, 1)), (1, 1)),
    ((1, 20, 21, 3), (2, 7, 7, 3), (2, 2), ((3, 3), (3, 2)), (1, 1)),
    ((2, 9, 14, 4), (4, 3, 3, 4), (2, 2), ((1, 1), (1, 1)), (1, 1)),
    ((1, 13, 17, 2), (3, 3, 3, 2), (1, 1), ((2, 2), (2, 2)), (2, 2)),
    ((2, 7, 8, 9, 3), (2, 3, 3, 3, 3), (1, 2, 1), ((1, 1), (1, 0), (0, 2)), (1, 1, 2)),
])
def test_corner_problem_matches_full_result(xs, ws, st, pads, dil):
    rng = np.random.default_rng(sum(xs))
    x = rng.standard_normal(xs)
    w = rng.standard_normal(ws)
    full = oracle.conv_fwd(x, w, st, pads, dilation=dil)
    nsp = len(xs) - 2
    for which in ("first", "last"):
        img = 0 if which == "first" else xs[0] - 1
        ranges = []
        for dim in range(nsp):
            o = full.shape[1 + dim]
            r = min(3 + dim, o)
            ranges.append((0, r) if which == "first" else (o - r, o))
        sl, sub_pads = _corner(x, ws[1:-1], st, pads, dil, ranges)
        sub = oracle.conv_fwd(x[(slice(img, img + 1), *sl)], w, st, sub_pads, dilation=dil)
        want = full[(slice(img, img + 1), *[slice(a, b) for a, b in ranges])]
        assert sub.shape == want.shape
        np.testing.assert_allclose(sub, want, rtol=1e-12, atol=1e-12)
