"""GPU tests of the measured selection table (conv_tune): the recorded choice is used by AUTO,
keeps parity with the oracle, serves shapes of the same bucket, and can be forgotten."""
import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
import oracle
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _clean_table():
    igc.tune_clear()
    yield
    igc.tune_clear()


def _inputs(xs, ws, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    x = (torch.rand(xs, generator=g) * 2 - 1).to(dtype)
    w = (torch.randn(ws, generator=g) / np.sqrt(np.prod(ws[1:]))).to(dtype)
    return x.to(DEV), w.to(DEV)


@pytest.mark.parametrize("xs,ws,st,dtype", [
    ((2, 9, 10, 11, 64), (128, 3, 3, 3, 64), 1, torch.float16),
    ((2, 9, 10, 32, 64), (64, 3, 3, 3, 64), 1, torch.bfloat16),
    ((2, 11, 12, 13, 64), (128, 3, 3, 3, 64), 2, torch.float16),
    ((2, 5, 6, 7, 5), (7, 3, 3, 3, 5), 1, torch.float32),
])
def test_tune_choice_is_used_and_keeps_parity(xs, ws, st, dtype):
    x, w = _inputs(xs, ws, dtype, 3)
    path, us = igc.tune(x, w, st, 1, reps=3)
    print(f"[tune] {xs} -> {path} {us:.1f} us", flush=True)
    assert us > 0
    assert igc.tuned_path(xs, ws, st, 1, dtype) == path
    assert igc.select_path(xs, ws, st, 1, dtype) == path
    y = igc.conv_fwd(x, w, st, 1)
    torch.cuda.synchronize()
    ref = oracle.conv_fwd(oracle.to_float64(x), oracle.to_float64(w), st, 1)
    name = {torch.float16: "fp16", torch.bfloat16: "bf16", torch.float32: "fp32"}[dtype]
    assert_parity(oracle.to_float64(y), ref, name, f"tuned {path}")


def test_tune_bucket_serves_nearby_shapes_and_clear_forgets():
    x, w = _inputs((2, 9, 10, 11, 64), (128, 3, 3, 3, 64), torch.float16, 4)
    path, _ = igc.tune(x, w, 1, 1, reps=2)
    near = (2, 12, 13, 14, 64)                     # same bucket: (2, 16, 16, 16)
    assert igc.tuned_path(near, (128, 3, 3, 3, 64), 1, 1) == path
    assert igc.tuned_path((2, 17, 13, 14, 64), (128, 3, 3, 3, 64), 1, 1) is None   # next bucket
    xn, wn = _inputs(near, (128, 3, 3, 3, 64), torch.float16, 5)
    y = igc.conv_fwd(xn, wn, 1, 1)
    torch.cuda.synchronize()
    ref = oracle.conv_fwd(oracle.to_float64(xn), oracle.to_float64(wn), 1, 1)
    assert_parity(oracle.to_float64(y), ref, "fp16", "bucketed")
    igc.tune_clear()
    assert igc.tuned_path((2, 9, 10, 11, 64), (128, 3, 3, 3, 64), 1, 1) is None
