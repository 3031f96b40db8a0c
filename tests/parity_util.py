"""Comparison helpers shared by the GPU parity tests, smoke() and bench.py.

The bar (fp outputs of unit-scale inputs): max-abs error <= 1e-2 and mean-abs
error <= 1e-3 against the fp64 oracle.  A relative L2 error bound of 1e-2 is
checked as well: bf16 operands and outputs put a correct kernel near 2e-3,
while a wrong key/value row (which can hide under the absolute bounds because
the outputs are small, ~0.01-0.1 rms) moves it to O(0.1-1).
"""
import numpy as np

MAX_ABS = 1e-2
MEAN_ABS = 1e-3
REL_L2 = 1e-2


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def error_stats(got, ref) -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = np.abs(got - ref)
    denom = np.sqrt(np.sum(ref * ref))
    return {
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "mean_abs": float(diff.mean()) if diff.size else 0.0,
        "rel_l2": float(np.sqrt(np.sum(diff * diff)) / denom) if denom > 0 else 0.0,
        "finite": bool(np.isfinite(got).all()),
        "n": int(diff.size),
    }


def assert_parity(got, ref, what=""):
    s = error_stats(got, ref)
    assert s["finite"], f"{what}: non-finite output {s}"
    assert s["max_abs"] <= MAX_ABS, f"{what}: max-abs {s}"
    assert s["mean_abs"] <= MEAN_ABS, f"{what}: mean-abs {s}"
    assert s["rel_l2"] <= REL_L2, f"{what}: rel-L2 {s}"
    return s
