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


def rounding_bound(ref, vmax, q_scaled_err=None):
    """Per-element error bound of bf16 attention with P and O rounded to bf16.

    The weights are the numerators P_j = 2^(S_j), each rounded to bf16 (relative
    error <= 2^-9), normalised by l summed from the same rounded values, so each
    normalised weight is off by at most 2^-8 relative and the output by at most
    2^-8 * max_j |V_j - O| <= 2^-8 * (vmax + |O|) per dimension (vmax: the
    largest |V| of that dimension over the row's keys); the final bf16 rounding
    of O adds 2^-9 |O|.  q_scaled_err: per row, a bound on the error of the
    scores in log2 units (max_j |dS_j|) when the scaled Q is itself rounded to
    bf16; it moves each weight by at most 2 ln 2 * max_j |dS_j| relative.
    ref [rows, D]; vmax [D] or [rows, D]; q_scaled_err [rows] or None."""
    ref = np.asarray(ref, np.float64)
    spread = np.asarray(vmax, np.float64) + np.abs(ref)
    b = 2.0 ** -8 * spread + 2.0 ** -9 * np.abs(ref)
    if q_scaled_err is not None:
        b = b + 2.0 * np.log(2.0) * np.asarray(q_scaled_err, np.float64)[:, None] * spread
    return b + 1e-6


def assert_within_bound(got, ref, bound, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: error exceeds the rounding bound by {worst:.3f}x (max-abs {err.max():.4g})"
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "worst_vs_bound": worst}
