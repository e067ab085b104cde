"""Rounding to storage dtypes and the tolerance comparators (test infrastructure).

The pages fix no precision.  The workloads store tensors as fp32, bf16 or u8;
the oracle computes in fp64 and rounds a value only where the graph gives it a
storage dtype (an op's output dtype).  bf16 here is the 16-bit format with an
8-bit exponent and 8 significant bits (7 stored), round to nearest, ties to
even, with gradual underflow and overflow to infinity.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
BF16_MIN_NORMAL_EXP = -126
BF16_FRAC_BITS = 7


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each fp64 input (ties to even), as float64.

    Rounds once, directly from the fp64 value (not via fp32), so a value just
    above a bf16 tie rounds up even when fp32 would have collapsed it onto
    the tie.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(ax)
    axf = np.where(finite, ax, 0.0)
    _, e = np.frexp(axf)                      # axf = m * 2**e, m in [0.5, 1)
    unbiased = e - 1                          # axf = 1.f * 2**unbiased
    ulp_exp = np.maximum(unbiased, BF16_MIN_NORMAL_EXP) - BF16_FRAC_BITS
    q = np.ldexp(axf, -ulp_exp)               # exact: power-of-two scaling
    r = np.rint(q)                            # round half to even
    y = np.ldexp(r, ulp_exp)
    y = np.where(y > BF16_MAX, np.inf, y)
    y = np.where(finite, y, ax)               # inf stays inf, nan stays nan
    return np.copysign(y, x)


def round_f32(x) -> np.ndarray:
    """Nearest fp32 value (IEEE round to nearest even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    if dtype == "u8":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# bf16 ulp arithmetic
# ---------------------------------------------------------------------------
def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (the ulp of the binade holding |x|)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(ax > 0, ax, 1.0))
    unbiased = np.where(ax > 0, e - 1, BF16_MIN_NORMAL_EXP)
    return np.ldexp(1.0, np.maximum(unbiased, BF16_MIN_NORMAL_EXP) - BF16_FRAC_BITS)


def bf16_ulp_distance(got, ref_exact, floor_frac=2.0 ** -8) -> np.ndarray:
    """|got - round_bf16(ref)| in bf16 ulps measured at a floored magnitude.

    The ulp is taken at max(|ref|, floor_frac * max_row|ref|): near-zero
    outputs of a normalisation come from cancellation, where a correct fp32
    pipeline may sit a few ulps of a tiny reference away; the floor measures
    those in the row's own scale.  ``ref_exact`` is the fp64 reference before
    rounding; ``got`` holds bf16 values.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref_exact, dtype=np.float64)
    ref_r = round_bf16(ref)
    if ref.ndim >= 1 and ref.size:
        row_max = np.max(np.abs(ref), axis=-1, keepdims=True)
    else:
        row_max = np.abs(ref)
    scale = np.maximum(np.abs(ref), floor_frac * row_max)
    return np.abs(got - ref_r) / bf16_ulp(scale)


# ---------------------------------------------------------------------------
# Comparators (return (ok, metric)) for the stated tolerances
# ---------------------------------------------------------------------------
F32_REL_TOL = 1e-5
BF16_ULP_TOL = 2.0
MATMUL_REL_TOL = 1e-2


def max_rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| over the whole tensor (fp32 criterion)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)


def check_f32(got, ref, tol=F32_REL_TOL):
    e = max_rel_err(got, ref)
    return e <= tol, e


def check_bf16(got, ref_exact, tol=BF16_ULP_TOL):
    if np.asarray(ref_exact).size == 0:
        return True, 0.0
    d = float(np.max(bf16_ulp_distance(got, ref_exact)))
    return d <= tol, d


def check_matmul(got, ref, tol=MATMUL_REL_TOL):
    e = max_rel_err(got, ref)
    return e <= tol, e


def frobenius_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den else float(np.linalg.norm(got))
