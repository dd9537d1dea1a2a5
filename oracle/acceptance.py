"""Acceptance rules for comparing a GPU result with the oracle (test infrastructure).

Tolerances, with S = |alpha s_A s_B| * sum_k |a_ik b_kj| from the oracle and
ulp_D(x) = 2^(max(floor(log2|x|), e_min) - p + 1) of the output format:

* integer-valued inputs: bit-exact against the once-rounded oracle value
  (+0 and -0 compare equal);
* fp32 output:            |D - ref| <= 1e-5 * S + 1e-6 + 2 ulp_f32(ref);
* fp16 / bf16 output:     |D - ref| <= 2 ulp_D(ref) + 2e-3 * S;
* fp8 inputs:             |D - ref| <= 2 ulp_D(ref) + 1.5e-2 * S.

The relative terms match fp32 accumulation of K products (each term carries
at most one fp32 rounding per addition, and fp16/bf16/fp8 inputs are exact in
the MFMA); the ulp terms cover the single rounding of the output. The extra
2 ulp_f32 term on the fp32 row covers the output rounding of a large beta*C,
which the relative term alone omits.
"""
from __future__ import annotations

import numpy as np

FORMAT = {  # precision p (with the hidden bit) and minimum normal exponent
    "f32": (24, -126),
    "f16": (11, -14),
    "bf16": (8, -126),
}


def ulp(dtype: str, x) -> np.ndarray:
    p, emin = FORMAT[dtype]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(ax > 0, np.maximum(e, emin), emin)
    return np.exp2(e - p + 1)


def tolerance(dtype_ab: str, dtype_d: str, ref, S) -> np.ndarray:
    ref = np.asarray(ref, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    if dtype_d == "f32":
        return 1e-5 * S + 1e-6 + 2.0 * ulp("f32", ref)
    # the fp8-input row of the tolerances also covers FP4 (MXFP4) inputs
    rel = 1.5e-2 if dtype_ab in ("f8e4m3", "f4e2m1") else 2e-3
    return 2.0 * ulp(dtype_d, ref) + rel * S


def check_close(got, ref, S, dtype_ab: str, dtype_d: str, what: str = ""):
    """Raise AssertionError naming the worst element if any is out of tolerance."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = tolerance(dtype_ab, dtype_d, ref, S)
    err = np.abs(got - ref)
    bad = ~(err <= tol)          # NaN counts as a failure
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(tol, 1e-300), 0)), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at "
            f"{tuple(int(i) for i in idx)}: got {got[idx]!r} ref {ref[idx]!r} "
            f"err {err[idx]:.3e} tol {tol[idx]:.3e}")
    return float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0


def check_exact(got_values, exact_values, what: str = ""):
    """Bit-exact by value (so +0 == -0); NaN never matches."""
    g = np.asarray(got_values, dtype=np.float64)
    e = np.asarray(exact_values, dtype=np.float64)
    bad = ~(g == e)
    if bad.any():
        idx = np.unravel_index(np.argmax(bad), g.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} differ; first at "
            f"{tuple(int(i) for i in idx)}: got {g[idx]!r} expected {e[idx]!r}")
