"""Tolerance used to compare a GPU result with the oracle -- TEST INFRASTRUCTURE ONLY.

The stated bar is a relative tolerance of 1e-2 against the output dtype's
rounding R of the fp64 reference.  A purely relative test cannot hold where the
sum nearly cancels: any fp32 summation order then changes the result by an
amount tied to S = sum_k |a_k b_k|, not to |R|.  So an entry passes when

    |D - R| <= 1e-2 |R| + F,    F = 2^-16 |alpha| L S + tiny_out,

L = 1.1 when SiLU is applied (|SiLU'| <= 1.0998), else 1, and tiny_out is the
smallest subnormal of the output type.  2^-16 S exceeds the worst-case error of
128 successive fp32 additions (K = 8192 folded 64 products per step) by 2x, so
F can only admit reordering error, never a wrong term.
Infinite R must be matched exactly; NaN must be matched by NaN.
"""
from __future__ import annotations

import numpy as np

from .oracle import bits_to_f64

REL_TOL = 1e-2
FLOOR_FACTOR = 2.0 ** -16
TINY = {"bf16": 2.0 ** -133, "f16": 2.0 ** -24}


def compare(d_bits: np.ndarray, ref: dict, alpha, silu: bool, out: str, rel: float = REL_TOL) -> dict:
    """Compare GPU output bits with oracle bits.  Returns a report dict with 'ok'."""
    D = bits_to_f64(d_bits, out)
    R = bits_to_f64(ref["bits"], out)
    S = ref["S"]
    L = 1.1 if silu else 1.0
    F = FLOOR_FACTOR * abs(float(np.float32(alpha))) * L * S + TINY[out]
    err = np.abs(D - R)
    finite_r = np.isfinite(R)
    with np.errstate(invalid="ignore"):
        ok_finite = finite_r & np.isfinite(D) & (err <= rel * np.abs(R) + F)
    ok_inf = np.isinf(R) & (D == R)
    ok_nan = np.isnan(R) & np.isnan(D)
    ok = ok_finite | ok_inf | ok_nan
    big = finite_r & (np.abs(R) >= 100.0 * F)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel_err = np.where(big, err / np.abs(R), 0.0)
        by_floor = ok_finite & (err > rel * np.abs(R))
    n_bad = int((~ok).sum())
    first_bad = None
    if n_bad:
        idx = np.argwhere(~ok)[0]
        first_bad = dict(index=tuple(int(i) for i in idx), D=float(D[tuple(idx)]), R=float(R[tuple(idx)]),
                         F=float(F[tuple(idx)]))
    return dict(ok=n_bad == 0, n_bad=n_bad, n=int(D.size),
                max_rel_err=float(rel_err.max()) if rel_err.size else 0.0,
                n_passed_by_floor=int(by_floor.sum()), first_bad=first_bad)
