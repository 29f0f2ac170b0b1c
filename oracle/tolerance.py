"""Tolerance used to compare a GPU result with the oracle -- TEST INFRASTRUCTURE ONLY.

The stated bar is a relative tolerance of 1e-2 against the output dtype's rounding R of the fp64
reference.  Two rules, both required:

1. Strict rule, on the entries the bar can be asked of: |D - R| <= 1e-2 |R|.  An entry is held to
   it ("resolvable") when its sum does not cancel and its epilogue does not amplify relative
   error:
       |acc| >= 2^-6 S                (S = sum_k |a_k b_k|: the sum keeps >= 1/64 of its mass)
       kappa_bias * kappa_silu <= 1.5 (kappa_bias = |alpha acc| / |x|, x = alpha acc + bias;
                                       kappa_silu = |x SiLU'(x) / SiLU(x)|, 1 without SiLU)
       R finite and non-zero.
   On such an entry any fp32-accumulating implementation whose accumulation error stays below
   about 2^-13 S lands within a few output ulps of R; a systematic error of 1.5% cannot pass.

2. Floor rule, on every entry: |D - R| <= 1e-2 |R| + F with
       F = lambda * delta + tiny_out,    delta = c_fmt(K) |alpha| S + 2^-22 |x|,
   where delta bounds the error of x (accumulation, then the fp32 epilogue multiply-add) and lambda
   is the largest |epi'| on [x - delta, x + delta] (1 for the identity; the exact interval maximum
   of |SiLU'| otherwise, so SiLU's flat negative tail gets a correspondingly small floor).
   tiny_out is the smallest subnormal of the output type.  Infinite R must be matched exactly;
   NaN must be matched by NaN.

The accumulation bound c_fmt(K) follows each format's route on the hardware:
* MXFP8 -- the scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) does not add its 64 products
  exactly: measured with one-hot and full-range random codes it aligns products to a shared
  exponent and keeps about 14 bits below it.  Under that model a group of 8 products loses at
  most 8 * 2^-13 of its largest product, i.e. at most 2^-10 S over any number of groups; fp32
  accumulation between instructions adds at most (K/64) 2^-24 S.  c = 2^-10 + (K/64 + 18) 2^-24.
  (Measured: 1.5e-4 S on full-range random codes, <= 1.8e-5 S on quantised Gaussian operands.)
* NVFP4 -- exact fp16 operands q * s * 2^-8 on v_mfma_f32_32x32x16_f16: every product is exact in
  fp32, and the instruction adds its 16 products to the accumulator with one fp32 rounding
  (measured: <= 6e-8 S on full-range random codes).  One rounding per instruction (K/16 of them),
  one per split-K partial (at most 16) and margin: c = (K/16 + 18) 2^-24.
"""
from __future__ import annotations

import math

import numpy as np

from .oracle import bits_to_f64

REL_TOL = 1e-2
RESOLVE_SUM = 2.0 ** -6      # |acc| >= RESOLVE_SUM * S: the sum does not cancel
RESOLVE_KAPPA = 1.5          # epilogue condition number limit for the strict rule
TINY = {"bf16": 2.0 ** -133, "f16": 2.0 ** -24}
U32 = 2.0 ** -24             # fp32 unit roundoff
MX_ALIGN = 2.0 ** -10        # scaled FP8 MFMA alignment loss bound, per unit of S


def accumulation_bound(fmt: str, K: int) -> float:
    """c_fmt(K): a bound on |acc_gpu - acc| / S for the format's MFMA route (module docstring)."""
    if fmt == "mxfp8":
        return MX_ALIGN + (K / 64.0 + 18.0) * U32
    if fmt == "nvfp4":
        return (K / 16.0 + 18.0) * U32
    raise ValueError(fmt)


def _sigmoid(t):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-t))


def silu_slope(t):
    """SiLU'(t) = sigma(t) (1 + t (1 - sigma(t))), fp64."""
    t = np.asarray(t, dtype=np.float64)
    s = _sigmoid(t)
    return s * (1.0 + t * (1.0 - s))


def _silu_slope_extremum() -> float:
    """The positive root of SiLU''(t) = 0, i.e. of t tanh(t/2) = 2 (|SiLU'| peaks at +-t*): bisection."""
    lo, hi = 1.0, 4.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid * math.tanh(mid / 2.0) < 2.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


SILU_T_STAR = _silu_slope_extremum()


def silu_slope_max(lo, hi):
    """max |SiLU'(t)| over t in [lo, hi] (elementwise): the endpoints, and the two extrema at +-t*
    when they lie inside (SiLU' is monotone between its critical points)."""
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    m = np.maximum(np.abs(silu_slope(lo)), np.abs(silu_slope(hi)))
    for c in (SILU_T_STAR, -SILU_T_STAR):
        inside = (lo <= c) & (c <= hi)
        m = np.where(inside, np.maximum(m, abs(float(silu_slope(c)))), m)
    return m


def silu_kappa(x):
    """Relative condition number of SiLU at x: |x SiLU'(x) / SiLU(x)| = |1 + x (1 - sigma(x))|."""
    x = np.asarray(x, dtype=np.float64)
    return np.abs(1.0 + x * (1.0 - _sigmoid(x)))


def compare(d_bits: np.ndarray, ref: dict, alpha, silu: bool, out: str, rel: float = REL_TOL) -> dict:
    """Compare GPU output bits with the oracle's.  `ref` is oracle.reference()'s result (it carries the
    format, K, acc, S and x).  Returns a report dict; 'ok' requires both rules of the module
    docstring."""
    D = bits_to_f64(d_bits, out)
    R = bits_to_f64(ref["bits"], out)
    S, acc, x = ref["S"], ref["acc"], ref["x"]
    a32 = float(np.float32(alpha))
    aS = abs(a32) * S
    with np.errstate(invalid="ignore", over="ignore"):
        delta = accumulation_bound(ref["fmt"], ref["K"]) * aS + 2.0 ** -22 * np.abs(x)
        lam = silu_slope_max(x - delta, x + delta) if silu else 1.0
        F = lam * delta + TINY[out]
        err = np.abs(D - R)
    finite_r = np.isfinite(R)
    with np.errstate(invalid="ignore"):
        ok_finite = finite_r & np.isfinite(D) & (err <= rel * np.abs(R) + F)
    ok_inf = np.isinf(R) & (D == R)
    ok_nan = np.isnan(R) & np.isnan(D)
    ok_floor = ok_finite | ok_inf | ok_nan
    # strict rule on resolvable entries
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        kappa = np.abs(a32 * acc) / np.abs(x)
        if silu:
            kappa = kappa * silu_kappa(x)
        resolvable = finite_r & (R != 0) & np.isfinite(x) & (np.abs(acc) >= RESOLVE_SUM * S) & \
            (kappa <= RESOLVE_KAPPA)
        rel_err = np.where(resolvable, err / np.abs(R), 0.0)
    ok_strict = ~resolvable | (np.isfinite(D) & (rel_err <= rel))
    ok = ok_floor & ok_strict
    with np.errstate(invalid="ignore", divide="ignore"):
        by_floor = ok_finite & (err > rel * np.abs(R))
        err_over_s = np.where(finite_r & (aS > 0), err / np.where(aS > 0, aS, 1.0), 0.0)
    n_bad = int((~ok).sum())
    first_bad = None
    if n_bad:
        idx = tuple(int(i) for i in np.argwhere(~ok)[0])
        first_bad = dict(index=idx, D=float(D[idx]), R=float(R[idx]), F=float(F[idx]) if np.ndim(F) else float(F),
                         resolvable=bool(resolvable[idx]))
    return dict(ok=n_bad == 0, n_bad=n_bad, n=int(D.size),
                n_resolvable=int(resolvable.sum()),
                max_rel_err=float(rel_err.max()) if rel_err.size else 0.0,
                max_err_over_S=float(err_over_s.max()) if err_over_s.size else 0.0,
                n_passed_by_floor=int(by_floor.sum()), first_bad=first_bad)
