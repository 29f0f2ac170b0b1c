"""CPU checks of the comparison rule (oracle/tolerance.py) against brute force and planted errors.

The workload slices below are the benchmark recipes at their own K, alpha, epilogue and output type
with fewer rows and columns (the first rows of A and B, and of the bias, of the seeded streams), so
that the ratio S / |acc| -- which decides how much the cancellation floor could hide -- is the
workloads' own.
"""
import numpy as np
import pytest
from scipy.special import expit

import seeded_inputs as si
from oracle import oracle as O
from oracle import tolerance as T

SLICES = {
    "mxfp8_256": lambda: si.workload("mxfp8_256"),
    "mxfp8_4096": lambda: si.mxfp8_problem(2, 64, 1024, 4096, alpha=0.5, out="bf16", outlier_rows=True),
    "mxfp8_8192_silu": lambda: si.mxfp8_problem(3, 48, 512, 8192, alpha=1.0, bias=True, silu=True, out="f16"),
    "nvfp4_128x8192x8192_silu": lambda: si.nvfp4_problem(4, 48, 512, 8192, bias=True, silu=True, out="bf16"),
    "nvfp4_256x4096x4096_loop": lambda: si.nvfp4_problem(5, 64, 1024, 4096, out="bf16"),
}


@pytest.fixture(scope="module", params=sorted(SLICES))
def workload_slice(request):
    p = SLICES[request.param]()
    return request.param, p, O.reference(p)


def _scaled(ref, p, factor):
    return O.round_output(ref["y"] * factor, p["out"])


def test_exact_result_passes(workload_slice):
    name, p, ref = workload_slice
    rep = T.compare(ref["bits"], ref, p["alpha"], p["silu"], p["out"])
    assert rep["ok"] and rep["max_rel_err"] == 0.0, (name, rep)
    # the strict rule covers a large share of the entries (the ones whose sum does not cancel)
    assert rep["n_resolvable"] >= 0.15 * rep["n"], (name, rep)


@pytest.mark.parametrize("factor", [1.015, 0.985])
def test_uniform_1p5_percent_error_fails(workload_slice, factor):
    name, p, ref = workload_slice
    rep = T.compare(_scaled(ref, p, factor), ref, p["alpha"], p["silu"], p["out"])
    assert not rep["ok"], (name, rep)
    # it fails on (nearly) every entry held to the strict rule, not on a stray one
    assert rep["n_bad"] >= 0.9 * rep["n_resolvable"], (name, rep)


def test_half_percent_error_passes(workload_slice):
    # within the stated 1e-2 bar even after the extra output rounding
    name, p, ref = workload_slice
    rep = T.compare(_scaled(ref, p, 1.005), ref, p["alpha"], p["silu"], p["out"])
    assert rep["ok"], (name, rep)


def test_measured_size_accumulation_noise_passes(workload_slice):
    # accumulation errors of the size measured on the device: MXFP8 <= 1.8e-5 S at K = 64 and less
    # at larger K (noise sigma 4e-6 S); NVFP4 at fp32 rounding, one rounding of up to 2^-24 of the
    # running sum per MFMA instruction (a random walk: sigma 2^-24 sqrt(K/16) S).  Then the epilogue
    # and one output rounding, as a kernel would.
    name, p, ref = workload_slice
    g = np.random.default_rng(5)
    sigma = 4e-6 if p["fmt"] == "mxfp8" else 2.0 ** -24 * np.sqrt(p["K"] / 16)
    acc = ref["acc"] + g.standard_normal(ref["acc"].shape) * sigma * ref["S"]
    y = O.epilogue(acc, p["alpha"], p["bias"], p["silu"])
    rep = T.compare(O.round_output(y, p["out"]), ref, p["alpha"], p["silu"], p["out"])
    assert rep["ok"], (name, rep)


def test_error_of_the_floor_size_passes_only_where_the_sum_cancels():
    # an error of the accumulation bound itself on a cancelling entry is what the floor admits
    p = si.problem("mxfp8", 32, 64, 1024, seed=3, out="f16")
    ref = O.reference(p)
    c = T.accumulation_bound("mxfp8", 1024)
    canc = np.abs(ref["acc"]) < 2.0 ** -8 * ref["S"]
    assert canc.any()
    y = ref["y"] + np.where(canc, 0.9 * c * float(p["alpha"]) * ref["S"], 0.0)
    assert T.compare(O.round_output(y, "f16"), ref, p["alpha"], False, "f16")["ok"]
    y = ref["y"] + np.where(canc, 1.5 * c * float(p["alpha"]) * ref["S"], 0.0)
    assert not T.compare(O.round_output(y, "f16"), ref, p["alpha"], False, "f16")["ok"]


def test_accumulation_bounds_per_format():
    # NVFP4's route (exact products, fp32 adds) is bounded far below the scaled FP8 MFMA's alignment loss
    assert T.accumulation_bound("nvfp4", 8192) == (8192 / 16 + 18) * 2.0 ** -24
    assert T.accumulation_bound("nvfp4", 8192) < 2.0 ** -14 < T.accumulation_bound("mxfp8", 64)
    assert T.accumulation_bound("mxfp8", 8192) < 2.0 ** -10 * 1.01


def test_silu_slope_matches_finite_differences():
    x = np.linspace(-40, 40, 4001)
    silu = lambda t: t * expit(t)  # noqa: E731
    h = 1e-6
    fd = (silu(x + h) - silu(x - h)) / (2 * h)
    assert np.allclose(T.silu_slope(x), fd, rtol=1e-6, atol=1e-9)


def test_silu_slope_extremum_and_interval_max():
    t = T.SILU_T_STAR
    # SiLU'' vanishes at t* and |SiLU'| peaks there at ~1.0998
    d2 = (T.silu_slope(t + 1e-5) - T.silu_slope(t - 1e-5)) / 2e-5
    assert abs(d2) < 1e-6 and abs(float(T.silu_slope(t)) - 1.0998) < 1e-4
    g = np.random.default_rng(11)
    lo = g.uniform(-12, 12, 400)
    hi = lo + g.exponential(2.0, 400)
    got = T.silu_slope_max(lo, hi)
    for a, b, m in zip(lo, hi, got):
        grid = np.linspace(a, b, 20001)
        brute = np.abs(T.silu_slope(grid)).max()
        assert brute <= m + 1e-12 and m - brute < 1e-6, (a, b, m, brute)


def test_silu_kappa_matches_its_definition():
    x = np.concatenate([np.linspace(-30, -0.01, 300), np.linspace(0.01, 30, 300)])
    silu = x * expit(x)
    assert np.allclose(T.silu_kappa(x), np.abs(x * T.silu_slope(x) / silu), rtol=1e-12)
    assert T.silu_kappa(np.array([50.0]))[0] == pytest.approx(1.0)
    assert T.silu_kappa(np.array([-50.0]))[0] == pytest.approx(49.0)
