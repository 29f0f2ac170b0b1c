"""Pins of the input quantisers (seeded_inputs): they only produce the synthetic operands, never a
result, but the workloads' value distributions depend on them.  Element rounding is checked against
a brute-force nearest-value search over each format's grid (ties to the even code), scales for
tightness, and whole quantised blocks against the dequantisation of the oracle (a separate
implementation) for the half-step error bound."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import oracle as O

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e4m3_positive_grid():
    """Every finite non-negative E4M3 value and its code (OCP E4M3: bias 7, subnormals, no inf)."""
    vals, codes = [], []
    for c in range(0x7F):  # 0x7F is NaN
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
        codes.append(c)
    return np.array(vals), np.array(codes)


def _nearest_even(v, grid, codes):
    """Index of the grid value nearest to v; a tie goes to the even code."""
    d = np.abs(grid[None, :] - v[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return codes[pick]


def test_e2m1_rounding_is_nearest_ties_to_even():
    g = np.random.default_rng(1)
    mids = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2  # every tie
    v = np.concatenate([g.uniform(0, 7, 4000), mids, E2M1_GRID, [6.5, 7.0]])
    x = np.concatenate([v, -v])
    got = si._to_e2m1_codes(x.astype(np.float32))
    want = _nearest_even(np.abs(x), E2M1_GRID, np.arange(8))
    want = np.where((x < 0) & (want != 0), want | 8, want)
    assert np.array_equal(got, want.astype(np.uint8))


def test_e4m3_rounding_is_nearest_ties_to_even():
    grid, codes = _e4m3_positive_grid()
    g = np.random.default_rng(2)
    mids = (grid[:-1] + grid[1:]) / 2
    v = np.concatenate([np.exp(g.uniform(np.log(2.0 ** -12), np.log(448.0), 4000)), mids, grid])
    v = v[v <= 448.0].astype(np.float32).astype(np.float64)  # as the quantiser sees them (fp32)
    got = si._to_e4m3_codes(v.astype(np.float32))
    assert np.array_equal(got, _nearest_even(v, grid, codes).astype(np.uint8))
    assert np.array_equal(si._to_e4m3_codes(np.array([500.0, -1e9], dtype=np.float32)), [0x7E, 0xFE])  # saturate


def _rows_with_outliers(seed, R=64, K=256):
    g = np.random.default_rng(seed)
    x = g.standard_normal((R, K)).astype(np.float32)
    x[g.choice(R, R // 8, replace=False)] *= 1000.0
    x[3, :32] = 0.0  # an all-zero block
    return x


def test_mxfp8_quantiser_scales_are_tight_and_error_is_half_a_step():
    x = _rows_with_outliers(3)
    codes, scales = si.quantize_mxfp8(x)
    assert not np.isin(codes, [0x7F, 0xFF]).any()
    R, K = x.shape
    s = O.decode_e8m0(scales).repeat(32, axis=1)
    v = O.decode_e4m3(codes) * s
    xb = np.abs(x).reshape(R, K // 32, 32).max(axis=2)
    peak = np.abs(O.decode_e4m3(codes)).reshape(R, K // 32, 32).max(axis=2)
    nz = xb > 0
    ratio = xb[nz] / O.decode_e8m0(scales)[nz]
    assert ((ratio > 224) & (ratio <= 448)).all()  # scale 2^ceil(log2(amax/448)): amax/scale in (224, 448]
    assert ((peak[nz] >= 224) & (peak[nz] <= 448)).all()  # rounding may take a ratio just above 224 to 224
    assert (scales[~nz] == 127).all() and (peak[~nz] == 0).all()
    # half an E4M3 step at the element's magnitude (below 2^-6: the subnormal step 2^-9)
    a = np.abs(x) / s
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert (np.abs(x - v) <= 0.5 * step * s * (1 + 2 ** -20)).all()


def test_nvfp4_quantiser_codes_and_error_bound():
    x = _rows_with_outliers(4)
    packed, scodes, gsc = si.quantize_nvfp4(x)
    assert not np.isin(scodes, [0x7F, 0xFF]).any()
    R, K = x.shape
    q = O.decode_e2m1(np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(R, K))
    sg = (O.decode_e4m3(scodes) * gsc).repeat(16, axis=1)
    assert (np.abs(q) <= 6).all()
    # the element is the nearest grid value to x / (s g) clipped to 6 (the block scale was itself
    # rounded to E4M3, so the block's largest element may exceed 6 s g by a fraction of a step)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(sg > 0, np.abs(x) / sg, 0.0)
    vc = np.minimum(v, 6.0)
    lo = E2M1_GRID[np.clip(np.searchsorted(E2M1_GRID, vc, side="right") - 1, 0, 7)]
    hi = E2M1_GRID[np.clip(np.searchsorted(E2M1_GRID, vc, side="left"), 0, 7)]
    err = np.abs(vc - np.abs(q))
    assert (err <= np.minimum(vc - lo, hi - vc) + 1e-6).all()
    assert (v[np.abs(q) == 6] >= 5.0).all() and (v.max(axis=1) <= 6 * (1 + 2 ** -3)).all()


def test_nvfp4_alpha_is_the_product_of_global_scales():
    g = np.random.default_rng(5)
    for _ in range(100):
        a, b = g.uniform(1e-3, 1e3, 2)
        ga, gb = np.float32(a / 2688.0), np.float32(b / 2688.0)
        assert float(si.nvfp4_alpha(a, b)) == pytest.approx(float(ga) * float(gb), rel=2 ** -22)
