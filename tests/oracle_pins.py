"""Pins of the CPU oracle to facts fixed outside it.

Each pin_* function raises AssertionError when the oracle disagrees with a
library routine, a spec table, a closed form, an exact rational brute force or
a hand-worked example.  tests/test_oracle_pins.py runs them; and
tests/test_oracle_mutants.py plants plausible mistakes in the oracle and checks
that at least one pin fails for each.

All oracle calls go through the module object O so that a planted mistake
(monkeypatched attribute) is seen by every call path.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import scipy.special
import torch

import seeded_inputs as si
from oracle import tolerance as C
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _kv_fixture(name):
    return {r[0]: r[1:] for r in _read_fixture(name)}


def _torch_e4m3(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, dtype=np.uint8)))
    return t.view(torch.float8_e4m3fn).double().numpy()


def _torch_e8m0(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, dtype=np.uint8)))
    return t.view(torch.float8_e8m0fnu).double().numpy()


def _e2m1_table() -> np.ndarray:
    return np.array([float(v) for _, v in _read_fixture("e2m1_values.txt")])


def _same(a, b) -> bool:
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return a.shape == b.shape and bool(np.all((a == b) | (np.isnan(a) & np.isnan(b)))) and \
        bool(np.all(np.signbit(a[a == 0]) == np.signbit(b[a == 0])))


# ----------------------------------------------------------------- codecs

def pin_e4m3_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    assert _same(O.decode_e4m3(codes), _torch_e4m3(codes)), "E4M3 decode != torch float8_e4m3fn"


def pin_e4m3_landmarks():
    for code_hex, val in _read_fixture("e4m3_landmarks.txt"):
        got = float(O.decode_e4m3(np.array([int(code_hex, 16)]))[0])
        want = float(val)
        assert (math.isnan(got) and math.isnan(want)) or (got == want and
                                                           math.copysign(1, got) == math.copysign(1, want)), \
            f"E4M3 {code_hex}: {got} != {want}"


def pin_e8m0_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = O.decode_e8m0(codes)
    assert _same(got, _torch_e8m0(codes)), "E8M0 decode != torch float8_e8m0fnu"
    # closed form: code 127 is 1, each code step doubles, code 255 is NaN
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127 and math.isnan(got[255])
    assert np.all(got[1:255] == 2.0 * got[0:254])


def pin_e2m1_table():
    codes = np.arange(16)
    assert _same(O.decode_e2m1(codes), _e2m1_table()), "E2M1 decode != OCP table"


def pin_e2m1_unpack_inverts_pack():
    # the packing convention (element 2t in the low nibble of byte t) is written once on the
    # generator side; the oracle's unpacking must invert it.  The GEMM itself cannot see this
    # convention when A and B share it, so it is pinned here, at the decode level.
    g = np.random.default_rng(5)
    codes = g.integers(0, 16, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(O.unpack_e2m1(si.pack_e2m1(codes), 64), codes), "unpack(pack(q)) != q"
    assert np.array_equal(O.unpack_e2m1(np.array([[0x21]], np.uint8), 2), np.array([[1, 2]], np.uint8))


def pin_nvfp4_products_exact_in_bf16_and_f16():
    q = O.decode_e2m1(np.arange(16))[:, None]
    s = O.decode_e4m3(np.arange(256))[None, :]
    prod = (q * s)[:, ~np.isnan(s[0])]
    t = torch.from_numpy(prod)
    assert torch.equal(t.to(torch.bfloat16).double(), t), "an E2M1 x E4M3 product is not exact in bf16"
    assert torch.equal(t.to(torch.float16).double(), t), "an E2M1 x E4M3 product is not exact in fp16"
    # and the product set equals table(E2M1) x torch(E4M3)
    want = _e2m1_table()[:, None] * _torch_e4m3(np.arange(256))[None, :]
    assert _same(prod, want[:, ~np.isnan(want[0])])


# ----------------------------------------------------------------- worked examples

def _fixture_bytes(tokens):
    return np.array([int(t, 16) for t in tokens], dtype=np.uint8)


def pin_nvfp4_worked_example():
    kv = _kv_fixture("nvfp4_worked.txt")
    K = int(kv["K"][0])
    p = dict(fmt="nvfp4", M=1, N=1, K=K, A=_fixture_bytes(kv["A"])[None, :], B=_fixture_bytes(kv["B"])[None, :],
             sA=_fixture_bytes(kv["sA"])[None, :], sB=_fixture_bytes(kv["sB"])[None, :],
             alpha=np.float32(float(kv["alpha"][0])), bias=np.array([float(kv["bias"][0])], np.float32),
             silu=False, out="bf16")
    r = O.reference(p)
    assert r["acc"][0, 0] == float(kv["acc"][0]), f"acc {r['acc'][0, 0]}"
    assert r["y"][0, 0] == float(kv["y"][0]), f"y {r['y'][0, 0]}"
    assert int(r["bits"][0, 0]) == int(kv["bf16_bits"][0], 16)
    p["silu"] = True
    r = O.reference(p)
    assert abs(r["y"][0, 0] - float(kv["y_silu"][0])) <= 1e-15 * 6.1, f"silu {r['y'][0, 0]}"


def pin_mxfp8_worked_example():
    kv = _kv_fixture("mxfp8_worked.txt")
    K = int(kv["K"][0])

    def row(tokens):
        r = np.zeros(K, dtype=np.uint8)
        for t in tokens:
            k, v = t.split(":")
            r[int(k)] = int(v, 16)
        return r

    A = np.stack([row(kv["A0"]), row(kv["A1"])])
    B = np.stack([row(kv["B0"]), row(kv["B1"])])
    sA = _fixture_bytes(kv["sA"]).reshape(2, 2)
    sB = _fixture_bytes(kv["sB"]).reshape(2, 2)
    p = dict(fmt="mxfp8", M=2, N=2, K=K, A=A, B=B, sA=sA, sB=sB, alpha=np.float32(1.0), bias=None,
             silu=False, out="bf16")
    r = O.reference(p)
    assert np.array_equal(r["acc"].ravel(), np.array([float(x) for x in kv["acc"]])), f"acc {r['acc']}"
    assert np.array_equal(r["bits"].ravel(), np.array([int(x, 16) for x in kv["bf16_bits"]], np.uint16))


# ----------------------------------------------------------------- exact rational brute force

def _fraction_gemm(a_vals, b_vals, sa_vals, sb_vals, blk):
    """Exact sum_k (a[i,k] sa[i,k//blk]) (b[j,k] sb[j,k//blk]) with Fractions."""
    M, K = a_vals.shape
    N = b_vals.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            tot = Fraction(0)
            for blk_i in range(K // blk):
                fa, fb = Fraction(float(sa_vals[i, blk_i])), Fraction(float(sb_vals[j, blk_i]))
                for kk in range(blk):
                    k = blk_i * blk + kk
                    tot += Fraction(float(a_vals[i, k])) * fa * Fraction(float(b_vals[j, k])) * fb
            out[i][j] = tot
    return out


def _finite_e4m3_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def _mx_case(seed, M, N, K, scale_lo, scale_hi):
    g = np.random.default_rng(seed)
    codes = _finite_e4m3_codes()
    A = g.choice(codes, size=(M, K))
    B = g.choice(codes, size=(N, K))
    assert A.size >= len(codes)
    A.ravel()[: len(codes)] = codes  # every finite code appears
    sA = g.integers(scale_lo, scale_hi + 1, size=(M, K // 32)).astype(np.uint8)
    sB = g.integers(scale_lo, scale_hi + 1, size=(N, K // 32)).astype(np.uint8)
    return A.astype(np.uint8), B.astype(np.uint8), sA, sB


def pin_mxfp8_fraction_exact():
    # scales within 2^-2..2^2: every partial sum has < 53 significant bits, so fp64 must be exact
    A, B, sA, sB = _mx_case(11, 4, 3, 64, 125, 129)
    want = _fraction_gemm(_torch_e4m3(A), _torch_e4m3(B), _torch_e8m0(sA), _torch_e8m0(sB), 32)
    p = dict(fmt="mxfp8", M=4, N=3, K=64, A=A, B=B, sA=sA, sB=sB, alpha=np.float32(1), bias=None, silu=False,
             out="bf16")
    acc = O.reference(p)["acc"]
    for i in range(4):
        for j in range(3):
            assert Fraction(float(acc[i, j])) == want[i][j], f"mxfp8 acc[{i},{j}] {acc[i, j]} != {float(want[i][j])}"


def pin_mxfp8_fraction_wide_scales():
    # full scale range: fp64 is then only within its summation bound K * 2^-53 * sum|ab|
    A, B, sA, sB = _mx_case(12, 3, 4, 96, 1, 254)
    want = _fraction_gemm(_torch_e4m3(A), _torch_e4m3(B), _torch_e8m0(sA), _torch_e8m0(sB), 32)
    absw = _fraction_gemm(np.abs(_torch_e4m3(A)), np.abs(_torch_e4m3(B)), _torch_e8m0(sA), _torch_e8m0(sB), 32)
    p = dict(fmt="mxfp8", M=3, N=4, K=96, A=A, B=B, sA=sA, sB=sB, alpha=np.float32(1), bias=None, silu=False,
             out="bf16")
    r = O.reference(p)
    for i in range(3):
        for j in range(4):
            bound = 96 * 2.0 ** -53 * float(absw[i][j])
            assert abs(Fraction(float(r["acc"][i, j])) - want[i][j]) <= Fraction(bound), f"acc[{i},{j}]"
            assert abs(float(r["S"][i, j]) - float(absw[i][j])) <= bound, f"S[{i},{j}]"


def pin_nvfp4_fraction_exact():
    g = np.random.default_rng(21)
    M, N, K = 3, 4, 64
    qa = g.integers(0, 16, size=(M, K)).astype(np.uint8)
    qb = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    qa[0, :16] = np.arange(16)  # every code appears
    finite = _finite_e4m3_codes()
    sA = g.choice(finite, size=(M, K // 16)).astype(np.uint8)
    sB = g.choice(finite, size=(N, K // 16)).astype(np.uint8)
    table = _e2m1_table()
    want = _fraction_gemm(table[qa], table[qb], _torch_e4m3(sA), _torch_e4m3(sB), 16)
    p = dict(fmt="nvfp4", M=M, N=N, K=K, A=si.pack_e2m1(qa), B=si.pack_e2m1(qb), sA=sA, sB=sB,
             alpha=np.float32(1), bias=None, silu=False, out="bf16")
    acc = O.reference(p)["acc"]
    for i in range(M):
        for j in range(N):
            assert Fraction(float(acc[i, j])) == want[i][j], f"nvfp4 acc[{i},{j}] {acc[i, j]} != {float(want[i][j])}"


# ----------------------------------------------------------------- library special case

def pin_mxfp8_unit_scales_vs_torch_matmul():
    g = np.random.default_rng(31)
    codes = _finite_e4m3_codes()
    normal = codes[((codes >> 3) & 0xF) >= 1]
    M, N, K = 96, 80, 256
    A = g.choice(normal, size=(M, K)).astype(np.uint8)
    B = g.choice(normal, size=(N, K)).astype(np.uint8)
    ones = lambda r: np.full((r, K // 32), 127, np.uint8)  # noqa: E731
    p = dict(fmt="mxfp8", M=M, N=N, K=K, A=A, B=B, sA=ones(M), sB=ones(N), alpha=np.float32(1), bias=None,
             silu=False, out="bf16")
    acc = O.reference(p)["acc"]
    ta = torch.from_numpy(A).view(torch.float8_e4m3fn).double()
    tb = torch.from_numpy(B).view(torch.float8_e4m3fn).double()
    want = (ta @ tb.T).numpy()
    assert np.array_equal(acc, want), "unit-scale MXFP8 GEMM != torch fp64 matmul"


# ----------------------------------------------------------------- closed forms

def _mx_identity_problem(n, seed, perm=None):
    g = np.random.default_rng(seed)
    A = np.zeros((n, n), np.uint8)
    rows = np.arange(n)
    cols = rows if perm is None else perm
    A[rows, cols] = 0x38  # 1.0
    B = g.choice(_finite_e4m3_codes(), size=(n, n)).astype(np.uint8)
    sA = np.full((n, n // 32), 127, np.uint8)
    sB = g.integers(110, 145, size=(n, n // 32)).astype(np.uint8)
    return dict(fmt="mxfp8", M=n, N=n, K=n, A=A, B=B, sA=sA, sB=sB, alpha=np.float32(1), bias=None, silu=False,
                out="bf16")


def pin_identity_and_permutation():
    n = 64
    p = _mx_identity_problem(n, 41)
    b = _torch_e4m3(p["B"]) * np.repeat(_torch_e8m0(p["sB"]), 32, axis=1)
    r = O.reference(p)
    assert np.array_equal(r["y"], b.T), "I x B^T != B^T"
    assert np.array_equal(O.bits_to_f64(r["bits"], "bf16"), b.T), "bf16 of exact E4M3 values must be exact"
    perm = np.random.default_rng(42).permutation(n)
    p = _mx_identity_problem(n, 41, perm)
    r = O.reference(p)
    assert np.array_equal(r["y"], b.T[perm, :]), "P x B^T != permuted rows of B^T"
    # NVFP4 identity: E2M1 code 2 (1.0) on the diagonal, E4M3 scale 0x38 (1.0)
    qa = np.zeros((32, 32), np.uint8)
    qa[np.arange(32), np.arange(32)] = 2
    g = np.random.default_rng(43)
    qb = g.integers(0, 16, size=(32, 32)).astype(np.uint8)
    sB = g.choice(_finite_e4m3_codes(), size=(32, 2)).astype(np.uint8)
    p = dict(fmt="nvfp4", M=32, N=32, K=32, A=si.pack_e2m1(qa), B=si.pack_e2m1(qb), sA=np.full((32, 2), 0x38, np.uint8),
             sB=sB, alpha=np.float32(1), bias=None, silu=False, out="f16")
    b = _e2m1_table()[qb] * np.repeat(_torch_e4m3(sB), 16, axis=1)
    r = O.reference(p)
    assert np.array_equal(r["y"], b.T), "NVFP4 I x B^T != B^T"


def pin_power_of_two_scaling():
    p = si.problem("mxfp8", 48, 40, 128, seed=51)
    base = O.reference(p)
    for k in (1, 3, -2):
        q = dict(p)
        q["sA"] = (p["sA"].astype(np.int64) + k).astype(np.uint8)
        r = O.reference(q)
        assert np.array_equal(r["acc"], base["acc"] * 2.0 ** k), f"sA code +{k} must scale acc by 2^{k}"
        assert np.array_equal(r["y"], base["y"] * 2.0 ** k)
        # bf16 rounding commutes with 2^k in the normal range: same mantissa bits, exponent +k
        nz = base["bits"] & 0x7FFF != 0
        assert np.array_equal((r["bits"][nz].astype(np.int64) - base["bits"][nz]) >> 7, np.full(nz.sum(), k))


def pin_all_ones_blocks():
    for K in (32, 96, 256):
        for ca, cb in ((127, 127), (120, 131), (130, 100)):
            M, N = 5, 7
            p = dict(fmt="mxfp8", M=M, N=N, K=K, A=np.full((M, K), 0x38, np.uint8), B=np.full((N, K), 0x38, np.uint8),
                     sA=np.full((M, K // 32), ca, np.uint8), sB=np.full((N, K // 32), cb, np.uint8),
                     alpha=np.float32(0.75), bias=None, silu=False, out="f16")
            r = O.reference(p)
            want = 0.75 * K * 2.0 ** (ca - 127) * 2.0 ** (cb - 127)
            assert np.all(r["y"] == want), f"all-ones K={K} {ca},{cb}"
    # NVFP4: E2M1 1.0 (code 2) everywhere, scales 1.5 (0x3c) and 0.25 (0x28)
    K = 64
    p = dict(fmt="nvfp4", M=3, N=2, K=K, A=np.full((3, K // 2), 0x22, np.uint8), B=np.full((2, K // 2), 0x22, np.uint8),
             sA=np.full((3, K // 16), 0x3C, np.uint8), sB=np.full((2, K // 16), 0x28, np.uint8),
             alpha=np.float32(2.0), bias=np.array([1.0, -3.0], np.float32), silu=False, out="bf16")
    r = O.reference(p)
    assert np.array_equal(r["y"], np.array([[2 * K * 1.5 * 0.25 + 1.0, 2 * K * 1.5 * 0.25 - 3.0]] * 3))


def pin_epilogue():
    x = np.linspace(-30, 30, 1201)
    y = O.epilogue(x[None, :], np.float32(1.0), None, True)[0]
    want = x * scipy.special.expit(x)
    assert np.allclose(y, want, rtol=1e-14, atol=1e-300), "SiLU != x * expit(x)"
    assert O.epilogue(np.zeros((1, 1)), np.float32(1), None, True)[0, 0] == 0.0
    ypos = O.epilogue(x[None, :], np.float32(1), None, True)[0]
    yneg = O.epilogue(-x[None, :], np.float32(1), None, True)[0]
    assert np.allclose(ypos - yneg, x, rtol=1e-13, atol=1e-13), "SiLU(x) - SiLU(-x) must equal x"
    assert O.epilogue(np.array([[1000.0]]), np.float32(1), None, True)[0, 0] == 1000.0
    assert O.epilogue(np.array([[-1000.0]]), np.float32(1), None, True)[0, 0] == 0.0
    # order: SiLU(alpha * acc + bias), bias per column, alpha at its fp32 value
    acc = np.array([[2.0, 2.0]])
    y = O.epilogue(acc, np.float32(0.1), np.array([0.5, -0.5], np.float32), True)[0]
    a32 = float(np.float32(0.1))
    t = np.array([a32 * 2.0 + 0.5, a32 * 2.0 - 0.5])
    assert np.allclose(y, t * scipy.special.expit(t), rtol=1e-15)


def _neighbours_ok(y, bits, nbits_mant, to_f64):
    """R must be one of the two representable neighbours of y, the nearer one, ties to the even code."""
    R = to_f64(bits)
    up = to_f64((bits.astype(np.int64) + 1).astype(np.uint16))
    dn = to_f64((bits.astype(np.int64) - 1).astype(np.uint16))
    fin = np.isfinite(R) & np.isfinite(up) & np.isfinite(dn) & ((bits & 0x7FFF) != 0)
    y, R, up, dn, b = y[fin], R[fin], up[fin], dn[fin], bits[fin]
    dR, du, dd = np.abs(y - R), np.abs(y - up), np.abs(y - dn)
    assert np.all(dR <= du) and np.all(dR <= dd), "not the nearest representable value"
    tie = (dR == du) | (dR == dd)
    assert np.all(b[tie] & 1 == 0), "ties must go to the even code"


def pin_output_rounding():
    g = np.random.default_rng(61)
    y = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-6, 6, 20000),
                        1.0 + np.arange(-300, 300) * 2.0 ** -10, 3.0 + np.arange(-300, 300) * 2.0 ** -13])
    _neighbours_ok(y, O.round_to_bf16_bits(y), 7, lambda b: O.bits_to_f64(b, "bf16"))
    _neighbours_ok(y, O.round_to_f16_bits(y), 10, lambda b: O.bits_to_f64(b, "f16"))
    # direct rounding from fp64: just above a tie goes up (no double rounding through fp32)
    assert O.round_to_bf16_bits(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert O.round_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert O.round_to_f16_bits(np.array([1.0 + 2.0 ** -11 + 2.0 ** -40]))[0] == 0x3C01
    assert O.round_to_bf16_bits(np.array([3.5e38]))[0] == 0x7F80
    assert O.round_to_f16_bits(np.array([-70000.0]))[0] == 0xFC00
    # bf16 values round-trip; torch agrees on values exactly representable in fp32
    t = torch.from_numpy(g.standard_normal(5000).astype(np.float32))
    want = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.round_to_bf16_bits(t.double().numpy()), want), "bf16 RNE != torch on fp32 inputs"


def pin_tolerance_rejects_wrong_values():
    p = si.problem("mxfp8", 64, 48, 256, seed=71, alpha=0.5)
    ref = O.reference(p)
    assert C.compare(ref["bits"], ref, p["alpha"], False, "bf16")["ok"]
    bad = ref["bits"].copy()
    D = O.bits_to_f64(bad, "bf16")
    big = np.argwhere(np.abs(D) > 4.0)[0]
    bad[tuple(big)] = O.round_to_bf16_bits(np.array([D[tuple(big)] * 1.05]))[0]
    rep = C.compare(bad, ref, p["alpha"], False, "bf16")
    assert not rep["ok"] and rep["n_bad"] == 1, "a 5% error must fail"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
