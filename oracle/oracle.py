"""CPU oracle for the block-scaled GEMM D = epi(alpha * A x B^T) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The library never calls it; it shares no code, table or constant
with the HIP path.  Everything here is plain fp64 numpy, written from the
definitions, in the order the pages state them:

* The operation: the nvFuser PR #5736 page ("Add Cutlass MxFp8 Block Scale
  Matrix Multiplication"), sequence diagram, "compute C = alpha * A @ B", with
  A row-major M x K and B stored K-contiguous as N x K (layout tags RowMajor /
  ColumnMajor in MxFp8GemmSm100, the test builds b as randn((n, k))), fp32
  accumulation (ElementAccumulator = float), FP16/BF16 output, and a reference
  that dequantises and multiplies (test_mxfp8_gemm / get_ref_results).
* MXFP8: E4M3 elements with one E8M0 scale per 32 K elements (same page,
  ElementA = mx_float8_t<float_e4m3_t>, ElementSFA = float_ue8m0_t,
  block_size = 32).
* NVFP4 and the fused epilogue: the CUTLASS issue #3003 page ("[QST]
  Performance overhead ..."), runNvfp4Gemm<T, kEnableSilu, kEnableBias>(...,
  bias, float alpha, M, N, K).  The page names NVFP4 but defines neither its
  block size nor its scale type; the reading used here is packed E2M1 with
  one E4M3 scale per 16 K elements and a global fp32 alpha.
* Bit-level element formats are not defined on the pages; they follow the
  OCP Microscaling v1.0 definitions of E4M3, E8M0 and E2M1.

Parity of every function below is pinned by tests that do not re-type its
formula (library casts, exhaustive tables from the spec, closed forms,
exact rational brute force).
"""
from __future__ import annotations

import numpy as np

MX_BLOCK = 32
NV_BLOCK = 16


# --------------------------------------------------------------------------
# Element and scale decoding (OCP MX v1.0 bit layouts)
# --------------------------------------------------------------------------

def decode_e4m3(codes) -> np.ndarray:
    """E4M3FN code -> exact fp64 value.

    sign s = bit 7, exponent e = bits 6..3 (bias 7), mantissa m = bits 2..0.
    e >= 1: (-1)^s 2^(e-7) (1 + m/8);  e = 0: (-1)^s 2^-6 (m/8);  e = 15, m = 7: NaN.
    No infinities; the largest finite magnitude is 448.
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    subnormal = np.ldexp(m / 8.0, -6)
    mag = np.where(e == 0, subnormal, normal)
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def decode_e8m0(codes) -> np.ndarray:
    """E8M0 code -> exact fp64 power of two 2^(e-127); code 255 is NaN."""
    e = np.asarray(codes).astype(np.int64)
    val = np.ldexp(np.ones(e.shape), e - 127)
    return np.where(e == 255, np.nan, val)


def decode_e2m1(codes) -> np.ndarray:
    """E2M1 nibble -> exact fp64 value.

    sign = bit 3, exponent e = bits 2..1 (bias 1), mantissa m = bit 0.
    e >= 1: (-1)^s 2^(e-1) (1 + m/2);  e = 0: (-1)^s (m/2).
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m / 2.0, np.ldexp(1.0 + m / 2.0, e - 1))
    return np.where(s == 1, -mag, mag)


def unpack_e2m1(packed: np.ndarray, K: int) -> np.ndarray:
    """uint8 [R, K/2] -> nibble codes [R, K]; element k = 2t is the low nibble of byte t."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], K), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# Dequantisation: value = element * scale of the block holding k
# --------------------------------------------------------------------------

def _decode_by_table(decode, codes, n_codes: int) -> np.ndarray:
    """decode(codes) for a large code array: decode each of the n_codes possible codes once, then index."""
    return decode(np.arange(n_codes))[np.asarray(codes, dtype=np.uint8)]


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[R, K] E4M3 codes, [R, K/32] E8M0 codes -> exact fp64 [R, K].

    Block b covers k in [32b, 32b + 32).
    """
    R, K = codes.shape
    assert scales.shape == (R, K // MX_BLOCK)
    out = _decode_by_table(decode_e4m3, codes, 256)
    out *= np.repeat(_decode_by_table(decode_e8m0, scales, 256), MX_BLOCK, axis=1)
    return out


def dequant_nvfp4(packed: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """[R, K/2] packed E2M1, [R, K/16] E4M3 scale codes -> exact fp64 [R, K].

    Block b covers k in [16b, 16b + 16).  Each product has at most 6 significant
    bits, so it is exact in fp64 (and in bf16/fp16).
    """
    R = packed.shape[0]
    assert packed.shape == (R, K // 2) and scales.shape == (R, K // NV_BLOCK)
    out = _decode_by_table(decode_e2m1, unpack_e2m1(packed, K), 16)
    out *= np.repeat(_decode_by_table(decode_e4m3, scales, 256), NV_BLOCK, axis=1)
    return out


def dequant(fmt: str, data: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    if fmt == "mxfp8":
        return dequant_mxfp8(data, scales)
    if fmt == "nvfp4":
        return dequant_nvfp4(data, scales, K)
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# Contraction, epilogue, output rounding
# --------------------------------------------------------------------------

def contract(a: np.ndarray, b: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """acc[i, j] = sum_k a[i, k] * b[j, k] (A x B^T) and S[i, j] = sum_k |a[i, k] * b[j, k]|.

    Both in fp64; S bounds the rounding error of any summation order.
    """
    return a @ b.T, np.abs(a) @ np.abs(b).T


def epilogue(acc: np.ndarray, alpha, bias, silu: bool) -> np.ndarray:
    """y = alpha * acc + bias[j]; then y / (1 + exp(-y)) when SiLU is on.  fp64.

    alpha and bias are taken at the fp32 values the GPU receives.
    """
    y = float(np.float32(alpha)) * acc
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    if silu:
        with np.errstate(over="ignore"):
            y = y / (1.0 + np.exp(-y))
    return y


def round_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit pattern (uint16), one round-to-nearest-even step.

    Rounding straight from fp64 (8 significant bits kept) avoids the double
    rounding of going through fp32.  Overflow -> +-inf; NaN -> canonical NaN.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.float64)
    finite = np.isfinite(y)
    yf = np.where(finite, y, 0.0)
    mant, ex = np.frexp(yf)                      # yf = mant * 2^ex, 0.5 <= |mant| < 1
    # normal range: keep 8 significant bits (np.round is half-to-even)
    normal = np.ldexp(np.round(np.ldexp(mant, 8)), ex - 8)
    # below the smallest normal 2^-126 the quantum is fixed at 2^-133
    sub = np.ldexp(np.round(np.ldexp(yf, 133)), -133)
    r = np.where(np.abs(yf) < 2.0 ** -126, sub, normal)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, yf), r)
    out[...] = np.where(finite, r, y)
    f32 = out.astype(np.float32)                 # exact: r has <= 8 significant bits
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.isnan(out), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def round_to_f16_bits(y: np.ndarray) -> np.ndarray:
    """fp64 -> IEEE binary16 bit pattern, numpy's direct round-to-nearest-even cast."""
    with np.errstate(over="ignore"):
        return np.asarray(y, dtype=np.float64).astype(np.float16).view(np.uint16)


def round_output(y: np.ndarray, out: str) -> np.ndarray:
    if out == "bf16":
        return round_to_bf16_bits(y)
    if out == "f16":
        return round_to_f16_bits(y)
    raise ValueError(out)


def bits_to_f64(bits: np.ndarray, out: str) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if out == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# Whole reference
# --------------------------------------------------------------------------

def reference(p: dict, rows=None) -> dict:
    """Oracle for a problem dict (fmt, M, N, K, A, B, sA, sB, alpha, bias, silu, out).

    rows: optional index array; then only those rows of D are computed (all N
    columns), for sampled checks at full size.
    Returns dict(bits=[r, N] uint16, y=fp64 before rounding, x=alpha*acc + bias (the epilogue's
    input), S=sum |a b|, acc=fp64 sum, fmt, K).
    """
    fmt, K = p["fmt"], p["K"]
    A, sA = p["A"], p["sA"]
    if rows is not None:
        rows = np.asarray(rows)
        A, sA = A[rows], sA[rows]
    a = dequant(fmt, A, sA, K)
    b = dequant(fmt, p["B"], p["sB"], K)
    acc, S = contract(a, b)
    x = epilogue(acc, p["alpha"], p["bias"], False)
    y = epilogue(acc, p["alpha"], p["bias"], p["silu"])
    return dict(bits=round_output(y, p["out"]), y=y, x=x, S=S, acc=acc, fmt=fmt, K=K)

