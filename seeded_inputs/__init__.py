"""Seeded synthetic operands for the block-scaled GEMM.

This module only *produces* inputs: fp32 Gaussian matrices drawn from a
counter-seeded PCG64 stream, quantised on the host to the two operand
formats the GEMM consumes.  It performs none of the GEMM's arithmetic
(no decoding of codes into values, no products, no epilogue): both the
HIP path and the CPU oracle receive the bytes made here and nothing else.

Formats (OCP Microscaling v1.0 element types, as named on the CUTLASS
issue #3003 page and the nvFuser PR #5736 page, "Add Cutlass MxFp8 Block
Scale Matrix Multiplication", KernelTraits/MxFp8GemmSm100 and the test
`test_mxfp8_gemm`):

* MXFP8: E4M3 element codes, one E8M0 power-of-two scale per 32
  consecutive K elements.  Scale exponent e = ceil(log2(amax / 448)) per
  block, elements = E4M3 round-to-nearest-even of x * 2^-e, clamped to
  +-448 first.  An all-zero block gets scale code 127 (2^0).
* NVFP4: packed E2M1 codes (element 2t in the low nibble of byte t),
  one E4M3 scale per 16 K elements, and a global fp32 alpha.  Two-level
  recipe: g = amax_T / (448*6); s = E4M3_RNE((amax_blk/6)/g);
  q = E2M1_RNE(x / (s*g)) saturating at +-6 (q = 0 where s = 0);
  alpha = fp32(amax_A * amax_B / (448*6)^2).

Seeds: numpy.random.Generator(PCG64(SeedSequence([config, operand, set]))).
Operand ids: A=0, B=1, bias=2, outlier rows of A=3, outlier rows of B=4.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0
MX_BLOCK = 32
NV_BLOCK = 16

OP_A, OP_B, OP_BIAS, OP_OUTLIER_A, OP_OUTLIER_B = 0, 1, 2, 3, 4


def rng(config_id: int, operand_id: int, set_id: int = 0) -> np.random.Generator:
    """Counter-seeded generator: one independent stream per (config, operand, set)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, operand_id, set_id])))


def gaussian(config_id: int, operand_id: int, rows: int, cols: int, set_id: int = 0) -> np.ndarray:
    return rng(config_id, operand_id, set_id).standard_normal((rows, cols), dtype=np.float32)


def scale_outlier_rows(x: np.ndarray, config_id: int, operand_id: int, frac: float = 0.05,
                       factor: float = 1000.0, set_id: int = 0) -> np.ndarray:
    """Multiply round(frac*rows) distinct seeded rows of x by `factor` (in place, returns x)."""
    n = int(round(frac * x.shape[0]))
    rows = rng(config_id, operand_id, set_id).choice(x.shape[0], size=n, replace=False)
    x[rows, :] *= np.float32(factor)
    return x


def _to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> E4M3FN codes, round-to-nearest-even (torch's CPU cast), saturating at +-448."""
    xc = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    return torch.from_numpy(np.ascontiguousarray(xc)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_codes_to_f32(codes: np.ndarray) -> np.ndarray:
    # torch's own cast, used here only to re-derive the quantisation step size
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).float().numpy()


def _ceil_log2_ratio(amax: np.ndarray, denom_frac: float, denom_exp: int) -> np.ndarray:
    """Smallest integer e with denom * 2^e >= amax, denom = denom_frac * 2^denom_exp, exactly.

    amax = f * 2^E (frexp, f in [0.5, 1)).  denom*2^e >= amax  <=>  2^(e+denom_exp-E) >= f/denom_frac.
    """
    f, E = np.frexp(amax.astype(np.float64))
    e = E - denom_exp
    return np.where(f > denom_frac, e + 1, e)


def quantize_mxfp8(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp32 [R, K] -> (E4M3 codes uint8 [R, K], E8M0 scale codes uint8 [R, K/32])."""
    R, K = x.shape
    assert K % MX_BLOCK == 0
    xb = x.reshape(R, K // MX_BLOCK, MX_BLOCK).astype(np.float32)
    amax = np.abs(xb).max(axis=2)
    # 448 = 0.875 * 2^9
    e = _ceil_log2_ratio(amax, 0.875, 9)
    e = np.where(amax == 0, 0, e)
    e = np.clip(e, -127, 127)
    scaled = xb.astype(np.float64) * np.ldexp(1.0, -e)[:, :, None]
    codes = _to_e4m3_codes(scaled.astype(np.float32)).reshape(R, K)
    scales = (e + 127).astype(np.uint8)
    return codes, scales


def _to_e2m1_codes(a: np.ndarray) -> np.ndarray:
    """Round |a| to the E2M1 grid {0,.5,1,1.5,2,3,4,6} (ties to the even code), sign in bit 3."""
    m = np.abs(a)
    # crossing points between neighbouring codes; at an exact tie the even code wins
    code = ((m > 0.25).astype(np.uint8) + (m >= 0.75) + (m > 1.25) + (m >= 1.75)
            + (m > 2.5) + (m >= 3.5) + (m > 5.0)).astype(np.uint8)
    sign = ((a < 0) & (code != 0)).astype(np.uint8) << 3
    return code | sign


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [R, K] (values 0..15) -> packed uint8 [R, K/2]; element 2t = low nibble of byte t."""
    lo = codes[:, 0::2] & 0xF
    hi = codes[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def quantize_nvfp4(x: np.ndarray) -> tuple[np.ndarray, np.ndarray, float]:
    """fp32 [R, K] -> (packed E2M1 uint8 [R, K/2], E4M3 scale codes uint8 [R, K/16], global g)."""
    R, K = x.shape
    assert K % NV_BLOCK == 0
    xb = x.reshape(R, K // NV_BLOCK, NV_BLOCK).astype(np.float32)
    amax_t = float(np.abs(xb).max())
    g = np.float32(amax_t / (E4M3_MAX * E2M1_MAX)) if amax_t > 0 else np.float32(1.0)
    amax_b = np.abs(xb).max(axis=2)
    s_codes = _to_e4m3_codes((amax_b / np.float32(E2M1_MAX)) / g)
    s = _e4m3_codes_to_f32(s_codes).astype(np.float32)
    denom = s * g
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(denom[:, :, None] > 0, xb / denom[:, :, None], 0.0).astype(np.float32)
    ratio = np.clip(ratio, -E2M1_MAX, E2M1_MAX)
    q = _to_e2m1_codes(ratio).reshape(R, K)
    return pack_e2m1(q), s_codes.astype(np.uint8), float(g)


def nvfp4_alpha(amax_a: float, amax_b: float) -> np.float32:
    return np.float32(float(amax_a) * float(amax_b) / (E4M3_MAX * E2M1_MAX) ** 2)


# ---------------------------------------------------------------------------
# The five workloads, by name.  Each returns a dict of host arrays:
#   fmt ('mxfp8'|'nvfp4'), M, N, K, A, B, sA, sB, alpha (np.float32),
#   bias (fp32 [N] or None), silu (bool), out ('bf16'|'f16').
# ---------------------------------------------------------------------------

def mxfp8_problem(config_id: int, M: int, N: int, K: int, *, alpha: float = 1.0, bias: bool = False,
                  silu: bool = False, out: str = "bf16", outlier_rows: bool = False,
                  set_id: int = 0) -> dict:
    a = gaussian(config_id, OP_A, M, K, set_id)
    b = gaussian(config_id, OP_B, N, K, set_id)
    if outlier_rows:
        scale_outlier_rows(a, config_id, OP_OUTLIER_A, set_id=set_id)
        scale_outlier_rows(b, config_id, OP_OUTLIER_B, set_id=set_id)
    A, sA = quantize_mxfp8(a)
    B, sB = quantize_mxfp8(b)
    bias_v = rng(config_id, OP_BIAS, set_id).standard_normal(N, dtype=np.float32) if bias else None
    return dict(fmt="mxfp8", M=M, N=N, K=K, A=A, B=B, sA=sA, sB=sB, alpha=np.float32(alpha),
                bias=bias_v, silu=silu, out=out)


def nvfp4_problem(config_id: int, M: int, N: int, K: int, *, bias: bool = False, silu: bool = False,
                  out: str = "bf16", set_id: int = 0) -> dict:
    a = gaussian(config_id, OP_A, M, K, set_id)
    b = gaussian(config_id, OP_B, N, K, set_id)
    A, sA, _ = quantize_nvfp4(a)
    B, sB, _ = quantize_nvfp4(b)
    alpha = nvfp4_alpha(np.abs(a).max(), np.abs(b).max())
    bias_v = rng(config_id, OP_BIAS, set_id).standard_normal(N, dtype=np.float32) if bias else None
    return dict(fmt="nvfp4", M=M, N=N, K=K, A=A, B=B, sA=sA, sB=sB, alpha=alpha,
                bias=bias_v, silu=silu, out=out)


WORKLOADS = {
    "mxfp8_256": dict(desc="MXFP8 GEMM M=N=K=256, bf16 out, alpha=1"),
    "mxfp8_4096": dict(desc="MXFP8 GEMM M=N=K=4096, 5% outlier rows x1000, bf16 out, alpha=0.5"),
    "mxfp8_8192_silu": dict(desc="MXFP8 GEMM M=N=K=8192, fp16 out, D=SiLU(alpha*AB^T+bias), alpha=1"),
    "nvfp4_128x8192x8192_silu": dict(desc="NVFP4 GEMM M=128 N=K=8192, bias+SiLU, bf16 out"),
    "nvfp4_256x4096x4096_loop": dict(desc="NVFP4 GEMM M=256 N=K=4096, bf16 out, 10 input sets"),
}


def workload(name: str, set_id: int = 0) -> dict:
    if name == "mxfp8_256":
        return mxfp8_problem(1, 256, 256, 256, alpha=1.0, out="bf16", set_id=set_id)
    if name == "mxfp8_4096":
        return mxfp8_problem(2, 4096, 4096, 4096, alpha=0.5, out="bf16", outlier_rows=True, set_id=set_id)
    if name == "mxfp8_8192_silu":
        return mxfp8_problem(3, 8192, 8192, 8192, alpha=1.0, bias=True, silu=True, out="f16", set_id=set_id)
    if name == "nvfp4_128x8192x8192_silu":
        return nvfp4_problem(4, 128, 8192, 8192, bias=True, silu=True, out="bf16", set_id=set_id)
    if name == "nvfp4_256x4096x4096_loop":
        return nvfp4_problem(5, 256, 4096, 4096, out="bf16", set_id=set_id)
    raise KeyError(name)


def problem(fmt: str, M: int, N: int, K: int, seed: int, *, alpha=None, bias=False, silu=False,
            out="bf16", outlier_rows=False) -> dict:
    """A generic seeded problem of either format (parity-test shapes)."""
    if fmt == "mxfp8":
        return mxfp8_problem(seed, M, N, K, alpha=1.0 if alpha is None else alpha, bias=bias, silu=silu,
                             out=out, outlier_rows=outlier_rows)
    p = nvfp4_problem(seed, M, N, K, bias=bias, silu=silu, out=out)
    if alpha is not None:
        p["alpha"] = np.float32(alpha)
    return p
