"""Helpers for GPU tests: move a seeded problem to the device and run it through the C ABI."""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_precision_gemm_amd as bsg
import seeded_inputs as si


def to_device(p: dict) -> dict:
    d = dict(A=torch.from_numpy(np.ascontiguousarray(p["A"])).cuda(),
             B=torch.from_numpy(np.ascontiguousarray(p["B"])).cuda(),
             sA=torch.from_numpy(np.ascontiguousarray(p["sA"])).cuda(),
             sB=torch.from_numpy(np.ascontiguousarray(p["sB"])).cuda(),
             bias=None if p["bias"] is None else torch.from_numpy(np.ascontiguousarray(p["bias"])).cuda(),
             D=torch.empty((p["M"], p["N"]), dtype=torch.int16, device="cuda"))
    return d


def make_plan(p: dict) -> bsg.Plan:
    return bsg.Plan(p["fmt"], p["M"], p["N"], p["K"], out=p["out"], bias=p["bias"] is not None, silu=p["silu"])


def run(p: dict, plan: bsg.Plan | None = None, dev: dict | None = None, stream=None) -> np.ndarray:
    """Run the GEMM on the GPU; return D as uint16 bits [M, N]."""
    own = plan is None
    plan = plan or make_plan(p)
    dev = dev or to_device(p)
    dev["D"].fill_(0x7FFF)  # poison: every entry must be written
    plan.run(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], alpha=float(p["alpha"]), bias=dev["bias"],
             stream=stream)
    torch.cuda.synchronize()
    out = dev["D"].cpu().numpy().view(np.uint16).copy()
    if own:
        plan.close()
    return out


def exact_regime_problem(fmt, M, N, K, seed, out):
    """Products confined to a narrow exponent range with per-row / per-column constant scales: the
    MFMA's internal alignment then drops no bit and every fp32 partial sum is exact, so D must equal
    the oracle bit for bit."""
    g = np.random.default_rng(seed)
    if fmt == "mxfp8":  # E4M3 elements +-[1, 1.875] (exponent field 7), E8M0 scales constant along K
        A = ((g.integers(0, 2, (M, K)) << 7) | (7 << 3) | g.integers(0, 8, (M, K))).astype(np.uint8)
        B = ((g.integers(0, 2, (N, K)) << 7) | (7 << 3) | g.integers(0, 8, (N, K))).astype(np.uint8)
        sA = np.repeat(g.integers(118, 136, (M, 1)), K // 32, axis=1).astype(np.uint8)
        sB = np.repeat(g.integers(118, 136, (N, 1)), K // 32, axis=1).astype(np.uint8)
    else:  # E2M1 elements +-{1, 1.5}, E4M3 scales constant along K
        qa = (g.integers(0, 2, (M, K)) << 3 | g.integers(2, 4, (M, K))).astype(np.uint8)
        qb = (g.integers(0, 2, (N, K)) << 3 | g.integers(2, 4, (N, K))).astype(np.uint8)
        A, B = si.pack_e2m1(qa), si.pack_e2m1(qb)
        sA = np.repeat(g.integers(0x20, 0x50, (M, 1)), K // 16, axis=1).astype(np.uint8)
        sB = np.repeat(g.integers(0x20, 0x50, (N, 1)), K // 16, axis=1).astype(np.uint8)
    return dict(fmt=fmt, M=M, N=N, K=K, A=A, B=B, sA=sA, sB=sB, alpha=np.float32(0.5), bias=None, silu=False,
                out=out)
