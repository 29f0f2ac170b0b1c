"""Helpers for GPU tests: move a seeded problem to the device and run it through the C ABI."""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_precision_gemm_amd as bsg


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
