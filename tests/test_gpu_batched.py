"""GPU parity of batched plans (batch problems of one shape per call, strides in bytes) against the
fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
import seeded_inputs as si
from gpu_util import exact_regime_problem, run
from oracle import compare, reference

pytestmark = pytest.mark.gpu

POISON = {"A": 0x7F, "B": 0x7F, "sA": 0xFF, "sB": 0xFF}  # NaN codes: a read of a gap byte poisons D


def _device_batch(arrays, stride, poison):
    """One device byte buffer holding arrays[z] (uint8) at byte offset z * stride; gap bytes = poison.
    stride 0: every problem reads arrays[0]."""
    n = arrays[0].nbytes
    size = n if stride == 0 else (len(arrays) - 1) * stride + n
    buf = np.full(size, poison, dtype=np.uint8)
    for z, a in enumerate(arrays if stride else arrays[:1]):
        buf[z * stride:z * stride + n] = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    return torch.from_numpy(buf).cuda()


def _run_batched(problems, strides, out="bf16", bias=False, silu=False):
    """Run the L problems as one batched plan; returns (D bits per problem, plan info)."""
    p0 = problems[0]
    L, M, N = len(problems), p0["M"], p0["N"]
    plan = bsg.Plan(p0["fmt"], M, N, p0["K"], out=out, bias=bias, silu=silu, batch=L, strides=strides)
    st = plan.strides
    dev = {k: _device_batch([q[k] for q in problems], st[kk], POISON[k])
           for k, kk in (("A", "a"), ("B", "b"), ("sA", "sa"), ("sB", "sb"))}
    bias_dev = None
    if bias:
        bias_dev = _device_batch([q["bias"].astype(np.float32) for q in problems], st["bias"], 0xFF)
    d_bytes = (L - 1) * st["d"] + 2 * M * N
    D = torch.full((d_bytes // 2,), 0x7FFF, dtype=torch.int16, device="cuda")
    plan.run(dev["A"], dev["B"], dev["sA"], dev["sB"], D, alpha=float(p0["alpha"]), bias=bias_dev)
    torch.cuda.synchronize()
    flat = D.cpu().numpy().view(np.uint16)
    outs = [flat[z * st["d"] // 2: z * st["d"] // 2 + M * N].reshape(M, N) for z in range(L)]
    info = plan.info()
    plan.close()
    return outs, info


def _share(problems, keys):
    for q in problems[1:]:
        for k in keys:
            q[k] = problems[0][k]
    return problems


@pytest.mark.parametrize("fmt,shape,L", [
    ("mxfp8", (96, 64, 256), 3), ("nvfp4", (96, 64, 256), 3),
    ("mxfp8", (1024, 1024, 512), 16),   # 16 tiles x 16 problems: the large-shape kernel
    ("nvfp4", (1024, 1024, 512), 16),   # ... and the 256 x 256 NVFP4 kernel
    ("nvfp4", (128, 1024, 4096), 2),    # split-K with one workspace slice per problem
    ("nvfp4", (128, 2048, 4096), 2),    # ... with 8 tiles: each tile's splits and finish on one XCD
    ("nvfp4", (128, 4096, 4096), 2),    # ... 4 MiB planes of streamed partials: two finish loads in flight
    ("mxfp8", (128, 1024, 4096), 2),    # (8 tiles of 128 x 128: the same placement)
], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_batched_exact_regime_bit_exact(fmt, shape, L):
    M, N, K = shape
    problems = [exact_regime_problem(fmt, M, N, K, seed=1000 * z + K, out="bf16") for z in range(L)]
    outs, info = _run_batched(problems, {})
    assert info["grid"][2] == L
    if K == 4096:  # split K: the workspace holds L x splits x M x N fp32 partials
        splits = info["grid"][0] // (N // info["tile"][1])
        assert splits > 1 and info["workspace_bytes"] == L * splits * M * N * 4
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 8)), [M - 1]]))
    for z, (q, D) in enumerate(zip(problems, outs)):
        assert not (D == 0x7FFF).any(), f"problem {z}: entries never written"
        R = reference(q, rows=rows)["bits"]
        assert np.array_equal(D[rows], R), f"problem {z}: {int((D[rows] != R).sum())} sampled entries differ"


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_batched_shared_b_padded_strides_bias_silu(fmt):
    M, N, K, L = 160, 96, 1024, 4
    problems = [si.problem(fmt, M, N, K, seed=70 + z, bias=True, silu=True, out="f16", alpha=0.5) for z in range(L)]
    problems = _share(problems, ("B", "sB"))  # one weight matrix for every problem
    pk = bsg.packed_strides(fmt, M, N, K)
    strides = dict(a=pk["a"] + 64, b=0, sa=pk["sa"] + 4 * 3, sb=0, bias=4 * N + 16, d=pk["d"] + 32)
    outs, _ = _run_batched(problems, strides, out="f16", bias=True, silu=True)
    for z, (q, D) in enumerate(zip(problems, outs)):
        rep = compare(D, reference(q), q["alpha"], q["silu"], q["out"])
        assert rep["ok"], (z, rep)


@pytest.mark.parametrize("fmt,shape", [("mxfp8", (130, 528, 1024)), ("nvfp4", (100, 80, 1056))])
def test_batched_equals_single_calls(fmt, shape):
    """A batched plan gives each problem the bits a single-problem plan of the same variant gives."""
    M, N, K = shape
    L = 3
    problems = [si.problem(fmt, M, N, K, seed=90 + z, out="bf16", alpha=0.75) for z in range(L)]
    outs, info = _run_batched(problems, {})
    single = bsg.Plan(fmt, M, N, K, out="bf16")
    sinfo = single.info()
    # same kernel and the same split of K: the same summation, so the same bits
    assert sinfo["variant"] == info["variant"] and sinfo["grid"][:2] == info["grid"][:2], (sinfo, info)
    for z, (q, D) in enumerate(zip(problems, outs)):
        assert np.array_equal(D, run(q, plan=single)), f"problem {z}"
    single.close()


def test_batched_split_partials_through_l2(monkeypatch, capfd):
    """Two 128x4096x8192 problems split 8 ways: 32 MiB of fp32 partials, one L2 per XCD, so the plan
    stores them through the L2, each problem's planes in its own workspace slice.  Exact regime:
    bit for bit against the oracle on sampled rows."""
    M, N, K, L = 128, 4096, 8192, 2
    monkeypatch.setenv("BSG_LOG", "1")
    problems = [exact_regime_problem("nvfp4", M, N, K, seed=7000 + z, out="bf16") for z in range(L)]
    outs, info = _run_batched(problems, {})
    log = capfd.readouterr().err
    assert "(partials through L2)" in log, log
    splits = info["grid"][0] // (N // info["tile"][1])
    assert info["workspace_bytes"] == L * splits * M * N * 4 >= 32 << 20, info
    rows = np.unique(np.concatenate([np.arange(0, M, 9), [M - 1]]))
    for z, (q, D) in enumerate(zip(problems, outs)):
        assert not (D == 0x7FFF).any(), f"problem {z}: entries never written"
        R = reference(q, rows=rows)["bits"]
        assert np.array_equal(D[rows], R), f"problem {z}: {int((D[rows] != R).sum())} sampled entries differ"
