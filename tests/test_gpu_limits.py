"""GPU parity at the largest accepted sizes: operands and outputs just under 2^31 elements (the bound
plan creation enforces), on each kernel that serves such shapes.  Offsets of whole rows are 64-bit
and offsets inside a tile 32-bit; these cases put both at their limits.

Operands are exact-regime codes (see exact_regime_problem: every fp32 partial sum exact, so D must
equal the oracle bit for bit) drawn on the device by torch's seeded generator -- a 2 GiB operand
takes a minute from numpy -- and the oracle checks a sub-problem: D[m, n] depends only on row m of A
and row n of B, so sampled rows of A and of B give D at the sampled rows x columns."""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
from oracle import reference

pytestmark = pytest.mark.gpu


def _codes(fmt, rows, K, gen):
    """Exact-regime element codes on the device: MXFP8 E4M3 +-[1, 1.875] (exponent field 7); NVFP4
    E2M1 +-{1, 1.5} in both nibbles of each byte."""
    if fmt == "mxfp8":
        x = torch.randint(0, 256, (rows, K), dtype=torch.uint8, device="cuda", generator=gen)
        return x.bitwise_and_(0x87).bitwise_or_(0x38)
    x = torch.randint(0, 256, (rows, K // 2), dtype=torch.uint8, device="cuda", generator=gen)
    return x.bitwise_and_(0x99).bitwise_or_(0x22)


def _scales(fmt, rows, K, gen):
    """One power-of-two scale code per row, constant along K: E8M0 2^-9 .. 2^8, or E4M3 2^-3 .. 2^2
    (mantissa 0).  With K = 32768 an NVFP4 row sum of element products needs 19 significant bits, so
    the scale product must add none for every fp32 partial sum to stay exact."""
    if fmt == "mxfp8":
        s = torch.randint(118, 136, (rows, 1), dtype=torch.uint8, device="cuda", generator=gen)
        return s.expand(rows, K // 32).contiguous()
    e = torch.randint(4, 10, (rows, 1), dtype=torch.uint8, device="cuda", generator=gen)
    return e.bitwise_left_shift_(3).expand(rows, K // 16).contiguous()


def _sample(n, tile):
    """Indices 0, n-1, both sides of tile boundaries near the start, middle and end, and a spread."""
    pts = {0, 1, n - 2, n - 1, n // 2}
    for b in (tile, (n // tile) * tile, (n // tile // 2) * tile):
        pts.update((b - 1, b))
    pts.update(np.linspace(0, n - 1, 17).astype(int).tolist())
    return np.array(sorted(p for p in pts if 0 <= p < n))


LIMIT_SHAPES = [
    ("mxfp8", (65535, 256, 32768), "mxfp8_pp"),              # A: 2^31 - 2^15 elements, ragged last M tile
    ("mxfp8", (256, 65520, 32768), "mxfp8_pp"),              # B: 2^31 - 2^19 elements
    ("mxfp8", (65536, 32752, 512), "mxfp8_pp"),              # D: 2^31 - 2^20 elements, ragged last N tile
    ("mxfp8", (65536, 32752, 96), "mxfp8_tiled_256x256"),    # D at the limit, one partial K tile
    ("nvfp4", (65535, 256, 32768), "nvfp4_256x256"),         # A at the limit (1 GiB packed)
    ("nvfp4", (128, 65520, 32768), "nvfp4_128x256_sharedA"),  # B at the limit
    ("nvfp4", (65536, 32752, 64), "nvfp4_256x256"),          # D at the limit
]


@pytest.mark.parametrize("fmt,shape,variant", LIMIT_SHAPES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_largest_sizes_bit_exact(fmt, shape, variant):
    M, N, K = shape
    assert M * K < 2 ** 31 and N * K < 2 ** 31 and M * N < 2 ** 31
    print(f"[limits] {fmt} {shape}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(M * 7 + N * 3 + K)
    A, B = _codes(fmt, M, K, gen), _codes(fmt, N, K, gen)
    sA, sB = _scales(fmt, M, K, gen), _scales(fmt, N, K, gen)
    D = torch.full((M, N), 0x7FFF, dtype=torch.int16, device="cuda")
    plan = bsg.Plan(fmt, M, N, K, out="bf16")
    info = plan.info()
    assert info["variant"].startswith(variant), info
    plan.run(A, B, sA, sB, D, alpha=0.5)
    torch.cuda.synchronize()
    assert not bool((D == 0x7FFF).any()), "entries never written"
    rows, cols = _sample(M, info["tile"][0]), _sample(N, info["tile"][1])
    r, c = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    sub = dict(fmt=fmt, M=len(rows), N=len(cols), K=K, alpha=np.float32(0.5), bias=None, silu=False, out="bf16",
               A=A[r].cpu().numpy(), B=B[c].cpu().numpy(), sA=sA[r].cpu().numpy(), sB=sB[c].cpu().numpy())
    got = D[r][:, c].cpu().numpy().view(np.uint16)
    want = reference(sub)["bits"]
    assert np.array_equal(got, want), f"{int((got != want).sum())} of {got.size} sampled entries differ"
    plan.close()
