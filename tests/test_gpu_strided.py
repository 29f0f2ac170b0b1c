"""GPU parity with leading dimensions (row pitches of A, B and D larger than packed).

The gaps of A and B hold codes that would change the result if read (E4M3 NaN 0x7F for MXFP8; E2M1
pairs of -6 for NVFP4), D is poisoned and its gap columns must stay untouched, and the result must
equal the packed problem's bits whenever the same kernel serves both (the same tile and split
choice: they depend on the shape only), and pass the fp64 oracle in every case."""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
import seeded_inputs as si
from gpu_util import make_plan, run
from oracle import compare, reference

pytestmark = pytest.mark.gpu


def _pitched(x: np.ndarray, pitch_bytes: int, fill: int) -> np.ndarray:
    """Rows of x (uint8) at `pitch_bytes` apart, the gap bytes set to `fill`."""
    out = np.full((x.shape[0], pitch_bytes), fill, dtype=np.uint8)
    out[:, :x.shape[1]] = x
    return out


STRIDED = [
    # fmt, (M, N, K), (lda, ldb, ldd), variant expected
    ("mxfp8", (128, 2048, 4096), (4160, 4224, 2056), "mxfp8_tiled_128x128"),  # split K, three stages
    ("mxfp8", (130, 528, 1056), (1072, 1088, 536), "mxfp8_tiled_128x128"),    # partial last K tile
    ("mxfp8", (96, 64, 288), (304, 320, 72), "mxfp8_tiled_128x128"),          # ragged, 9 K blocks
    ("mxfp8", (4096, 4096, 512), (528, 512, 4104), "mxfp8_tiled_256x256"),    # strided A: not ping-pong
    ("mxfp8", (4096, 4096, 512), (0, 0, 4104), "mxfp8_pp"),                   # ping-pong with a D pitch
    ("nvfp4", (100, 80, 1056), (1088, 1120, 88), "nvfp4_128x256_sharedA"),    # split, final half K tile
    ("nvfp4", (300, 2048, 1056), (1088, 1152, 2056), "nvfp4_256x128_sharedB"),
    ("nvfp4", (4096, 4096, 288), (320, 352, 4112), "nvfp4_256x256_sharedB"),
]


@pytest.mark.parametrize("fmt,shape,lds,variant", STRIDED,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_leading_dimensions(fmt, shape, lds, variant):
    M, N, K = shape
    lda, ldb, ldd = (x or d for x, d in zip(lds, (K, K, N)))
    print(f"[strided] {fmt} {shape} lda={lda} ldb={ldb} ldd={ldd}", flush=True)
    p = si.problem(fmt, M, N, K, seed=M + 5 * N + 11 * K + lda, bias=True, silu=True, out="bf16", alpha=0.5)
    epb = 1 if fmt == "mxfp8" else 2  # elements per byte
    fill = 0x7F if fmt == "mxfp8" else 0xFF
    plan = bsg.Plan(fmt, M, N, K, out="bf16", bias=True, silu=True, lda=lds[0], ldb=lds[1], ldd=lds[2])
    info = plan.info()
    assert info["variant"].startswith(variant), info
    A = torch.from_numpy(_pitched(p["A"], lda // epb, fill)).cuda()
    B = torch.from_numpy(_pitched(p["B"], ldb // epb, fill)).cuda()
    sA, sB = torch.from_numpy(p["sA"]).cuda(), torch.from_numpy(p["sB"]).cuda()
    bias = torch.from_numpy(p["bias"].astype(np.float32)).cuda()
    D = torch.full((M, ldd), 0x7FFF, dtype=torch.int16, device="cuda")
    plan.run(A, B, sA, sB, D, alpha=0.5, bias=bias)
    torch.cuda.synchronize()
    Dh = D.cpu().numpy().view(np.uint16)
    assert (Dh[:, N:] == 0x7FFF).all(), "a store landed in D's row gap"
    got = np.ascontiguousarray(Dh[:, :N])
    assert not (got == 0x7FFF).any(), "entries never written"
    packed = make_plan(p)
    if packed.info()["variant"] == info["variant"]:
        assert np.array_equal(got, run(p, plan=packed)), "differs from the packed problem's bits"
    packed.close()
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 24)), [M - 1]]))
    rep = compare(got[rows], reference(p, rows=rows), p["alpha"], p["silu"], p["out"])
    assert rep["ok"], rep
    plan.close()


def test_leading_dimensions_batched():
    """Batched problems with row pitches: each problem's A, B and D at rows x pitch, back to back."""
    fmt, (M, N, K), L = "mxfp8", (96, 64, 288), 3
    lda, ldb, ldd = 320, 304, 80
    problems = [si.problem(fmt, M, N, K, seed=500 + z, out="f16", alpha=0.75) for z in range(L)]
    plan = bsg.Plan(fmt, M, N, K, out="f16", batch=L, lda=lda, ldb=ldb, ldd=ldd)
    st = plan.strides
    assert st["a"] == M * lda and st["b"] == N * ldb and st["d"] == 2 * M * ldd
    A = torch.from_numpy(np.concatenate([_pitched(q["A"], lda, 0x7F) for q in problems])).cuda()
    B = torch.from_numpy(np.concatenate([_pitched(q["B"], ldb, 0x7F) for q in problems])).cuda()
    sA = torch.from_numpy(np.concatenate([q["sA"] for q in problems])).cuda()
    sB = torch.from_numpy(np.concatenate([q["sB"] for q in problems])).cuda()
    D = torch.full((L, M, ldd), 0x7FFF, dtype=torch.int16, device="cuda")
    plan.run(A, B, sA, sB, D, alpha=0.75)
    torch.cuda.synchronize()
    Dh = D.cpu().numpy().view(np.uint16)
    assert (Dh[:, :, N:] == 0x7FFF).all()
    for z, q in enumerate(problems):
        got = np.ascontiguousarray(Dh[z, :, :N])
        assert np.array_equal(got, run(q)), f"problem {z}"
        rep = compare(got, reference(q), q["alpha"], q["silu"], q["out"])
        assert rep["ok"], (z, rep)
    plan.close()
