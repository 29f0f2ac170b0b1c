"""GPU checks of the K-tile-major scale layout (BSG_SCALES_KTILE): the device pack utility against the
layout's definition, and GEMMs reading packed scales against the same problems on row-major scales
(the same kernel and summation, so the same bits) and against the fp64 oracle, for every kernel
family, split-K and batched plans."""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
import seeded_inputs as si
from gpu_util import make_plan, run
from oracle import compare, reference

pytestmark = pytest.mark.gpu


def ktile_layout(s: np.ndarray) -> np.ndarray:
    """The layout written out from its definition: code 4g + c of row r at byte (g * rows + r) * 4 + c,
    codes past the row's last one (padding of the last group) 0."""
    rows, kb = s.shape
    out = np.zeros(-(-kb // 4) * rows * 4, dtype=np.uint8)
    r = np.arange(rows)
    for k in range(kb):
        g, c = divmod(k, 4)
        out[(g * rows + r) * 4 + c] = s[:, k]
    return out


@pytest.mark.parametrize("rows,kb", [(1, 1), (3, 6), (130, 33), (257, 128), (64, 2), (1000, 130)],
                         ids=lambda v: str(v))
def test_pack_scales_matches_definition(rows, kb):
    s = np.random.default_rng(rows * 1000 + kb).integers(0, 256, (rows, kb), dtype=np.uint8)
    n = bsg.scales_ktile_bytes(rows, kb)
    dst = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")  # padding must be overwritten with 0
    bsg.pack_scales(torch.from_numpy(s).cuda(), dst, rows, kb)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), ktile_layout(s))


def _ktile_problem(p):
    q = dict(p)
    q["sA"], q["sB"] = ktile_layout(p["sA"]), ktile_layout(p["sB"])
    return q


KTILE_SHAPES = [
    ("mxfp8", (4096, 4096, 512)),   # large-shape ping-pong kernel
    ("mxfp8", (4096, 4096, 384)),   # tiled 256 x 256
    ("mxfp8", (128, 2048, 4096)),   # tiled 128 x 128, split K
    ("mxfp8", (130, 528, 1056)),    # tiled, a partial last K tile; the last group of 4 codes is half padding
    ("mxfp8", (100, 80, 160)),      # tiled, ragged, 5 codes per row
    ("nvfp4", (100, 80, 1056)),     # 128 x 256 tiles (shared A), split, a final half K tile
    ("nvfp4", (128, 1024, 4096)),   # shared A, split
    ("nvfp4", (300, 2048, 1056)),   # 256 x 128 tiles (shared B), ragged M, half K tile
    ("nvfp4", (640, 4096, 256)),    # shared B, unsplit
    ("nvfp4", (200, 1040, 1280)),   # shared B, ragged M and N, split into whole 4-tile scale groups
    ("nvfp4", (96, 2048, 4864)),    # shared A, ragged M, split (19 scale groups over the splits)
    ("nvfp4", (4096, 4096, 288)),   # 256 x 256 tiles, a final half K tile
]


@pytest.mark.parametrize("fmt,shape", KTILE_SHAPES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_ktile_scales_match_row_major_and_oracle(fmt, shape):
    M, N, K = shape
    p = si.problem(fmt, M, N, K, seed=M + 3 * N + 7 * K, bias=True, silu=True, out="bf16", alpha=0.75)
    lin_plan = make_plan(p)
    kt_plan = bsg.Plan(fmt, M, N, K, out="bf16", bias=True, silu=True, scale_layout="ktile")
    li, ki = lin_plan.info(), kt_plan.info()
    assert (li["variant"], li["grid"]) == (ki["variant"], ki["grid"]), (li, ki)
    print(f"[plan] {fmt} {shape} {ki['variant']} grid={ki['grid']}", flush=True)
    D_lin = run(p, plan=lin_plan)
    D = run(_ktile_problem(p), plan=kt_plan)
    assert not (D == 0x7FFF).any()
    assert np.array_equal(D, D_lin), f"{int((D != D_lin).sum())} entries differ from the row-major-scale run"
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 24)), [M - 1]]))
    rep = compare(D[rows], reference(p, rows=rows), p["alpha"], p["silu"], p["out"])
    assert rep["ok"], rep
    lin_plan.close()
    kt_plan.close()


@pytest.mark.parametrize("fmt,shape", [("mxfp8", (130, 528, 1056)), ("mxfp8", (4096, 4096, 4128)),
                                       ("nvfp4", (100, 80, 1056)), ("nvfp4", (300, 2048, 1056))],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_ktile_padding_codes_are_ignored(fmt, shape):
    """Padding codes of the last group (K not a multiple of 4 blocks) are never used: NaN codes there
    (E8M0 0xFF, E4M3 0x7F) give the bits of the zero-padded layout."""
    M, N, K = shape
    p = si.problem(fmt, M, N, K, seed=K + M, out="bf16", alpha=0.5)
    q = _ktile_problem(p)
    kb = p["sA"].shape[1]
    assert kb % 4, "a shape whose last group has padding"
    nan = 0xFF if fmt == "mxfp8" else 0x7F
    poisoned = dict(q)
    for key, rows in (("sA", M), ("sB", N)):
        lay = q[key].copy().reshape(-1, rows, 4)
        lay[-1, :, kb % 4:] = nan
        poisoned[key] = lay.reshape(-1)
    plan = bsg.Plan(fmt, M, N, K, out="bf16", scale_layout="ktile")
    assert np.array_equal(run(poisoned, plan=plan), run(q, plan=plan))
    plan.close()


@pytest.mark.parametrize("fmt,shape", [("mxfp8", (1024, 1024, 512)), ("nvfp4", (128, 1024, 4096)),
                                       ("mxfp8", (96, 64, 288))], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_ktile_scales_batched(fmt, shape):
    """Batched plans read each problem's packed scales at its own stride (packed_strides)."""
    M, N, K = shape
    L = 16 if M == 1024 else 3
    problems = [si.problem(fmt, M, N, K, seed=40 + z, out="bf16", alpha=0.5) for z in range(L)]
    plan = bsg.Plan(fmt, M, N, K, out="bf16", batch=L, scale_layout="ktile")
    st = plan.strides
    assert st == bsg.packed_strides(fmt, M, N, K, "ktile")
    cat = lambda key, f=lambda a: a: torch.from_numpy(np.concatenate([np.ascontiguousarray(f(q[key])).reshape(-1)
                                                                      for q in problems])).cuda()
    A, B = cat("A"), cat("B")
    sA, sB = cat("sA", ktile_layout), cat("sB", ktile_layout)
    assert sA.numel() == L * st["sa"] and sB.numel() == L * st["sb"]
    D = torch.full((L * M * N,), 0x7FFF, dtype=torch.int16, device="cuda")
    plan.run(A, B, sA, sB, D, alpha=0.5)
    torch.cuda.synchronize()
    out = D.cpu().numpy().view(np.uint16).reshape(L, M, N)
    for z, q in enumerate(problems):
        single = run(q)  # row-major scales, single-problem plan
        if plan.info()["variant"] == make_plan(q).info()["variant"]:
            assert np.array_equal(out[z], single), f"problem {z}"
        rep = compare(out[z], reference(q), q["alpha"], q["silu"], q["out"])
        assert rep["ok"], (z, rep)
    plan.close()


@pytest.mark.parametrize("fmt,shape,L", [
    ("mxfp8", (128, 2048, 8224), 2),   # split K, three LDS stages, a partial last K tile
    ("mxfp8", (128, 1024, 4160), 2),   # split K, two stages (4 K tiles per split), partial last tile
    ("mxfp8", (128, 2048, 8192), 2),   # split K, three stages, whole K tiles
    ("mxfp8", (512, 512, 4224), 3),    # 128 x 128 tiles, split, K % 512 != 0
    ("nvfp4", (100, 1024, 4128), 2),   # NVFP4 split with a final half K tile
], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
@pytest.mark.parametrize("layout", ["linear", "ktile"])
def test_batched_split_tail_combinations(fmt, shape, L, layout):
    """Batched split plans across the kernels' K-range paths, on either scale layout: every problem's
    D passes the oracle, and each equals a single-problem plan of the same kernel."""
    M, N, K = shape
    problems = [si.problem(fmt, M, N, K, seed=300 + 7 * z + K % 97, bias=True, silu=True, out="f16", alpha=0.5)
                for z in range(L)]
    plan = bsg.Plan(fmt, M, N, K, out="f16", bias=True, silu=True, batch=L, scale_layout=layout)
    info = plan.info()
    assert info["workspace_bytes"] > 0, info  # a split plan
    st = plan.strides
    pack = ktile_layout if layout == "ktile" else (lambda a: a)
    cat = lambda key, f=lambda a: a: torch.from_numpy(np.concatenate([np.ascontiguousarray(f(q[key])).reshape(-1)
                                                                      for q in problems])).cuda()
    A, B, sA, sB = cat("A"), cat("B"), cat("sA", pack), cat("sB", pack)
    bias = torch.from_numpy(problems[0]["bias"].astype(np.float32)).cuda()  # stride 0: shared bias
    for q in problems:
        q["bias"] = problems[0]["bias"]
    assert sA.numel() == L * st["sa"] and sB.numel() == L * st["sb"]
    D = torch.full((L * M * N,), 0x7FFF, dtype=torch.int16, device="cuda")
    plan.run(A, B, sA, sB, D, alpha=0.5, bias=bias)
    torch.cuda.synchronize()
    out = D.cpu().numpy().view(np.uint16).reshape(L, M, N)
    single = bsg.Plan(fmt, M, N, K, out="f16", bias=True, silu=True, scale_layout=layout)
    same_kernel = single.info()["variant"] == info["variant"] and single.info()["grid"][:2] == info["grid"][:2]
    for z, q in enumerate(problems):
        rep = compare(out[z], reference(q), q["alpha"], q["silu"], q["out"])
        assert rep["ok"], (z, rep)
        if same_kernel:
            qq = dict(q)
            qq["sA"], qq["sB"] = pack(q["sA"]), pack(q["sB"])
            assert np.array_equal(out[z], run(qq, plan=single)), f"problem {z}"
    plan.close()
    single.close()
