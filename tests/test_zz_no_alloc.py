"""bsg_run_noalloc (no allocation; split-K partials in the library's static device scratch) against the
plan path (bsg_plan_create + bsg_run) through the C ABI: same kernels, same partial-sum order, so the
same bits; and against the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
import seeded_inputs as si
from gpu_util import make_plan, run, to_device
from oracle import compare, reference

pytestmark = pytest.mark.gpu


def _noalloc(p, dev):
    dev["D"].fill_(0x7FFF)
    bsg.run_noalloc(p["fmt"], p["M"], p["N"], p["K"], dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"],
                    alpha=float(p["alpha"]), bias=dev["bias"], out=p["out"], silu=p["silu"])
    torch.cuda.synchronize()
    return dev["D"].cpu().numpy().view(np.uint16).copy()


@pytest.mark.parametrize("fmt,shapes", [
    ("nvfp4", [(128, 4096, 4096), (96, 2048, 2048)]),
    ("mxfp8", [(128, 2048, 4096), (64, 1024, 2048)]),
], ids=["nvfp4", "mxfp8"])
def test_noalloc_matches_plan_path_twice_second_smaller(fmt, shapes):
    for i, (M, N, K) in enumerate(shapes):
        p = si.problem(fmt, M, N, K, seed=4100 + i, bias=True, silu=True, out="bf16", alpha=0.75)
        plan = make_plan(p)
        info = plan.info()
        assert 0 < info["workspace_bytes"] <= bsg.NOALLOC_SCRATCH_BYTES, info  # a split plan: uses the scratch
        dev = to_device(p)
        want = run(p, plan=plan, dev=dev)
        plan.close()
        got = _noalloc(p, dev)
        print(f"[noalloc] {fmt} {M}x{N}x{K} {info['variant']} workspace={info['workspace_bytes']}", flush=True)
        assert np.array_equal(got, want), f"{int((got != want).sum())} entries differ from the plan path"
        rep = compare(got, reference(p), p["alpha"], p["silu"], p["out"])
        assert rep["ok"], rep


def test_noalloc_unsplit_and_allocates_nothing():
    p = si.problem("mxfp8", 512, 512, 512, seed=4200, out="f16", alpha=0.5)
    plan = make_plan(p)
    assert plan.info()["workspace_bytes"] == 0
    dev = to_device(p)
    want = run(p, plan=plan, dev=dev)
    plan.close()
    assert np.array_equal(_noalloc(p, dev), want)
    q = si.problem("nvfp4", 128, 2048, 4096, seed=4201, out="bf16")
    dq = to_device(q)
    _noalloc(q, dq)  # a split problem: the scratch address is looked up by now
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(200):
        bsg.run_noalloc(q["fmt"], q["M"], q["N"], q["K"], dq["A"], dq["B"], dq["sA"], dq["sB"], dq["D"],
                        alpha=float(q["alpha"]), out=q["out"])
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_noalloc_refuses_a_workspace_above_the_scratch():
    # a split plan whose partials exceed the scratch is refused before anything is launched
    for M, N, K in ((256, 12288, 8192), (256, 14336, 8192), (256, 10240, 16384), (128, 16384, 16384)):
        with bsg.Plan("nvfp4", M, N, K, out="bf16") as plan:
            need = plan.info()["workspace_bytes"]
        if need > bsg.NOALLOC_SCRATCH_BYTES:
            break
    else:
        pytest.fail("no candidate shape needs more than the scratch")
    D = torch.full((M, N), 0x7FFF, dtype=torch.int16, device="cuda")
    A = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    B = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    sA = torch.zeros((M, K // 16), dtype=torch.uint8, device="cuda")
    sB = torch.zeros((N, K // 16), dtype=torch.uint8, device="cuda")
    with pytest.raises(bsg.BsgError) as e:
        bsg.run_noalloc("nvfp4", M, N, K, A, B, sA, sB, D)
    assert e.value.status_name == "BSG_ERR_UNSUPPORTED" and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((D == 0x7FFF).all())
