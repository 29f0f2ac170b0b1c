"""GPU parity of the block-scaled GEMM against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
import seeded_inputs as si
from gpu_util import exact_regime_problem as _exact_regime_problem
from gpu_util import make_plan, run, to_device
from oracle import compare, reference

pytestmark = pytest.mark.gpu

# the four shapes of the nvFuser page's test_mxfp8_gemm, plus ragged / multi-tile shapes
PAGE_SHAPES = [(128, 128, 128), (128, 128, 256), (256, 128, 128), (128, 256, 256)]
RAGGED_SHAPES = [(1, 16, 32), (33, 48, 96), (100, 80, 160), (257, 272, 320), (130, 528, 1024)]


def _check(p, rows=None, rel=1e-2):
    D = run(p)
    ref = reference(p, rows=rows)
    if rows is not None:
        D = D[rows]
    rep = compare(D, ref, p["alpha"], p["silu"], p["out"], rel=rel)
    print(f"[parity] {p['fmt']} {p['M']}x{p['N']}x{p['K']} {p['out']} resolvable={rep['n_resolvable']}/{rep['n']} "
          f"max_rel(resolvable)={rep['max_rel_err']:.3g} max_err/S={rep['max_err_over_S']:.3g} "
          f"by_floor={rep['n_passed_by_floor']}", flush=True)
    assert rep["ok"], rep
    return rep


def _check_workload(p, rows=None, min_resolvable=0.1):
    """A benchmark workload: the comparison rule, and the 1e-2 relative bar on the resolvable entries
    (sums that keep >= 2^-6 of their absolute mass, well-conditioned epilogue) asserted on their own."""
    rep = _check(p, rows=rows)
    assert rep["n_resolvable"] >= min_resolvable * rep["n"], rep
    assert rep["max_rel_err"] <= 1e-2, rep
    return rep


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(160, 96, 1024), (33, 272, 96), (256, 256, 2048), (384, 256, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_exact_regime_bit_exact(fmt, out, shape):
    p = _exact_regime_problem(fmt, *shape, seed=sum(shape), out=out)
    D = run(p)
    R = reference(p)["bits"]
    assert np.array_equal(D, R), f"{int((D != R).sum())} of {D.size} entries differ"


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("shape", PAGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_page_shapes(fmt, out, shape):
    M, N, K = shape
    _check(si.problem(fmt, M, N, K, seed=100 + M + N + K, out=out))


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("shape", RAGGED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ragged_shapes(fmt, shape):
    M, N, K = shape
    _check(si.problem(fmt, M, N, K, seed=200 + M, out="bf16", alpha=0.75))


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
@pytest.mark.parametrize("bias,silu", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_epilogue_variants(fmt, bias, silu, out):
    _check(si.problem(fmt, 192, 160, 256, seed=300, bias=bias, silu=silu, out=out, alpha=0.5))


def _band_rows(M, extra=()):
    """Two rows in every 256-row band (one per 128-row half, at varying offsets) plus `extra`."""
    rows = [r for b in range(0, M, 256) for r in (b + (37 * b // 256) % 128, b + 128 + (53 * b // 256) % 128)]
    return np.unique(np.array([r for r in rows if r < M] + list(extra)))


def _is_large_kernel(info):
    """The large-shape MXFP8 kernel (K % 512 == 0, 256 x 256 tiles)."""
    return info["variant"].startswith("mxfp8_pp") and info["tile"][:2] == (256, 256)


def _full_coverage(D):
    """Every entry was written (the poison fill is a NaN pattern that finite inputs cannot produce)."""
    assert not (D == 0x7FFF).any(), f"{int((D == 0x7FFF).sum())} entries of D were never written"


# Large-shape MXFP8 kernel (>= 256 tiles of 256 x 256, K % 512 == 0): bit-exact in the exact regime,
# including the banded tile order (M a multiple of 2048, N of 8192), and a ragged shape.
@pytest.mark.parametrize("shape", [(4096, 4096, 512), (2048, 8192, 1024)], ids=lambda s: "x".join(map(str, s)))
def test_large_mxfp8_exact_regime_bit_exact(shape):
    M, N, K = shape
    p = _exact_regime_problem("mxfp8", M, N, K, seed=M + K, out="bf16")
    plan = make_plan(p)
    assert _is_large_kernel(plan.info()), plan.info()
    D = run(p, plan=plan)
    _full_coverage(D)
    rows = _band_rows(M, extra=(M - 1,))
    R = reference(p, rows=rows)["bits"]
    assert np.array_equal(D[rows], R), f"{int((D[rows] != R).sum())} of {R.size} sampled entries differ"


@pytest.mark.parametrize("shape,epi", [((4000, 4112, 1024), dict(out="bf16", alpha=0.5)),
                                       ((2048, 8192, 512), dict(out="f16", bias=True, silu=True, alpha=0.25))],
                         ids=["ragged", "band_bias_silu"])
def test_large_mxfp8_sampled(shape, epi):
    M, N, K = shape
    p = si.problem("mxfp8", M, N, K, seed=K + 11, **epi)
    plan = make_plan(p)
    assert _is_large_kernel(plan.info()), plan.info()
    D = run(p, plan=plan)
    _full_coverage(D)
    rows = _band_rows(M, extra=(M - 2, M - 1))
    ref = reference(p, rows=rows)
    rep = compare(D[rows], ref, p["alpha"], p["silu"], p["out"])
    print(f"[parity] mxfp8 {M}x{N}x{K} sampled {len(rows)} rows max_rel={rep['max_rel_err']:.3g}", flush=True)
    assert rep["ok"], rep


def test_config_mxfp8_256():
    _check_workload(si.workload("mxfp8_256"))


def test_config_mxfp8_4096_sampled_rows():
    p = si.workload("mxfp8_4096")
    rows = np.unique(np.concatenate([np.arange(0, 4096, 97), [4095]]))
    _check_workload(p, rows=rows)


def test_config_mxfp8_8192_silu_sampled_rows():
    p = si.workload("mxfp8_8192_silu")
    rows = np.unique(np.concatenate([np.arange(0, 8192, 331), [8191]]))
    _check_workload(p, rows=rows)


def test_config_nvfp4_128x8192x8192_full():
    _check_workload(si.workload("nvfp4_128x8192x8192_silu"))


def test_config_nvfp4_256x4096x4096_all_sets():
    plan = None
    for s in range(10):
        p = si.workload("nvfp4_256x4096x4096_loop", set_id=s)
        plan = plan or make_plan(p)
        D = run(p, plan=plan)
        rep = compare(D, reference(p), p["alpha"], p["silu"], p["out"])
        print(f"[parity] nvfp4 256x4096x4096 set {s}: resolvable={rep['n_resolvable']}/{rep['n']} "
              f"max_rel(resolvable)={rep['max_rel_err']:.3g}", flush=True)
        assert rep["ok"] and rep["n_resolvable"] >= 0.1 * rep["n"], (s, rep)


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_power_of_two_scale_bump_is_exact(fmt):
    # raising every scale of A by 2^k multiplies each product, hence each fp32 partial sum, by 2^k
    # exactly; so D's bits shift by k in the exponent field (no bias, no SiLU, values in range)
    p = si.problem(fmt, 96, 64, 256, seed=400, out="bf16")
    if fmt == "nvfp4":  # normal E4M3 scales with exponent fields 4..11, so +1 stays normal
        g = np.random.default_rng(7)
        p["sA"] = (g.integers(4, 12, size=p["sA"].shape) << 3 | g.integers(0, 8, size=p["sA"].shape)).astype(np.uint8)
    D0 = run(p)
    q = dict(p)
    k = 3 if fmt == "mxfp8" else 1
    q["sA"] = (p["sA"].astype(np.int64) + (3 if fmt == "mxfp8" else 8)).astype(np.uint8)
    D1 = run(q)
    nz = (D0 & 0x7FFF) != 0
    assert np.array_equal(D1[nz].astype(np.int64) - D0[nz], np.full(int(nz.sum()), k << 7))
    assert np.array_equal(D1[~nz], D0[~nz])


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_permuting_b_rows_permutes_d_columns(fmt):
    p = si.problem(fmt, 64, 128, 256, seed=500, out="f16", bias=True, silu=True)
    D0 = run(p)
    perm = np.random.default_rng(1).permutation(128)
    q = dict(p, B=p["B"][perm], sB=p["sB"][perm], bias=p["bias"][perm])
    D1 = run(q)
    assert np.array_equal(D1, D0[:, perm])


def test_deterministic_and_alpha_ptr_matches():
    p = si.problem("mxfp8", 300, 256, 512, seed=600, bias=True, out="bf16", alpha=0.37)
    plan = make_plan(p)
    dev = to_device(p)
    D0 = run(p, plan=plan, dev=dev)
    D1 = run(p, plan=plan, dev=dev)
    assert np.array_equal(D0, D1)
    alpha_dev = torch.tensor([float(p["alpha"])], dtype=torch.float32, device="cuda")
    dev["D"].zero_()
    plan.run_alpha_ptr(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], alpha_dev, bias=dev["bias"])
    torch.cuda.synchronize()
    assert np.array_equal(dev["D"].cpu().numpy().view(np.uint16), D0)


@pytest.mark.parametrize("fmt,shape,prefix", [
    ("mxfp8", (4096, 4096, 512), "mxfp8_pp"), ("mxfp8", (128, 4096, 8192), "mxfp8_tiled_128"),
    ("nvfp4", (128, 2048, 4096), "nvfp4_128x256"), ("nvfp4", (4096, 4096, 256), "nvfp4_256x256")],
    ids=["mxfp8_pp", "mxfp8_tiled_split", "nvfp4_split", "nvfp4_256x256"])
def test_every_kernel_family_is_deterministic(fmt, shape, prefix):
    # the same inputs twice give bit-identical D: no race between LDS stages or split partials
    p = si.problem(fmt, *shape, seed=610, bias=True, silu=True, out="bf16")
    plan = make_plan(p)
    assert plan.info()["variant"].startswith(prefix), plan.info()
    dev = to_device(p)
    D0 = run(p, plan=plan, dev=dev)
    D1 = run(p, plan=plan, dev=dev)
    assert np.array_equal(D0, D1)
    plan.close()


def test_e8m0_extreme_scales():
    # one nonzero product per entry: A[i, 0] = B[j, 0] = 1.0; sA[i, 0] sweeps every E8M0 code 0..255
    # (0 = 2^-127, 255 = NaN) against sB in {2^-1, 2^0, 2^1}, so products span 2^-128 .. 2^128 (fp32
    # subnormals and overflow to inf included) and a NaN scale code reaches the MFMA
    M, N, K = 256, 48, 32
    A = np.zeros((M, K), np.uint8)
    A[:, 0] = 0x38
    B = np.zeros((N, K), np.uint8)
    B[:, 0] = 0x38
    sA = np.arange(0, 256, dtype=np.uint8)[:, None]
    sB = (126 + np.arange(N) % 3).astype(np.uint8)[:, None]
    p = dict(fmt="mxfp8", M=M, N=N, K=K, A=A, B=B, sA=sA, sB=sB, alpha=np.float32(1), bias=None, silu=False,
             out="bf16")
    D = run(p)
    R = reference(p)["bits"]
    nan_d, nan_r = (D & 0x7FFF) > 0x7F80, (R & 0x7FFF) > 0x7F80
    assert nan_r[255].all() and not nan_r[:255].any()
    assert np.array_equal(nan_d, nan_r), f"NaN pattern differs: rows {np.unique(np.argwhere(nan_d != nan_r)[:, 0])}"
    diff = (D != R) & ~nan_r
    assert not diff.any(), [(int(i), int(j), hex(D[i, j]), hex(R[i, j])) for i, j in np.argwhere(diff)[:8]]


def test_bias_four_byte_offset_on_large_mxfp8_kernel():
    # the ABI promises only 4-byte bias alignment: a bias at a 4-byte offset gives the same bits as an
    # aligned copy, on the large-shape kernel (whose epilogue reads 4 consecutive bias values per lane)
    p = si.problem("mxfp8", 4096, 4096, 512, seed=31, bias=True, silu=True, out="f16", alpha=0.5)
    plan = make_plan(p)
    assert _is_large_kernel(plan.info()), plan.info()
    dev = to_device(p)
    D0 = run(p, plan=plan, dev=dev)
    shifted = torch.zeros(p["N"] + 4, dtype=torch.float32, device="cuda")
    shifted[1:p["N"] + 1] = dev["bias"]
    dev["D"].fill_(0x7FFF)
    plan.run(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], alpha=float(p["alpha"]),
             bias=shifted.data_ptr() + 4)
    torch.cuda.synchronize()
    D1 = dev["D"].cpu().numpy().view(np.uint16)
    assert np.array_equal(D0, D1)
    rows = _band_rows(4096)
    assert compare(D1[rows], reference(p, rows=rows), p["alpha"], True, "f16")["ok"]
    with pytest.raises(bsg.BsgError) as e:
        plan.run(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], alpha=1.0, bias=shifted.data_ptr() + 2)
    assert e.value.status_name == "BSG_ERR_ALIGN"


def test_errors_reported_without_launch():
    p = si.problem("mxfp8", 64, 64, 64, seed=700)
    plan = make_plan(p)
    dev = to_device(p)
    with pytest.raises(bsg.BsgError) as e:
        plan.run(dev["A"].data_ptr() + 1, dev["B"], dev["sA"], dev["sB"], dev["D"])
    assert e.value.status_name == "BSG_ERR_ALIGN"
    with pytest.raises(bsg.BsgError) as e:
        plan.run(0, dev["B"], dev["sA"], dev["sB"], dev["D"])
    assert e.value.status_name == "BSG_ERR_NULL"
    pb = bsg.Plan("mxfp8", 64, 64, 64, bias=True)
    with pytest.raises(bsg.BsgError) as e:
        pb.run(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], bias=None)
    assert e.value.status_name == "BSG_ERR_NULL"


def test_no_device_allocation_per_call():
    p = si.workload("nvfp4_256x4096x4096_loop")
    plan = make_plan(p)
    dev = to_device(p)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(1000):
        plan.run(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], alpha=float(p["alpha"]))
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_plan_info():
    plan = bsg.Plan("mxfp8", 4096, 4096, 4096, out="bf16")
    info = plan.info()
    assert info["workspace_bytes"] == 0 and info["block"] > 0 and info["variant"].startswith("mxfp8")


def test_persistent_launch_shape():
    # the ping-pong kernel loops over tiles: at most one workgroup per CU (a multiple of 8, so each
    # keeps its XCD); the tiled kernels keep one workgroup per tile
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = bsg.Plan("mxfp8", 8192, 8192, 8192, out="f16", bias=True, silu=True)
    info = plan.info()
    assert info["variant"].startswith("mxfp8_pp")
    assert info["grid"][0] == (min(1024, cus) if cus % 8 == 0 else 1024), (info, cus)
    small = bsg.Plan("mxfp8", 1024, 1024, 512)  # a tiled plan: one workgroup per tile
    si_ = small.info()
    assert not si_["variant"].startswith("mxfp8_pp") and si_["grid"][0] == (1024 // si_["tile"][0]) * (1024 // si_["tile"][1])
    plan.close()
    small.close()


def test_log_levels_and_forced_architecture(monkeypatch, capfd):
    p = si.problem("nvfp4", 128, 1024, 4096, seed=701)
    dev = to_device(p)
    capfd.readouterr()
    monkeypatch.setenv("BSG_LOG", "2")
    plan = make_plan(p)  # BSG_LOG is read at plan creation
    info = plan.info()
    plan.run(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], alpha=float(p["alpha"]))
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert f"-> {info['variant']} " in err and f"splits {info['grid'][0] // 4}" in err, err
    assert f"bsg: run {info['variant']} " in err, err
    monkeypatch.setenv("BSG_LOG", "0")
    quiet = make_plan(p)
    quiet.run(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], alpha=float(p["alpha"]))
    torch.cuda.synchronize()
    assert "bsg:" not in capfd.readouterr().err
    monkeypatch.setenv("BSG_FORCE_ARCH", "gfx942")
    with pytest.raises(bsg.BsgError) as e:
        make_plan(p)
    assert e.value.status_name == "BSG_ERR_DEVICE" and "BSG_FORCE_ARCH=gfx942" in str(e.value)
    monkeypatch.setenv("BSG_FORCE_ARCH", "gfx950")  # the real device is checked, and it is gfx950
    make_plan(p).close()
    plan.close()
    quiet.close()


# NVFP4 small-M problems split K across workgroups (fp32 partials in the plan's workspace, summed in
# split order by a second kernel); these shapes cover split and unsplit plans, ragged M / N, a final
# half K tile (K % 64 == 32), and, with K % 256 == 0 (the warp-specialised kernel: splits take whole
# 4-tile scale groups), one group in all (K = 256), one group per split (K = 768, 1280) and groups
# that do not divide evenly over the splits (K = 1792: 7 groups, K = 4864: 19).
NVFP4_SPLIT_SHAPES = [(100, 80, 1056), (1, 16, 4128), (129, 4000, 2080), (256, 1024, 2048), (640, 4096, 256),
                      (512, 1024, 4096), (300, 2048, 1056), (128, 2048, 1792), (64, 1024, 768), (200, 512, 1280),
                      (96, 2048, 4864)]


@pytest.mark.parametrize("shape", NVFP4_SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("epi", ["plain", "bias_silu"])
def test_nvfp4_split_k(shape, epi):
    M, N, K = shape
    p = si.problem("nvfp4", M, N, K, seed=900 + M + N + K, bias=epi != "plain", silu=epi != "plain", out="bf16",
                   alpha=0.75)
    plan = make_plan(p)
    info = plan.info()
    tiles = -(-M // info["tile"][0]) * -(-N // info["tile"][1])
    splits = info["grid"][0] // tiles
    assert info["grid"][0] == tiles * splits
    assert info["workspace_bytes"] == (0 if splits == 1 else splits * M * N * 4)
    print(f"[plan] {shape} {info['variant']} splits={splits}", flush=True)
    D = run(p, plan=plan)
    rep = compare(D, reference(p), p["alpha"], p["silu"], p["out"])
    assert rep["ok"], rep


def _graph_replay_matches_eager(plan, problems):
    """Replayed HIP graphs (every kernel of a call captured) give the eager bits, for each input set."""
    devs, eager = [], []
    for q in problems:
        d = to_device(q)
        eager.append(run(q, plan=plan, dev=d))
        devs.append(d)
    sets = []
    for d, q in zip(devs, problems):
        d["D"].fill_(0x7FFF)
        sets.append(dict(A=d["A"], B=d["B"], sA=d["sA"], sB=d["sB"], D=d["D"], alpha=float(q["alpha"]),
                         bias=d["bias"]))
    stream = torch.cuda.Stream()
    bsg.bench_loop(plan, sets, 3, 1, stream)
    torch.cuda.synchronize()
    for d, want in zip(devs, eager):
        assert np.array_equal(d["D"].cpu().numpy().view(np.uint16), want)


# MXFP8 problems with too few 256 x 256 tiles to fill the chip run 128 x 128 tiles and, when those are
# still fewer than the CUs, split K the same way; shapes cover split and unsplit plans, ragged M / N,
# a split count that does not divide the K tiles, and K not a multiple of 512.
MXFP8_SPLIT_SHAPES = [(100, 80, 1024), (1, 16, 4096), (129, 4000, 2048), (256, 1024, 1152), (640, 4096, 384),
                      (512, 1024, 4096), (1024, 1024, 1024), (33, 2000, 1408), (33, 2000, 2816)]


@pytest.mark.parametrize("shape", MXFP8_SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("epi", ["plain", "bias_silu_f16"])
def test_mxfp8_split_k(shape, epi):
    M, N, K = shape
    plain = epi == "plain"
    p = si.problem("mxfp8", M, N, K, seed=700 + M + N + K, bias=not plain, silu=not plain,
                   out="bf16" if plain else "f16", alpha=0.75)
    plan = make_plan(p)
    info = plan.info()
    tiles = -(-M // info["tile"][0]) * -(-N // info["tile"][1])
    splits = info["grid"][0] // tiles
    assert info["grid"][0] == tiles * splits
    assert info["workspace_bytes"] == (0 if splits == 1 else splits * M * N * 4)
    print(f"[plan] {shape} {info['variant']} splits={splits}", flush=True)
    D = run(p, plan=plan)
    rep = compare(D, reference(p), p["alpha"], p["silu"], p["out"])
    assert rep["ok"], rep


# MXFP8 K % 128 != 0 (K % 32 == 0): the tiled kernels' last K tile is partial -- its chunks past K
# read as zeros and its missing 32-blocks take scale code 127, so they add exact zeros.  Large
# (256 x 256) and small (128 x 128) tiles, split and unsplit, a single partial tile (K = 32).
MXFP8_KTAIL_SHAPES = [(4096, 4096, 4128), (128, 2048, 4192), (300, 528, 1120), (64, 64, 32), (257, 272, 96),
                      (1, 16, 4160)]


@pytest.mark.parametrize("shape", MXFP8_KTAIL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mxfp8_k_tail(shape):
    M, N, K = shape
    p = si.problem("mxfp8", M, N, K, seed=500 + K % 128 + M, bias=True, silu=True, out="f16", alpha=0.5)
    plan = make_plan(p)
    info = plan.info()
    assert info["variant"].startswith("mxfp8_tiled"), info
    print(f"[plan] {shape} {info['variant']} grid={info['grid']}", flush=True)
    D = run(p, plan=plan)
    _full_coverage(D)
    rows = _band_rows(M, extra=(M - 1,)) if M >= 2048 else np.arange(M)
    rep = compare(D[rows], reference(p, rows=rows), p["alpha"], p["silu"], p["out"])
    assert rep["ok"], rep


@pytest.mark.parametrize("shape", [(256, 512, 4128), (128, 1024, 2080)], ids=lambda s: "x".join(map(str, s)))
def test_mxfp8_k_tail_exact_regime_bit_exact(shape):
    M, N, K = shape
    p = _exact_regime_problem("mxfp8", M, N, K, seed=K, out="bf16")
    D = run(p)
    assert np.array_equal(D, reference(p)["bits"])


def test_mxfp8_split_k_plans():
    # 64 tiles of 128 x 128: four K splits fill the 256 CUs
    info = bsg.Plan("mxfp8", 128, 8192, 8192, out="bf16").info()
    assert info["variant"].startswith("mxfp8_tiled_128x128")
    assert info["grid"][0] == 64 * 4 and info["workspace_bytes"] == 4 * 128 * 8192 * 4
    # at most one split per 4 K tiles of 128
    info = bsg.Plan("mxfp8", 256, 256, 768, out="bf16").info()
    assert info["variant"].startswith("mxfp8_tiled_128x128")
    assert info["grid"][0] == 4 and info["workspace_bytes"] == 0
    # 64 tiles of 8 K tiles: a split would save 4 K tiles per workgroup but cost the finish pass and
    # 8 MiB of partials (measured 11.8 vs 8.2 us unsplit), so the cost model keeps it whole
    info = bsg.Plan("mxfp8", 1024, 1024, 1024, out="bf16").info()
    assert info["grid"][0] == 64 and info["workspace_bytes"] == 0
    # 32 tiles of 32 K tiles: split (23.8 us unsplit, 14.9-15.1 us at four to eight splits)
    info = bsg.Plan("mxfp8", 512, 1024, 4096, out="bf16").info()
    splits = info["grid"][0] // 32
    assert 4 <= splits <= 8 and info["workspace_bytes"] == splits * 512 * 1024 * 4, info
    # 256x4096x2048: 64 tiles of 16 K tiles stay whole (13.1 us; 15.3 us at two splits)
    info = bsg.Plan("mxfp8", 256, 4096, 2048, out="bf16").info()
    assert info["grid"][0] == 64 and info["workspace_bytes"] == 0
    # short K: 128 x 128 tiles while 256 x 256 ones would not fill the CUs
    for shape in ((256, 256, 256), (1024, 1024, 512), (64, 4096, 96)):
        assert bsg.Plan("mxfp8", *shape, out="bf16").info()["variant"].startswith("mxfp8_tiled_128x128"), shape


def test_mxfp8_split_k_exact_regime_bit_exact_and_graph():
    """In the exact regime every partial sum is exact in fp32, so any split gives the oracle's bits."""
    p = _exact_regime_problem("mxfp8", 128, 2048, 4096, seed=77, out="bf16")
    plan = make_plan(p)
    info = plan.info()
    assert info["grid"][0] // 16 > 1, info
    D = run(p, plan=plan)
    assert np.array_equal(D, reference(p)["bits"])
    q = si.problem("mxfp8", 128, 2048, 4096, seed=78, out="bf16", alpha=0.5)
    _graph_replay_matches_eager(plan, [p, q])


def test_nvfp4_split_k_deterministic_alpha_ptr_and_graph():
    p = si.problem("nvfp4", 256, 1024, 4096, seed=1234, bias=True, silu=True, out="bf16", alpha=0.3)
    plan = make_plan(p)
    assert plan.info()["workspace_bytes"] > 0
    dev = to_device(p)
    D0 = run(p, plan=plan, dev=dev)
    D1 = run(p, plan=plan, dev=dev)
    assert np.array_equal(D0, D1)
    alpha_dev = torch.tensor([float(p["alpha"])], dtype=torch.float32, device="cuda")
    dev["D"].fill_(0x7FFF)
    plan.run_alpha_ptr(dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"], alpha_dev, bias=dev["bias"])
    torch.cuda.synchronize()
    assert np.array_equal(dev["D"].cpu().numpy().view(np.uint16), D0)
    q = si.problem("nvfp4", 256, 1024, 4096, seed=4321, bias=True, silu=True, out="bf16", alpha=0.3)
    _graph_replay_matches_eager(plan, [p, q])


def test_nvfp4_loop_workload_graph_replay():
    p = si.workload("nvfp4_256x4096x4096_loop")
    plan = make_plan(p)
    _graph_replay_matches_eager(plan, [p, si.workload("nvfp4_256x4096x4096_loop", set_id=1)])


def test_nvfp4_plan_info():
    # M <= 128: 128 x 256 tiles sharing the decoded A tile; the 32 tiles of 128 x 8192 split K
    info = bsg.Plan("nvfp4", 128, 8192, 8192, out="bf16", bias=True, silu=True).info()
    assert info["variant"].startswith("nvfp4_128x256_sharedA")
    splits = info["grid"][0] // (8192 // info["tile"][1])
    assert splits > 1 and info["workspace_bytes"] == splits * 128 * 8192 * 4
    # the looped 256x4096x4096 problem: 32 tiles of 64 K tiles; the cost model stops short of filling
    # every CU (8 splits) because each further split adds 4 MiB of partials for one K tile less
    info = bsg.Plan("nvfp4", 256, 4096, 4096, out="bf16").info()
    splits = info["grid"][0] // 32
    assert info["variant"].startswith("nvfp4_256x128_sharedB") and 4 <= splits < 8, info
    assert info["workspace_bytes"] == splits * 256 * 4096 * 4
    # larger M shares the decoded B tile: 256 x 128 tiles, split when too few ...
    info = bsg.Plan("nvfp4", 1024, 4096, 4096, out="f16").info()
    assert info["variant"].startswith("nvfp4_256x128") and info["workspace_bytes"] > 0
    # ... and 256 x 256 tiles, unsplit, once those alone give every CU a workgroup
    info = bsg.Plan("nvfp4", 4096, 4096, 4096, out="f16").info()
    assert info["variant"].startswith("nvfp4_256x256") and info["workspace_bytes"] == 0
    assert info["grid"][0] == 256


# Split plans whose fp32 partials come to at least one L2 (4 MiB) per XCD store them with
# device-scope stores, which write through the L2; smaller partial sets use streaming stores.  Both
# forms against the oracle: the single-tile kernel (K % 256 != 0) and the shared-B warp-specialised
# kernel with partials stored through, the looped 256x4096x4096 shape (24 MiB) streamed.  The
# plan's choice is read from its BSG_LOG line.
@pytest.mark.parametrize("shape,through", [((128, 8192, 8224), True), ((256, 8192, 4096), True),
                                           ((256, 4096, 4096), False)], ids=lambda v: str(v))
def test_nvfp4_partial_store_forms(shape, through, monkeypatch, capfd):
    M, N, K = shape
    monkeypatch.setenv("BSG_LOG", "1")
    p = si.problem("nvfp4", M, N, K, seed=M + N + K, bias=True, out="bf16")
    _check(p, rows=np.unique(np.concatenate([np.arange(0, M, 7), [M - 1]])))
    log = capfd.readouterr().err
    assert "splits" in log and ("(partials through L2)" in log) == through, log


# NVFP4 grids of at least one 256 x 256 tile per CU: 256 x 256 tiles (B shared: 256 rows decoded per K
# tile into LDS; 8 waves of 64 x 128).  Ragged M / N, a final half K tile, every epilogue.
NVFP4_256_SHAPES = [(4096, 4096, 256), (4000, 4112, 1056), (2048, 8192, 512)]


@pytest.mark.parametrize("shape", NVFP4_256_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("epi", ["plain", "bias_silu_f16"])
def test_nvfp4_256x256(shape, epi):
    M, N, K = shape
    plain = epi == "plain"
    p = si.problem("nvfp4", M, N, K, seed=M + N + K, bias=not plain, silu=not plain,
                   out="bf16" if plain else "f16", alpha=0.75)
    plan = make_plan(p)
    assert plan.info()["variant"].startswith("nvfp4_256x256"), plan.info()
    D = run(p, plan=plan)
    _full_coverage(D)
    rows = _band_rows(M, extra=(M - 1,))
    rep = compare(D[rows], reference(p, rows=rows), p["alpha"], p["silu"], p["out"])
    print(f"[parity] nvfp4 {shape} {epi} max_rel={rep['max_rel_err']:.3g}", flush=True)
    assert rep["ok"], rep


def test_nvfp4_256x256_exact_regime_bit_exact():
    p = _exact_regime_problem("nvfp4", 4096, 4096, 512, seed=41, out="bf16")
    plan = make_plan(p)
    assert plan.info()["variant"].startswith("nvfp4_256x256")
    D = run(p, plan=plan)
    rows = _band_rows(4096, extra=(4095,))
    R = reference(p, rows=rows)["bits"]
    assert np.array_equal(D[rows], R), f"{int((D[rows] != R).sum())} of {R.size} sampled entries differ"