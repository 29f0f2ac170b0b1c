"""Light performance-regression guard: the benchmark workloads' kernel times stay within a margin of
their measured steady-state values on MI355X (HIP events on the launch stream, after a warm-up).

The limits sit ~30% above the measured times, so that box-to-box spread and the clock transient of a
fresh process do not trip them while a kernel that loses its pipelining, its tile order or its
split-K choice does.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
import seeded_inputs as si
from gpu_util import make_plan, to_device

pytestmark = pytest.mark.gpu

# workload: (limit in us per call, warm-up calls, timed calls)
LIMITS = {
    "mxfp8_8192_silu": (520.0, 40, 20),
    "mxfp8_4096": (75.0, 300, 100),
    "nvfp4_128x8192x8192_silu": (45.0, 300, 100),
    "nvfp4_256x4096x4096_loop": (33.0, 300, 100),
}


@pytest.mark.parametrize("name", sorted(LIMITS))
def test_kernel_time_within_limit(name):
    limit, warm, steps = LIMITS[name]
    p = si.workload(name)
    plan = make_plan(p)
    dev = to_device(p)
    stream = torch.cuda.Stream()
    args = (dev["A"], dev["B"], dev["sA"], dev["sB"], dev["D"])
    kw = dict(alpha=float(p["alpha"]), bias=dev["bias"], stream=stream)
    for _ in range(warm):
        plan.run(*args, **kw)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        plan.run(*args, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    print(f"[perf] {name} {plan.info()['variant']}: {us:.1f} us per call (limit {limit})", flush=True)
    assert np.isfinite(us) and us <= limit, (name, us, limit)
    plan.close()


def test_per_call_host_overhead_under_ten_percent():
    # the looped small-M workload from C++: host wall time per call within 10% of the GPU time per call,
    # for direct calls and for HIP-graph replays
    sets = []
    for s in range(2):
        p = si.workload("nvfp4_256x4096x4096_loop", set_id=s)
        d = to_device(p)
        d["alpha"] = float(p["alpha"])
        sets.append(d)
    plan = make_plan(p)
    stream = torch.cuda.Stream()
    bsg.bench_loop(plan, sets, 50, 0, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for d in sets:
        for _ in range(200):
            plan.run(d["A"], d["B"], d["sA"], d["sB"], d["D"], alpha=d["alpha"], stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    gpu_us = e0.elapsed_time(e1) * 1e3 / 400
    direct = bsg.bench_loop(plan, sets, 200, 0, stream) / 400
    graph = bsg.bench_loop(plan, sets, 200, 1, stream) / 400
    print(f"[perf] loop: gpu {gpu_us:.2f} us, direct {direct:.2f} us, graph {graph:.2f} us per call", flush=True)
    assert direct <= 1.1 * gpu_us and graph <= 1.1 * gpu_us, (gpu_us, direct, graph)
