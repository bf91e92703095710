"""The workgroup timeline build (libflce_timeline.so) on the GPU, through
bench.py --timeline in a child process (the child loads that library instead
of libflce.so)."""
import json
import os
import subprocess
import sys

import pytest

import linear_cross_entropy_flce_amd as flce

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(300)
def test_timeline_of_one_step():
    """One step of a 4,096 x 2,048 x 32,000 bf16 workload: every workgroup of
    the forward sweep, the dZ recompute and the dH/dW launch is recorded, on
    all 256 compute units, and each kernel's compute-unit time splits into
    shares that sum to one."""
    T, d, V = 4096, 2048, 32000
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--timeline", "--shape", str(T),
           str(d), str(V), "--warmup", "1", "--cpu-rows", "0", "--shard-steps", "0",
           "--configs", "none"]
    print("running", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    print(r.stderr[-1500:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    tl = json.loads(r.stdout.strip().splitlines()[-1])
    plan = flce.flce_plan(T, d, V, "bf16")
    n_tt, n_vt = T // 256, -(-V // 256)
    ks = tl["kernels"]
    assert tl["compute_units"] == 256
    assert ks["fwd_sweep"]["workgroups"] == n_tt * plan.fwd_splits
    assert ks["bwd_dz"]["workgroups"] == n_tt * n_vt  # one block, one slab, no ignored token
    assert ks["bwd_dhdw"]["workgroups"] >= (d // 256) * n_vt  # the dW tiles, plus dH's
    for name in ("fwd_sweep", "bwd_dz", "bwd_dhdw"):
        e = ks[name]
        assert abs(e["busy"] + e["head"] + e["turnover"] + e["tail"] - 1.0) < 1e-3, (name, e)
        assert 0.5 < e["busy"] <= 1.0, (name, e)
