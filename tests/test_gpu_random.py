"""Seeded random shapes against the oracle, unsharded and as vocab shards.

Each case draws its dtype, a ragged token count, hidden size and vocabulary,
an ignored fraction, a weight scale, a gradient scale, sometimes a small
workspace cap (several token blocks and vocab slabs, with or without the dH
partial buffer) and sometimes dW accumulation, so that tile tails, planner
choices and the accumulator modes meet in combinations the hand-picked tests
do not list.  Every plan is made and checked on the host before anything is
launched.
"""
import numpy as np
import pytest
import torch

import linear_cross_entropy_flce_amd as flce
import oracle
import workloads as wl
from gpu_helpers import TOL, compare, log, logit_tol, run_gpu, run_gpu_shards

pytestmark = pytest.mark.gpu

IGN = wl.IGNORE_INDEX
N_CASES = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    flce.load()
    yield
    torch.cuda.empty_cache()


def _case(i):
    rng = np.random.default_rng(9000 + i)
    dtype = (wl.DTYPE_F32, wl.DTYPE_BF16)[i % 2]
    T = int(rng.integers(1, 2500))
    d = 8 * int(rng.integers(1, 65))
    V = int(rng.integers(1, 20001))
    return dict(dtype=dtype, T=T, d=d, V=V,
                ign=float(rng.choice([0.0, 0.1, 0.5, 0.95])),
                sigma=float(rng.choice([0.02, 0.1, 0.4])),
                g=float(rng.choice([1.0, 1.0 / T, 0.37])),
                cap_frac=float(rng.choice([0.0, 0.0, 0.02, 0.05, 0.3])),
                acc=bool(rng.random() < 0.3), seed=int(rng.integers(1 << 30)))


def _code(dtype):
    return flce.FLCE_BF16 if dtype == wl.DTYPE_BF16 else flce.FLCE_F32


def _cap(c):
    """0 (the default) or a fraction of the default plan's backward
    workspace, raised until some plan fits."""
    if c["cap_frac"] == 0.0:
        return 0
    full = flce.flce_plan(c["T"], c["d"], c["V"], c["dtype"])
    cap = max(int(full.bwd_ws_bytes * c["cap_frac"]), 4096)
    while flce.flce_plan_status(c["T"], c["d"], c["V"], _code(c["dtype"]), cap=cap)[0] != flce.FLCE_OK:
        cap = int(cap * 1.5)
    return cap


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = _case(i)
    cap = _cap(c)
    st, plan = flce.flce_plan_status(c["T"], c["d"], c["V"], _code(c["dtype"]), cap=cap)
    assert st == flce.FLCE_OK
    log(f"case {i}: {c} cap={cap} blocks={plan.n_blocks} slabs={plan.n_slabs} "
        f"split={plan.dh_split_bytes}")
    inp = wl.make_inputs(c["T"], c["d"], c["V"], c["dtype"], seed=c["seed"], sigma_w=c["sigma"],
                         ignore_frac=c["ign"])
    base = None
    if c["acc"]:
        base = np.random.default_rng(c["seed"] + 1).standard_normal((c["V"], c["d"])).astype(
            np.float32)
    got = run_gpu(inp, loss_scale=c["g"], grad_scale=c["g"], cap=cap, accumulate_dW=c["acc"],
                  dW_init=base)
    Hf, Wf = inp.H_f32(), inp.W_f32()
    loss, lse, dH, dW = oracle.forward_backward(Hf, Wf, inp.y, IGN, c["g"])
    if base is not None:
        dW = dW + base
    # fp32: sums of d terms in the kernels' order differ from the oracle's by
    # about sqrt(d) ulps of |z|; the same absolute error in z - lse is the
    # relative error of each dZ entry
    zmax = float(np.abs(oracle.logits(Hf, Wf)).max()) if c["T"] * c["V"] else 0.0
    ltol = logit_tol(c["dtype"], c["d"], zmax)
    errs = compare(got, dict(loss=loss, lse=lse, dH=dH, dW=dW), c["dtype"], loss_tol=ltol,
                   grad_tol=TOL[c["dtype"]]["grad"] + (ltol - TOL[c["dtype"]]["loss"]))
    red = float(got["red"][0])
    ref_red = oracle.reduced_loss(loss, c["g"])
    assert abs(red - ref_red) <= ltol * max(1.0, c["g"] * c["T"]), (red, ref_red)
    log("  errors", errs)


N_SHARD_CASES = 24


@pytest.mark.parametrize("i", range(N_SHARD_CASES))
def test_random_shard_case(i):
    """The vocab-parallel path over random shard cuts (2 to 4 shards, some
    narrower than a vocab tile), merged in order, against the unsharded
    oracle."""
    rng = np.random.default_rng(7000 + i)
    dtype = (wl.DTYPE_F32, wl.DTYPE_BF16)[i % 2]
    T = int(rng.integers(1, 1500))
    d = 8 * int(rng.integers(1, 49))
    V = int(rng.integers(4, 12001))
    n = int(rng.integers(2, 5))
    cuts = np.sort(rng.choice(np.arange(1, V), size=min(n - 1, V - 1), replace=False))
    bounds = [0, *[int(c) for c in cuts], V]
    ign = float(rng.choice([0.0, 0.2, 0.9]))
    targets = str(rng.choice(["uniform", "zipf"]))
    g = float(rng.choice([1.0, 1.0 / T]))
    log(f"shard case {i}: {dtype} T={T} d={d} V={V} bounds={bounds} ign={ign} {targets}")
    inp = wl.make_inputs(T, d, V, dtype, seed=int(rng.integers(1 << 30)), sigma_w=0.3,
                         targets=targets, ignore_frac=ign)
    got = run_gpu_shards(inp, bounds, loss_scale=g, grad_scale=g)
    Hf, Wf = inp.H_f32(), inp.W_f32()
    loss, lse, dH, dW = oracle.forward_backward(Hf, Wf, inp.y, IGN, g)
    zmax = float(np.abs(oracle.logits(Hf, Wf)).max())
    ltol = logit_tol(dtype, d, zmax)
    errs = compare(got, dict(loss=loss, lse=lse, dH=dH, dW=dW), dtype, loss_tol=ltol,
                   grad_tol=TOL[dtype]["grad"] + (ltol - TOL[dtype]["loss"]))
    log("  errors", errs)
