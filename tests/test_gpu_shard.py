"""Vocab-parallel shard mode on one GPU against the oracle.

The shards of W are run one after another on the same GPU and their
statistics stacked as an all-gather would; merged, they must give the
unsharded method's loss and lse, and the shards' backward must give its dH
(sum of the partials) and dW (concatenation).  The oracle is the plain
unsharded computation; the shard statistics are also checked one by one."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import (TOL, compare, device_inputs, log, logit_tol, max_abs, run_gpu,
                         run_gpu_shards)

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_flce_amd as flce
    flce.load()
    yield
    torch.cuda.empty_cache()


def _ref(inp, g):
    loss, lse, dH, dW = oracle.forward_backward(inp.H_f32(), inp.W_f32(), inp.y, IGN, g)
    return dict(loss=loss, lse=lse, dH=dH, dW=dW)


CASES = [
    # T, d, V, dtype, shard bounds, targets, ignore fraction
    (520, 64, 3001, wl.DTYPE_BF16, [0, 1500, 3001], "zipf", 0.1),
    (300, 136, 515, wl.DTYPE_F32, [0, 100, 315, 515], "uniform", 0.2),
    (257, 72, 32007, wl.DTYPE_BF16, [0, 256, 20000, 32007], "uniform", 0.0),
]


@pytest.mark.parametrize("form", ["in_tile", "gather"])
@pytest.mark.parametrize("T,d,V,dtype,bounds,targets,ign", CASES)
def test_shards_match_unsharded(T, d, V, dtype, bounds, targets, ign, form):
    """Either form of the target logit: taken in each shard's tiles, or by index."""
    inp = wl.make_inputs(T, d, V, dtype, seed=500 + T + V, sigma_w=0.5, targets=targets,
                         ignore_frac=ign)
    g = 0.01
    got = run_gpu_shards(inp, bounds, loss_scale=1.0 / T, grad_scale=g, gather=form == "gather")
    ref = _ref(inp, g)
    zmax = float(np.abs(oracle.logits(inp.H_f32(), inp.W_f32())).max())
    # a gathered fp32 target logit sums in another order than the tile: sqrt(d) ulps of |z|
    ztol = logit_tol(dtype, d, zmax) if form == "gather" else TOL[dtype]["loss"]
    errs = compare(got, ref, dtype, loss_tol=ztol)
    log("  errors", errs)
    assert abs(got["red"][0] - oracle.reduced_loss(ref["loss"], 1.0 / T)) <= TOL[dtype]["loss"]
    # each shard's statistics against the oracle restricted to its columns
    Z = oracle.logits(inp.H_f32(), inp.W_f32())
    for s, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        lse_s = oracle.log_sum_exp_rows(Z[:, a:b])
        assert max_abs(got["lse_shards"][s], lse_s) <= TOL[dtype]["loss"]
        inside = (inp.y >= a) & (inp.y < b)
        zt = got["zt_shards"][s]
        assert np.all(np.isneginf(zt[~inside]))
        rows = np.nonzero(inside)[0]
        assert max_abs(zt[rows], Z[rows, inp.y[rows]]) <= ztol


def test_one_shard_equals_unsharded():
    """A single shard covering the vocabulary is the unsharded method, bit for bit."""
    inp = wl.make_inputs(300, 136, 1000, wl.DTYPE_BF16, seed=77, sigma_w=0.5, ignore_frac=0.2)
    a = run_gpu_shards(inp, [0, 1000], grad_scale=0.5)
    b = run_gpu(inp, grad_scale=0.5)
    for k in ("loss", "lse", "dH", "dW"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_merge_order_and_missing_shard():
    """Merging the shards in another order changes only rounding; merging
    without a shard leaves the tokens whose target it holds with a NaN loss;
    out-of-range targets are NaN, ignored tokens 0."""
    T, d, V = 400, 64, 2000
    bounds = [0, 700, 1300, 2000]
    inp = wl.make_inputs(T, d, V, wl.DTYPE_BF16, seed=91, sigma_w=0.5, ignore_frac=0.1)
    inp.y[5] = V + 3          # invalid
    inp.y[6] = -7             # invalid
    fwd = run_gpu_shards(inp, bounds, backward=False)
    rev = run_gpu_shards(inp, bounds, merge=[2, 1, 0], backward=False)
    valid = (inp.y >= 0) & (inp.y < V)
    assert max_abs(fwd["lse"], rev["lse"]) <= 1e-5
    assert max_abs(fwd["loss"], rev["loss"], valid) <= 1e-5
    assert np.all(np.isnan(fwd["loss"][[5, 6]]))
    ign = inp.y == IGN
    assert np.all(fwd["loss"][ign] == 0.0)
    part = run_gpu_shards(inp, bounds, merge=[0, 2], backward=False)
    in_mid = (inp.y >= 700) & (inp.y < 1300)
    assert np.all(np.isnan(part["loss"][in_mid]))
    ok = valid & ~in_mid
    assert np.all(np.isfinite(part["loss"][ok]))


@pytest.mark.timeout(900)
def test_pages_tp2_rank_shape():
    """The pages' vocab-parallel setting: a 248,320-id vocabulary on two ranks
    of 124,160 rows, d = 2,048, bf16, one 8,192-token block.  Both shards run
    on this GPU; the oracle checks 128 seeded rows (loss, lse, dH) and a
    512-token sub-batch (dW); at full size the dW rows of both shards
    together sum to zero."""
    T, d, Vt = 8192, 2048, 248320
    inp = wl.make_inputs(T, d, Vt, wl.DTYPE_BF16, seed=4242, sigma_w=0.02)
    bounds = [0, 124160, 248320]
    log("  gpu shards")
    got = run_gpu_shards(inp, bounds)
    assert np.all(np.isfinite(got["loss"])) and np.all(np.isfinite(got["dW"]))
    rows = np.sort(wl.streams(4242)[4].choice(T, 128, replace=False))
    log("  oracle rows")
    loss, lse, dH = oracle.rows_forward_dH(inp.H_f32(), inp.W_f32(), inp.y, rows, IGN, 1.0)
    errs = compare(got, dict(loss=loss, lse=lse, dH=dH), wl.DTYPE_BF16,
                   what=("loss", "lse", "dH"), rows=rows)
    log("  row errors", errs)
    colsum = got["dW"].astype(np.float64).sum(axis=0)
    scale = np.abs(got["dW"]).astype(np.float64).sum(axis=0).max()
    assert np.abs(colsum).max() <= 1e-3 * scale
    del got
    torch.cuda.empty_cache()
    sub = np.sort(wl.streams(4243)[4].choice(T, 512, replace=False))
    sinp = inp.rows(sub)
    log("  gpu sub-batch")
    sg = run_gpu_shards(sinp, bounds)
    log("  oracle sub-batch")
    errs = compare(sg, _ref(sinp, 1.0), wl.DTYPE_BF16)
    log("  sub-batch errors", errs)
