"""Metamorphic properties of the GPU path that hold whatever the oracle says:
permuting the tokens permutes every per-token output and leaves dW alone;
permuting the vocabulary (rows of W, targets remapped) permutes dW's rows and
leaves the rest alone; the dW of a batch is the sum of its token parts."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import TOL, log, max_abs, rel_fro, run_gpu

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


def _inputs(dtype):
    # several token blocks' worth of tiles and a ragged vocab tail
    return wl.make_inputs(1300, 128, 5003, dtype, seed=61, sigma_w=0.3, ignore_frac=0.1)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_token_permutation(dtype):
    inp = _inputs(dtype)
    perm = np.random.default_rng(1).permutation(inp.T)
    a = run_gpu(inp, grad_scale=0.01)
    b = run_gpu(wl.Inputs(inp.H[perm], inp.W, inp.y[perm], dtype), grad_scale=0.01)
    tol = TOL[dtype]
    # a token's row is computed by the same tile arithmetic wherever it sits
    # in the batch only up to the tile it lands in; compare within tolerance
    assert max_abs(b["loss"], a["loss"][perm]) <= tol["loss"]
    assert max_abs(b["lse"], a["lse"][perm]) <= tol["loss"]
    assert rel_fro(b["dH"], a["dH"][perm]) <= tol["grad"]
    assert rel_fro(b["dW"], a["dW"]) <= tol["grad"]


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_vocab_permutation(dtype):
    inp = _inputs(dtype)
    perm = np.random.default_rng(2).permutation(inp.V)   # new row r holds old row perm[r]
    inv = np.argsort(perm)
    y2 = inp.y.copy()
    valid = y2 != IGN
    y2[valid] = inv[y2[valid]]
    a = run_gpu(inp, grad_scale=0.01)
    b = run_gpu(wl.Inputs(inp.H, inp.W[perm], y2, dtype), grad_scale=0.01)
    tol = TOL[dtype]
    assert max_abs(b["loss"], a["loss"]) <= tol["loss"]
    assert max_abs(b["lse"], a["lse"]) <= tol["loss"]
    assert rel_fro(b["dH"], a["dH"]) <= tol["grad"]
    assert rel_fro(b["dW"], a["dW"][perm]) <= tol["grad"]


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_dW_is_sum_over_token_parts(dtype):
    inp = _inputs(dtype)
    cuts = [0, 300, 301, 1024, inp.T]          # uneven parts, one of a single token
    whole = run_gpu(inp, grad_scale=0.01)
    total = np.zeros_like(whole["dW"], dtype=np.float64)
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = run_gpu(inp.rows(np.arange(a, b)), grad_scale=0.01)
        assert max_abs(part["loss"], whole["loss"][a:b]) <= TOL[dtype]["loss"]
        total += part["dW"]
    err = rel_fro(total, whole["dW"])
    log("  dW parts vs whole", err)
    assert err <= TOL[dtype]["grad"]
