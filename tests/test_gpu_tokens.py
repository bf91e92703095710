"""Token scoring (gathered logits minus lse) against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import linear_cross_entropy_flce_amd as flce
import oracle
import workloads as wl
from gpu_helpers import TOL, device_inputs, log, logit_tol, max_abs

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    flce.load()
    yield
    torch.cuda.empty_cache()


def _tokens(seed, T, K, V, n_bad=0):
    g = np.random.default_rng(seed)
    tok = g.integers(0, V, size=(T, K), dtype=np.int64)
    if n_bad:
        idx = g.choice(T * K, n_bad, replace=False)
        tok.reshape(-1)[idx[: n_bad // 2]] = -1
        tok.reshape(-1)[idx[n_bad // 2:]] = V
    return tok


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("T,d,V,K", [(1, 8, 1, 1), (63, 72, 1000, 3), (300, 136, 515, 5),
                                     (257, 64, 32007, 2)])
def test_scores_match_oracle(T, d, V, K, dtype):
    inp = wl.make_inputs(T, d, V, dtype, seed=700 + T + V, sigma_w=0.5)
    H, W, y = device_inputs(inp)
    tok = _tokens(T + K, T, K, V, n_bad=min(4, T * K // 2) if V > 1 else 0)
    plan = flce.flce_plan(T, d, V, dtype)
    _, lse, _ = flce.flce_forward(plan, H, W, y, IGN)
    tt = torch.from_numpy(tok).cuda()
    got = flce.flce_token_logprobs(H, W, tt, lse).cpu().numpy()
    raw = flce.flce_token_logprobs(H, W, tt).cpu().numpy()
    Z = oracle.logits(inp.H_f32(), inp.W_f32())
    lse_ref = oracle.log_sum_exp_rows(Z)
    ok = (tok >= 0) & (tok < V)
    assert np.all(np.isnan(got[~ok])) and np.all(np.isnan(raw[~ok]))
    r, c = np.nonzero(ok)
    ref_logit = Z[r, tok[r, c]]
    # the gathered dot product and the forward's lse are fp32 sums of d terms
    # in their own orders (sigma_W = 0.5 gives |z| ~ 25 here)
    tol = logit_tol(dtype, d, float(np.abs(Z).max()))
    assert max_abs(raw[r, c], ref_logit) <= tol
    assert max_abs(got[r, c], ref_logit - lse_ref[r]) <= tol


@pytest.mark.parametrize("i", range(16))
def test_random_scoring_case(i):
    """Random T, d, V and K = 1..20 tokens per position (the kernel takes up
    to eight gathered rows per pass, so K spans one to three passes and the
    padded widths 1, 2, 4 and 8), with and without lse, some ids invalid."""
    rng = np.random.default_rng(8000 + i)
    dtype = (wl.DTYPE_F32, wl.DTYPE_BF16)[i % 2]
    T = int(rng.integers(1, 800))
    d = 8 * int(rng.integers(1, 129))
    V = int(rng.integers(2, 9001))
    K = int(rng.integers(1, 21))
    log(f"scoring case {i}: {dtype} T={T} d={d} V={V} K={K}")
    inp = wl.make_inputs(T, d, V, dtype, seed=int(rng.integers(1 << 30)), sigma_w=0.3)
    H, W, y = device_inputs(inp)
    tok = _tokens(int(rng.integers(1 << 30)), T, K, V, n_bad=min(6, T * K // 3))
    plan = flce.flce_plan(T, d, V, dtype)
    _, lse, _ = flce.flce_forward(plan, H, W, y, IGN)
    tt = torch.from_numpy(tok).cuda()
    got = flce.flce_token_logprobs(H, W, tt, lse).cpu().numpy()
    raw = flce.flce_token_logprobs(H, W, tt).cpu().numpy()
    Z = oracle.logits(inp.H_f32(), inp.W_f32())
    lse_ref = oracle.log_sum_exp_rows(Z)
    ok = (tok >= 0) & (tok < V)
    assert np.all(np.isnan(got[~ok])) and np.all(np.isnan(raw[~ok]))
    r, c = np.nonzero(ok)
    tol = logit_tol(dtype, d, float(np.abs(Z).max()))
    assert max_abs(raw[r, c], Z[r, tok[r, c]]) <= tol
    assert max_abs(got[r, c], Z[r, tok[r, c]] - lse_ref[r]) <= tol


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_target_scores_are_minus_loss(dtype):
    inp = wl.make_inputs(400, 128, 3000, dtype, seed=31, sigma_w=0.5, ignore_frac=0.2)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(inp.T, inp.d, inp.V, dtype)
    loss, lse, _ = flce.flce_forward(plan, H, W, y, IGN)
    valid = inp.y != IGN
    yv = torch.where(y == IGN, torch.zeros_like(y), y)
    lp = flce.flce_token_logprobs(H, W, yv, lse).cpu().numpy()
    # the score's logit and the loss's target logit are the same fp32 value up
    # to summation order (sqrt(d) ulps of the logits' magnitude, as above)
    tol = logit_tol(dtype, inp.d, float(np.abs(oracle.logits(inp.H_f32(), inp.W_f32())).max()))
    assert max_abs(lp, -loss.cpu().numpy(), valid) <= tol


@pytest.mark.timeout(600)
def test_pages_shape_sampled():
    """T = 65,536, d = 2,048, V = 124,160, bf16, four tokens per position;
    the oracle checks 256 seeded rows."""
    cfg = wl.CONFIGS[3]
    inp = wl.config_inputs(cfg)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(cfg.T, cfg.d, cfg.V, cfg.dtype)
    _, lse, _ = flce.flce_forward(plan, H, W, y, IGN)
    tok = _tokens(99, cfg.T, 4, cfg.V)
    got = flce.flce_token_logprobs(H, W, torch.from_numpy(tok).cuda(), lse).cpu().numpy()
    rows = wl.sample_rows(cfg, 256)
    log("  oracle rows")
    Z = oracle.logits(inp.H_f32()[rows], inp.W_f32())
    lse_ref = oracle.log_sum_exp_rows(Z)
    ref = np.take_along_axis(Z, tok[rows], axis=1) - lse_ref[:, None]
    err = max_abs(got[rows], ref)
    log("  max abs error", err)
    assert err <= TOL[cfg.dtype]["loss"]
