"""flce_forward_backward: the fused call against the separate calls (bit for
bit) and the oracle; the device-side mean over non-ignored tokens; the bf16
copy of dW; gradient accumulation across micro-batches."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import linear_cross_entropy_flce_amd as flce
import oracle
import workloads as wl
from gpu_helpers import gather_plan, TOL, compare, device_inputs, log, logit_tol, max_abs

pytestmark = pytest.mark.gpu
IGN = wl.IGNORE_INDEX


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    flce.load()
    yield
    torch.cuda.empty_cache()


def _np(t):
    return t.float().cpu().numpy()


def _separate(plan, H, W, y, scale, g):
    red = torch.empty(1, dtype=torch.float32, device=W.device)
    loss, lse, _ = flce.flce_forward(plan, H, W, y, IGN, scale, loss_reduced=red)
    dH, dW = flce.flce_backward(plan, H, W, y, lse, IGN, g)
    torch.cuda.synchronize()
    return dict(loss=_np(loss), lse=_np(lse), red=_np(red), dH=_np(dH), dW=_np(dW))


def _fused(plan, H, W, y, reduction, scale, **kw):
    out = flce.flce_forward_backward(plan, H, W, y, IGN, reduction, scale, **kw)
    torch.cuda.synchronize()
    return {k: (_np(v) if v is not None else None) for k, v in out.items()}


@pytest.mark.parametrize("form", ["in_tile", "gather"])
@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("T,d,V,ign", [(257, 72, 32007, 0.1), (300, 136, 515, 0.3),
                                       (1100, 64, 2049, 0.0)])
def test_fused_equals_separate_and_oracle(T, d, V, ign, dtype, form):
    """The fused call equals the separate calls bit for bit, with either form
    of the forward's target logit, and both match the oracle."""
    inp = wl.make_inputs(T, d, V, dtype, seed=900 + T, sigma_w=0.5, ignore_frac=ign)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(T, d, V, dtype)
    if form == "gather":
        plan = gather_plan(plan)
    n_valid = int((inp.y != IGN).sum())
    # sum: g = scale
    a = _fused(plan, H, W, y, "sum", 0.25)
    b = _separate(plan, H, W, y, 0.25, 0.25)
    for k in ("loss", "lse", "dH", "dW"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    assert np.array_equal(a["loss_reduced"], b["red"])
    # mean over the non-ignored tokens: g = 1 / N, counted on the device
    g = float(np.float32(1.0 / n_valid))
    a = _fused(plan, H, W, y, "mean_valid", 1.0)
    b = _separate(plan, H, W, y, g, g)
    for k in ("loss", "lse", "dH", "dW"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    ref_loss, ref_lse, ref_dH, ref_dW = oracle.forward_backward(inp.H_f32(), inp.W_f32(), inp.y,
                                                                IGN, 1.0 / n_valid)
    tl = logit_tol(dtype, d, float(np.abs(oracle.logits(inp.H_f32(), inp.W_f32())).max()))
    errs = compare(a, dict(loss=ref_loss, lse=ref_lse, dH=ref_dH, dW=ref_dW), dtype, loss_tol=tl)
    mean = oracle.reduced_loss(ref_loss, 1.0 / n_valid)
    assert abs(float(a["loss_reduced"][0]) - mean) <= tl
    log("  mean_valid errors", errs)


@pytest.mark.parametrize("i", range(12))
def test_random_fused_case(i):
    """Random shapes through the fused call: either reduction, sometimes
    accumulating into an existing dW, sometimes with the bf16 copy; against
    the oracle, and bit for bit against the separate calls with the same g."""
    rng = np.random.default_rng(6000 + i)
    dtype = (wl.DTYPE_F32, wl.DTYPE_BF16)[i % 2]
    T = int(rng.integers(1, 2000))
    d = 8 * int(rng.integers(1, 49))
    V = int(rng.integers(2, 15001))
    reduction = ("sum", "mean_valid")[int(rng.integers(2))]
    scale = float(rng.choice([1.0, 0.5]))
    acc = bool(rng.random() < 0.4)
    with_bf16 = bool(rng.random() < 0.5)
    ign = float(rng.choice([0.0, 0.3, 0.8]))
    log(f"fused case {i}: {dtype} T={T} d={d} V={V} {reduction} scale={scale} acc={acc} "
        f"bf16={with_bf16} ign={ign}")
    inp = wl.make_inputs(T, d, V, dtype, seed=int(rng.integers(1 << 30)), sigma_w=0.3,
                         ignore_frac=ign)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(T, d, V, dtype)
    n_valid = int((inp.y != IGN).sum())
    g = scale if reduction == "sum" else (float(np.float32(scale) / np.float32(n_valid))
                                          if n_valid else 0.0)
    base = rng.standard_normal((V, d)).astype(np.float32)
    dW = torch.from_numpy(base).cuda() if acc else None
    dWb = torch.empty((V, d), dtype=torch.bfloat16, device=W.device) if with_bf16 else None
    a = _fused(plan, H, W, y, reduction, scale, dW=dW, accumulate_dW=acc, dW_bf16=dWb)
    # the separate calls with the same g
    red = torch.empty(1, dtype=torch.float32, device=W.device)
    loss, lse, _ = flce.flce_forward(plan, H, W, y, IGN, g, loss_reduced=red)
    dW2 = torch.from_numpy(base).cuda() if acc else None
    dH2, dW2 = flce.flce_backward(plan, H, W, y, lse, IGN, g, dW=dW2, accumulate_dW=acc)
    torch.cuda.synchronize()
    for k, v in (("loss", loss), ("lse", lse), ("dH", dH2), ("dW", dW2)):
        assert np.array_equal(a[k], _np(v), equal_nan=True), k
    if with_bf16:
        assert np.array_equal(a["dW_bf16"], _np(dW2.to(torch.bfloat16)))
    ref_loss, ref_lse, ref_dH, ref_dW = oracle.forward_backward(inp.H_f32(), inp.W_f32(), inp.y,
                                                                IGN, g)
    if acc:
        ref_dW = ref_dW + base
    tl = logit_tol(dtype, d, float(np.abs(oracle.logits(inp.H_f32(), inp.W_f32())).max()))
    compare(a, dict(loss=ref_loss, lse=ref_lse, dH=ref_dH, dW=ref_dW), dtype, loss_tol=tl,
            grad_tol=TOL[dtype]["grad"] + (tl - TOL[dtype]["loss"]))
    ref_red = oracle.reduced_loss(ref_loss, g)
    assert abs(float(a["loss_reduced"][0]) - ref_red) <= tl * max(1.0, g * T)


def test_mean_over_no_tokens_is_zero():
    inp = wl.make_inputs(300, 64, 1000, wl.DTYPE_BF16, seed=5, sigma_w=0.5, ignore_frac=1.0)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(inp.T, inp.d, inp.V, inp.dtype)
    a = _fused(plan, H, W, y, "mean_valid", 1.0)
    assert a["loss_reduced"][0] == 0.0
    assert not np.any(a["dH"]) and not np.any(a["dW"])


def test_dW_bf16_is_rounded_dW():
    inp = wl.make_inputs(600, 128, 3001, wl.DTYPE_BF16, seed=6, sigma_w=0.5)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(inp.T, inp.d, inp.V, inp.dtype)
    dWb = torch.empty((inp.V, inp.d), dtype=torch.bfloat16, device=W.device)
    out = flce.flce_forward_backward(plan, H, W, y, IGN, "sum", 1.0, dW_bf16=dWb)
    torch.cuda.synchronize()
    got = dWb.view(torch.int16).cpu().numpy().view(np.uint16)
    want = wl.f32_to_bf16_bits(out["dW"].cpu().numpy())
    assert np.array_equal(got, want)


def _bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("ign,acc", [(0.6, False), (0.6, True), (0.0, True), (1.0, False),
                                     (1.0, True)])
def test_dW_bf16_over_token_blocks(dtype, ign, acc):
    """Six token blocks of 256 (a small workspace cap), the trailing ones
    empty when most tokens are ignored, or all of them: the bf16 copy, which
    the dW tiles of the last block holding tokens write (block 0 when none
    does), is dW rounded to nearest even in every element, and dW equals the
    separate calls' bit for bit."""
    T, d, V = 1500, 64, 3000
    inp = wl.make_inputs(T, d, V, dtype, seed=4100 + int(10 * ign) + acc, sigma_w=0.5,
                         ignore_frac=ign)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(T, d, V, dtype, 400_000)
    n_valid = int((inp.y != IGN).sum())
    log(f"  {plan.n_blocks} blocks of {plan.bwd_block}, {plan.n_slabs} slabs, "
        f"{n_valid} tokens not ignored")
    assert plan.n_blocks >= 3
    base = np.random.default_rng(41).standard_normal((V, d)).astype(np.float32)
    dW = torch.from_numpy(base).cuda() if acc else None
    # NaN everywhere first, so that an element the kernels skip shows
    dWb = torch.full((V, d), float("nan"), dtype=torch.bfloat16, device=W.device)
    a = flce.flce_forward_backward(plan, H, W, y, IGN, "sum", 0.5, dW=dW, accumulate_dW=acc,
                                   dW_bf16=dWb)
    dW2 = torch.from_numpy(base).cuda() if acc else None
    _, lse, _ = flce.flce_forward(plan, H, W, y, IGN, 0.5)
    _, dW2 = flce.flce_backward(plan, H, W, y, lse, IGN, 0.5, dW=dW2, accumulate_dW=acc)
    torch.cuda.synchronize()
    assert np.array_equal(_np(a["dW"]), _np(dW2))
    assert np.array_equal(_bf16_bits(dWb), wl.f32_to_bf16_bits(_np(a["dW"])))
    if n_valid == 0:
        assert np.array_equal(_np(a["dW"]), base if acc else np.zeros_like(base))


@pytest.mark.parametrize("acc", [False, True])
def test_dW_bf16_without_tokens(acc):
    """T = 0: no dW tile runs, so the copy takes a pass of its own; it is the
    caller's dW rounded (accumulating) or zeros."""
    d, V = 64, 1000
    dev = torch.device("cuda:0")
    H = torch.empty((0, d), dtype=torch.bfloat16, device=dev)
    W = torch.randn((V, d), device=dev).to(torch.bfloat16)
    y = torch.empty(0, dtype=torch.int64, device=dev)
    plan = flce.flce_plan(0, d, V, wl.DTYPE_BF16)
    base = torch.randn((V, d), device=dev)
    dW = base.clone()
    dWb = torch.full((V, d), float("nan"), dtype=torch.bfloat16, device=dev)
    flce.flce_forward_backward(plan, H, W, y, IGN, "sum", 1.0, dW=dW, accumulate_dW=acc,
                               dW_bf16=dWb)
    torch.cuda.synchronize()
    want = base if acc else torch.zeros_like(base)
    assert torch.equal(dW, want)
    assert np.array_equal(_bf16_bits(dWb), wl.f32_to_bf16_bits(_np(want)))


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_micro_batch_accumulation(dtype):
    """Two micro-batches, the second accumulating into the first's fp32 dW,
    give the gradient of the whole batch (sum reduction, one g)."""
    inp = wl.make_inputs(800, 96, 5000, dtype, seed=7, sigma_w=0.5, ignore_frac=0.1)
    H, W, y = device_inputs(inp)
    g = 1.0 / inp.T
    half = inp.T // 2
    p1 = flce.flce_plan(half, inp.d, inp.V, dtype)
    p2 = flce.flce_plan(inp.T - half, inp.d, inp.V, dtype)
    dWb = torch.empty((inp.V, inp.d), dtype=torch.bfloat16, device=W.device)
    o1 = flce.flce_forward_backward(p1, H[:half].contiguous(), W, y[:half].contiguous(), IGN,
                                    "sum", g)
    o2 = flce.flce_forward_backward(p2, H[half:].contiguous(), W, y[half:].contiguous(), IGN,
                                    "sum", g, dW=o1["dW"], accumulate_dW=True, dW_bf16=dWb)
    torch.cuda.synchronize()
    ref_loss, ref_lse, ref_dH, ref_dW = oracle.forward_backward(inp.H_f32(), inp.W_f32(), inp.y,
                                                                IGN, g)
    dH = np.concatenate([_np(o1["dH"]), _np(o2["dH"])])
    tl = logit_tol(dtype, inp.d, float(np.abs(oracle.logits(inp.H_f32(), inp.W_f32())).max()))
    errs = compare(dict(loss=np.concatenate([_np(o1["loss"]), _np(o2["loss"])]),
                        lse=np.concatenate([_np(o1["lse"]), _np(o2["lse"])]),
                        dH=dH, dW=_np(o2["dW"])),
                   dict(loss=ref_loss, lse=ref_lse, dH=ref_dH, dW=ref_dW), dtype, loss_tol=tl)
    got = dWb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, wl.f32_to_bf16_bits(_np(o2["dW"])))
    log("  micro-batch errors", errs)


@pytest.mark.timeout(600)
def test_config2_mean_valid_fused():
    """The 16,384-token workload (d = 2,048, V = 151,936, Zipf targets, 25%
    ignored; mean over the valid tokens): the fused call's device count gives
    the same bits as the separate calls with g = 1/N_valid, which the unfused
    test of that workload checks against the oracle."""
    cfg = wl.CONFIGS[2]
    inp = wl.config_inputs(cfg)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(cfg.T, cfg.d, cfg.V, cfg.dtype)
    ls, gs = cfg.scales()
    a = _fused(plan, H, W, y, "mean_valid", 1.0)
    b = _separate(plan, H, W, y, ls, gs)
    for k in ("loss", "lse", "dH", "dW"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    assert max_abs(a["loss_reduced"], b["red"]) <= 1e-6 * abs(float(b["red"][0]))
