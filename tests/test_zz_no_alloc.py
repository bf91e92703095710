"""The allocation-free entry point against the one it varies.

flce_forward_backward_scratch runs on the library's static scratch array; it
must give, bit for bit, what flce_forward_backward gives with a caller
workspace and the same plan: two calls in a row, the second with a smaller
input (the array keeps the first call's contents), for bf16 and fp32, with
the device-side mean over valid tokens and the bf16 copy of dW, and with dW
accumulated.
"""
import numpy as np
import pytest
import torch

import linear_cross_entropy_flce_amd as flce
import workloads as wl
from gpu_helpers import device_inputs, gather_plan, log

pytestmark = pytest.mark.gpu

CAP = flce.FLCE_SCRATCH_BYTES - 256


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    flce.load()
    yield


def _outputs(plan, dev, et, base_dW):
    T, d, V = plan.T, plan.d, plan.V
    return dict(loss=torch.full((T,), float("nan"), device=dev),
                lse=torch.full((T,), float("nan"), device=dev),
                loss_reduced=torch.full((1,), float("nan"), device=dev),
                dH=torch.full((T, d), float("nan"), device=dev).to(et),
                dW=base_dW.clone(),
                dW_bf16=torch.full((V, d), float("nan"), device=dev).to(torch.bfloat16))


def _check_pair(T, d, V, dtype, seed, reduction, accumulate, gather=False):
    log(f"scratch call T={T} d={d} V={V} {dtype} {reduction} acc={accumulate} gather={gather}")
    inp = wl.make_inputs(T, d, V, dtype, seed=seed, sigma_w=0.3, ignore_frac=0.1)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(T, d, V, dtype, CAP)
    if gather:
        plan = gather_plan(plan)
    assert plan.ws_bytes <= flce.FLCE_SCRATCH_BYTES
    dev = W.device
    base = torch.randn((V, d), device=dev, generator=torch.Generator(dev).manual_seed(seed))
    a = _outputs(plan, dev, H.dtype, base)
    b = _outputs(plan, dev, H.dtype, base)
    ws = flce.workspace(plan, dev)
    flce.flce_forward_backward(plan, H, W, y, wl.IGNORE_INDEX, reduction, 0.5,
                               accumulate_dW=accumulate, ws=ws, **a)
    flce.flce_forward_backward_scratch(plan, H, W, y, wl.IGNORE_INDEX, reduction, 0.5,
                                       accumulate_dW=accumulate, **b)
    torch.cuda.synchronize()
    for k in a:
        # identical bits (NaN-safe: compare the raw bytes)
        x = a[k].contiguous().view(torch.uint8).cpu().numpy()
        z = b[k].contiguous().view(torch.uint8).cpu().numpy()
        assert np.array_equal(x, z), k
    assert np.all(np.isfinite(a["loss"].cpu().numpy()))
    return plan


@pytest.mark.parametrize("dtype", [wl.DTYPE_BF16, wl.DTYPE_F32])
def test_scratch_call_matches_workspace_call(dtype):
    # a first call with several token blocks and vocab slabs in the array,
    # then a smaller one over what the first left there
    p1 = _check_pair(6000, 1024 if dtype == wl.DTYPE_BF16 else 512, 30000, dtype, 71,
                     "mean_valid", False)
    assert p1.n_slabs >= 2 or p1.n_blocks >= 2
    _check_pair(700, 256, 5000, dtype, 72, "sum", True, gather=True)


def test_scratch_call_refuses_a_large_plan():
    """The default plan at the pages' shape needs 902 MB: refused, nothing
    launched, outputs untouched."""
    plan = flce.flce_plan(65536, 2048, 124160, wl.DTYPE_BF16)
    assert plan.ws_bytes > flce.FLCE_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    T, d, V = 65536, 2048, 124160
    H = torch.zeros((T, d), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((V, d), dtype=torch.bfloat16, device=dev)
    y = torch.zeros(T, dtype=torch.int64, device=dev)
    loss = torch.full((T,), 3.0, device=dev)
    lse = torch.full((T,), 3.0, device=dev)
    dH = torch.zeros((T, d), dtype=torch.bfloat16, device=dev)
    dW = torch.full((V, d), 3.0, device=dev)
    with pytest.raises(flce.FlceError) as e:
        flce.flce_forward_backward_scratch(plan, H, W, y, wl.IGNORE_INDEX, "sum", 1.0, loss, lse,
                                           None, dH, dW)
    assert e.value.status == flce.FLCE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(loss == 3.0).item() and torch.all(dW == 3.0).item()
