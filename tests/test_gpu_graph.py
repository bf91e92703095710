"""HIP graph capture of the library's calls.

Every call is kernel launches on the caller's stream (no memset, copy,
allocation or host synchronisation), so a forward + backward, or the fused
call with its device-side mean, can be captured once and replayed.  Each
test replays several times, with eager library work and synchronisations in
between, and checks every replay bit for bit against the eager result (the
library is deterministic), plus the eager result against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import compare, device_inputs, log

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


def _np(t):
    return t.float().cpu().numpy()


def _bit_equal(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.bfloat16 else a.view(torch.int16),
                       b.view(torch.uint8) if b.dtype != torch.bfloat16 else b.view(torch.int16))


def _capture(fn):
    """Captures fn() into a graph after one warm-up on a side stream (the
    pattern torch documents for capture)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_forward_backward_graph_replays(dtype):
    import linear_cross_entropy_flce_amd as flce
    T, d, V = 700, 136, 5003
    log(f"graph fwd+bwd T={T} d={d} V={V} {dtype}")
    inp = wl.make_inputs(T, d, V, dtype, seed=61, sigma_w=0.4, ignore_frac=0.2)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(T, d, V, dtype)
    dev = W.device
    ws = flce.workspace(plan, dev)
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    red = torch.empty(1, dtype=torch.float32, device=dev)
    dH = torch.empty((T, d), dtype=H.dtype, device=dev)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    g_scale = 1.0 / T

    def step():
        flce.flce_forward(plan, H, W, y, IGN, g_scale, loss=loss, lse=lse, loss_reduced=red, ws=ws)
        flce.flce_backward(plan, H, W, y, lse, IGN, g_scale, dH=dH, dW=dW, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (loss, lse, red, dH, dW)]
    ref_l, ref_s, ref_h, ref_w = oracle.forward_backward(inp.H_f32(), inp.W_f32(), inp.y, IGN,
                                                         g_scale)
    compare(dict(loss=_np(loss), lse=_np(lse), dH=_np(dH), dW=_np(dW)),
            dict(loss=ref_l, lse=ref_s, dH=ref_h, dW=ref_w), dtype)

    graph = _capture(step)
    # other eager work on different inputs between the replays
    other = wl.make_inputs(T, d, V, dtype, seed=62, sigma_w=0.4)
    Ho, Wo, yo = device_inputs(other)
    for rep in range(4):
        for t in (loss, lse, red, dW):
            t.fill_(float("nan"))
        dH.fill_(float("nan"))
        flce.flce_forward(plan, Ho, Wo, yo, IGN, 1.0, ws=flce.workspace(plan, dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("loss", "lse", "reduced", "dH", "dW"), (loss, lse, red, dH, dW),
                              eager):
            assert _bit_equal(a, b), f"replay {rep}: {name} differs from the eager result"
    log("  4 replays bit-identical")


def test_fused_mean_valid_graph_replays():
    """The fused call's device-side valid count and gradient scale live in
    the workspace and are rewritten by every replay."""
    import linear_cross_entropy_flce_amd as flce
    T, d, V = 1100, 96, 3000
    dtype = wl.DTYPE_BF16
    inp = wl.make_inputs(T, d, V, dtype, seed=63, sigma_w=0.4, ignore_frac=0.3)
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(T, d, V, dtype)
    dev = W.device
    ws = flce.workspace(plan, dev)
    outs = {}

    def step():
        outs.update(flce.flce_forward_backward(plan, H, W, y, IGN, "mean_valid", 1.0, ws=ws,
                                               **{k: v for k, v in outs.items()}))

    step()
    torch.cuda.synchronize()
    names = sorted(k for k, v in outs.items() if isinstance(v, torch.Tensor))
    eager = {k: outs[k].clone() for k in names}
    n_valid = int((inp.y != IGN).sum())
    ref_l, ref_s, ref_h, ref_w = oracle.forward_backward(inp.H_f32(), inp.W_f32(), inp.y, IGN,
                                                         1.0 / n_valid)
    compare(dict(loss=_np(outs["loss"]), lse=_np(outs["lse"]), dH=_np(outs["dH"]),
                 dW=_np(outs["dW"])), dict(loss=ref_l, lse=ref_s, dH=ref_h, dW=ref_w), dtype)

    graph = _capture(step)
    for rep in range(3):
        for k in names:
            if outs[k].is_floating_point():
                outs[k].fill_(float("nan"))
        # eager work between replays: an unrelated fused call on its own workspace
        flce.flce_forward_backward(plan, H, W, y, IGN, "sum", 2.0, ws=flce.workspace(plan, dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in names:
            assert _bit_equal(outs[k], eager[k]), f"replay {rep}: {k} differs from the eager result"
    log("  3 replays bit-identical")
