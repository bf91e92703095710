"""Helpers shared by the GPU tests: upload seeded inputs, run the library
through its C-ABI binding, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import linear_cross_entropy_flce_amd as flce
import workloads as wl

# Tolerances fixed for this operation: per-token loss and lse absolute error,
# and relative Frobenius error of dH and dW, by input precision.
TOL = {
    wl.DTYPE_BF16: dict(loss=2e-3, grad=1e-2),
    wl.DTYPE_F32: dict(loss=1e-5, grad=1e-5),
}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_inputs(inp: wl.Inputs):
    if inp.dtype == wl.DTYPE_BF16:
        H = torch.from_numpy(inp.H.view(np.int16)).cuda().view(torch.bfloat16)
        W = torch.from_numpy(inp.W.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        H = torch.from_numpy(inp.H).cuda()
        W = torch.from_numpy(inp.W).cuda()
    y = torch.from_numpy(inp.y).cuda()
    return H, W, y


def gather_plan(plan):
    """A copy of the plan whose forward takes the target logit as a gathered
    dot product (pure log-sum-exp sweep)."""
    p = type(plan).from_buffer_copy(plan)
    p.target_logit = flce.FLCE_TARGET_GATHER
    return p


def run_gpu(inp: wl.Inputs, loss_scale=1.0, grad_scale=1.0, cap=0, backward=True, dev=None,
            accumulate_dW=False, dW_init=None, gather=True):
    """One forward (+ backward) through the C-ABI.  Returns numpy results.

    With `gather`, the forward also runs a second time with the target logit
    gathered by index (loss_gather, lse_gather, red_gather)."""
    H, W, y = dev if dev is not None else device_inputs(inp)
    plan = flce.flce_plan(inp.T, inp.d, inp.V, inp.dtype, cap)
    ws = flce.workspace(plan, W.device)
    red = torch.empty(1, dtype=torch.float32, device=W.device)
    loss, lse, _ = flce.flce_forward(plan, H, W, y, inp.ignore_index, loss_scale,
                                     loss_reduced=red, ws=ws)
    out = dict(plan=plan, loss=loss, lse=lse, red=red)
    if gather:
        gred = torch.empty(1, dtype=torch.float32, device=W.device)
        gl, gs, _ = flce.flce_forward(gather_plan(plan), H, W, y, inp.ignore_index, loss_scale,
                                      loss_reduced=gred, ws=ws)
        out.update(loss_gather=gl, lse_gather=gs, red_gather=gred)
    if backward:
        dW = None
        if dW_init is not None:
            dW = torch.from_numpy(dW_init).cuda()
        dH, dW = flce.flce_backward(plan, H, W, y, lse, inp.ignore_index, grad_scale, dW=dW,
                                    accumulate_dW=accumulate_dW, ws=ws)
        out.update(dH=dH, dW=dW)
    torch.cuda.synchronize()
    return {k: (v.float().cpu().numpy() if isinstance(v, torch.Tensor) else v)
            for k, v in out.items()}


def max_abs(a, b, mask=None):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if mask is not None:
        a, b = a[mask], b[mask]
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    d = np.linalg.norm(a - b)
    if nb == 0.0:
        return d
    return float(d / nb)


def logit_tol(dtype, d, zmax):
    """Loss/lse tolerance when the logits reach |z| = zmax: fp32 results carry
    a rounding of about sqrt(d) ulps of |z| (sums of d terms in a kernel's own
    order), which the fixed 1e-5 covers only for moderate logits; the bf16
    tolerance is far above it."""
    return TOL[dtype]["loss"] + (np.sqrt(d) * 2.0 ** -23 * zmax if dtype == wl.DTYPE_F32 else 0.0)


def compare(got, ref, dtype, what=("loss", "lse", "dH", "dW"), rows=None, loss_tol=None,
            grad_tol=None, gather_tol=None):
    """Asserts the tolerances; returns the error figures.

    When `got` holds the gathered-target forward's loss and lse too, they are
    held to the same loss tolerance, widened for fp32 to `gather_tol` if given
    (the gathered fp32 dot product sums in another order than the tile)."""
    tol = dict(TOL[dtype])
    if loss_tol is not None:
        tol["loss"] = loss_tol
    if grad_tol is not None:
        tol["grad"] = grad_tol
    errs = {}
    loss_ref, lse_ref = ref["loss"], ref["lse"]
    if "loss" in what:
        g = got["loss"] if rows is None else got["loss"][rows]
        errs["loss"] = max_abs(g, loss_ref)
        assert errs["loss"] <= tol["loss"], errs
    if "lse" in what:
        g = got["lse"] if rows is None else got["lse"][rows]
        errs["lse"] = max_abs(g, lse_ref)
        assert errs["lse"] <= tol["loss"], errs
    if "dH" in what:
        g = got["dH"] if rows is None else got["dH"][rows]
        errs["dH"] = rel_fro(g, ref["dH"])
        assert errs["dH"] <= tol["grad"], errs
    if "dW" in what:
        errs["dW"] = rel_fro(got["dW"], ref["dW"])
        assert errs["dW"] <= tol["grad"], errs
    if "loss_gather" in got:
        if gather_tol is None and dtype == wl.DTYPE_F32 and np.ndim(got.get("dH")) == 2:
            # |z_t| = |lse - loss|: the gathered fp32 dot product carries about
            # sqrt(d) ulps of it (logit_tol), like any fp32 sum of d products
            zt = np.abs(np.asarray(lse_ref, np.float64) - np.asarray(loss_ref, np.float64))
            zmax = float(max(np.abs(lse_ref).max(initial=0.0), zt.max(initial=0.0)))
            gather_tol = logit_tol(dtype, got["dH"].shape[1], zmax)
        gt = tol["loss"] if gather_tol is None else max(tol["loss"], gather_tol)
        # both forms run the same log-sum-exp arithmetic: identical lse bits
        assert np.array_equal(got["lse_gather"], got["lse"]), "lse differs between the forms"
        for k, r in (("loss", loss_ref), ("lse", lse_ref)):
            if k in what:
                g = got[k + "_gather"] if rows is None else got[k + "_gather"][rows]
                errs[k + "_gather"] = max_abs(g, r)
                assert errs[k + "_gather"] <= gt, errs
    return errs


def run_gpu_shards(inp: wl.Inputs, bounds, loss_scale=1.0, grad_scale=1.0, merge=None,
                   backward=True, dev=None, gather=False):
    """The vocab-parallel path on one GPU: W's rows cut at `bounds` (ascending
    vocab ids, 0 .. V), each shard through flce_forward_shard, the statistics
    stacked as an all-gather would, merged by flce_merge_shards (over the
    shard indices in `merge`, default all in order), then flce_backward_shard
    per shard with the merged lse.  dH is the sum of the shards' partials
    (what the caller's all-reduce does), dW the concatenation of the slices.
    With `gather`, each shard's forward takes its target logits by index."""
    H, W, y = dev if dev is not None else device_inputs(inp)
    V = inp.V
    shards = list(zip(bounds[:-1], bounds[1:]))
    merge = list(range(len(shards))) if merge is None else list(merge)
    plans, stats = [], []
    for (a, b) in shards:
        plan = flce.flce_plan(inp.T, inp.d, b - a, inp.dtype)
        if gather:
            plan = gather_plan(plan)
        ws = flce.workspace(plan, W.device)
        lse_s, zt_s = flce.flce_forward_shard(plan, H, W[a:b], y, a, V, inp.ignore_index, ws=ws)
        plans.append((plan, ws))
        stats.append((lse_s, zt_s))
    lse_all = torch.stack([stats[i][0] for i in merge]).contiguous()
    zt_all = torch.stack([stats[i][1] for i in merge]).contiguous()
    red = torch.empty(1, dtype=torch.float32, device=W.device)
    loss, lse, _ = flce.flce_merge_shards(lse_all, zt_all, y, V, inp.ignore_index, loss_scale,
                                          loss_reduced=red)
    out = dict(loss=loss, lse=lse, red=red,
               lse_shards=torch.stack([s[0] for s in stats]),
               zt_shards=torch.stack([s[1] for s in stats]))
    if backward:
        dH = None
        dWs = []
        for (a, b), (plan, ws) in zip(shards, plans):
            dHp, dWp = flce.flce_backward_shard(plan, H, W[a:b], y, lse, a, V, inp.ignore_index,
                                                grad_scale, ws=ws)
            dH = dHp.float() if dH is None else dH + dHp.float()
            dWs.append(dWp)
        out.update(dH=dH, dW=torch.cat(dWs, 0))
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in out.items()}
