"""CPU oracle for fused linear cross-entropy -- TEST INFRASTRUCTURE ONLY.

This module is the plain, slow, obviously-correct definition that the GPU
library is checked against.  It is imported only by the test suite, by the
smoke check and by the benchmark's CPU-baseline leg; the library itself never
imports, links or calls it, and it shares no code with the library.

Everything is computed in float64 with numpy from the given inputs (bf16
inputs are widened exactly; products of bf16 values are exact in float64).
The logits are materialised, chunk by chunk over token rows, exactly the
thing the fused method avoids; the method reaches the same result up to
rounding order.

Source: "Long-Sequence MoE RL Training: From First Principles to MI300X",
section 3 ("Linear cross-entropy"): logits Z = H W^T over [tokens x vocab],
reduced through softmax to one cross-entropy value per token, and the only
quantity the backward needs is dZ = softmax(Z) - onehot(target), which is
contracted into dW^T and dH.  The same section names the numerically stable
running-max log-sum-exp; here the plain definition (global row max, then
log-sum-exp) is used.

Readings where the pages are silent (each also listed in the design notes):
  * ignore_index rows: lse is still computed (it does not depend on the
    target); their loss, dZ row and dH row are zero.
  * targets outside [0, V) other than ignore_index are rejected (ValueError).
  * loss is always the unscaled per-token value; `scale` applies only to the
    reduced loss; the backward scalar `grad_scale` multiplies dZ.
  * no bias, soft-capping, temperature, label smoothing or z-loss.

Pinning (tests/test_oracle.py): closed form at W = 0, the V = 1 and V = 2
cases, equal W rows, translation invariance, dZ rows summing to zero, central
finite differences of the loss against the analytic gradients, and torch's
own float64 cross_entropy on the CPU.  No function here is unpinned.
"""
from __future__ import annotations

import math

import numpy as np

IGNORE_INDEX = -100


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _check_targets(target: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    """Returns the boolean mask of valid (non-ignored) rows; rejects bad ids."""
    target = np.asarray(target, dtype=np.int64)
    valid = target != ignore_index
    bad = valid & ((target < 0) | (target >= V))
    if bad.any():
        raise ValueError("target id outside [0, V) that is not ignore_index")
    return valid


def logits(H, W) -> np.ndarray:
    """Z = H W^T, [tokens x vocab] (section 3 of the first page)."""
    return _f64(H) @ _f64(W).T


def log_sum_exp_rows(Z: np.ndarray) -> np.ndarray:
    """lse_i = M_i + ln sum_j exp(Z_ij - M_i) with M_i = max_j Z_ij.

    The row max makes every exponent <= 0, the stabilisation section 3 and
    section 8 of the first page call load-bearing."""
    M = Z.max(axis=1)
    return M + np.log(np.exp(Z - M[:, None]).sum(axis=1))


def grad_logits(Z: np.ndarray, lse: np.ndarray, target: np.ndarray, valid: np.ndarray,
                grad_scale: float) -> np.ndarray:
    """dZ = g * (softmax(Z) - onehot(target)) for valid rows, 0 for ignored rows.

    softmax(Z)_ij = exp(Z_ij - lse_i) (section 3 of the first page)."""
    P = np.exp(Z - lse[:, None])
    rows = np.nonzero(valid)[0]
    P[rows, target[rows]] -= 1.0
    P[~valid] = 0.0
    return grad_scale * P


def forward(H, W, target, ignore_index: int = IGNORE_INDEX, row_chunk: int = 1024):
    """Per-token loss and lse.

    loss_i = lse_i - Z_{i, target_i} = -log softmax(Z_i)[target_i] for valid
    rows, 0 for ignored rows.  Returns (loss [T], lse [T]) in float64."""
    H = _f64(H)
    W = _f64(W)
    target = np.asarray(target, dtype=np.int64)
    T, V = H.shape[0], W.shape[0]
    valid = _check_targets(target, V, ignore_index)
    loss = np.zeros(T)
    lse = np.zeros(T)
    for r0 in range(0, T, row_chunk):
        r1 = min(T, r0 + row_chunk)
        Z = logits(H[r0:r1], W)
        lse[r0:r1] = log_sum_exp_rows(Z)
        v = valid[r0:r1]
        idx = np.nonzero(v)[0]
        zt = Z[idx, target[r0:r1][idx]]
        loss[r0 + idx] = lse[r0 + idx] - zt
    return loss, lse


def forward_backward(H, W, target, ignore_index: int = IGNORE_INDEX, grad_scale: float = 1.0,
                     row_chunk: int = 512, need_dW: bool = True, progress=None):
    """loss, lse, dH = dZ W and dW = dZ^T H (the page writes dW^T = H^T dZ).

    Each row chunk materialises its slice of Z once and uses it for all
    outputs.  Returns (loss [T], lse [T], dH [T,d], dW [V,d] or None)."""
    H = _f64(H)
    W = _f64(W)
    target = np.asarray(target, dtype=np.int64)
    T, d = H.shape
    V = W.shape[0]
    valid = _check_targets(target, V, ignore_index)
    loss = np.zeros(T)
    lse = np.zeros(T)
    dH = np.zeros((T, d))
    dW = np.zeros((V, d)) if need_dW else None
    for r0 in range(0, T, row_chunk):
        r1 = min(T, r0 + row_chunk)
        Z = logits(H[r0:r1], W)
        l = log_sum_exp_rows(Z)
        lse[r0:r1] = l
        v = valid[r0:r1]
        tg = target[r0:r1]
        idx = np.nonzero(v)[0]
        loss[r0 + idx] = l[idx] - Z[idx, tg[idx]]
        dZ = grad_logits(Z, l, tg, v, grad_scale)
        del Z
        dH[r0:r1] = dZ @ W
        if need_dW:
            dW += dZ.T @ H[r0:r1]
        if progress is not None:
            progress(r1, T)
    return loss, lse, dH, dW


def backward(H, W, target, ignore_index: int = IGNORE_INDEX, grad_scale: float = 1.0,
             row_chunk: int = 512):
    """(dH, dW) of grad_scale * sum_i loss_i."""
    _, _, dH, dW = forward_backward(H, W, target, ignore_index, grad_scale, row_chunk)
    return dH, dW


def reduced_loss(loss: np.ndarray, scale: float) -> float:
    """scale * sum_i loss_i (scale = 1/N gives the mean), summed exactly."""
    return float(scale) * math.fsum(float(x) for x in np.asarray(loss, dtype=np.float64))


def rows_forward_dH(H, W, target, rows, ignore_index: int = IGNORE_INDEX,
                    grad_scale: float = 1.0):
    """loss, lse and dH restricted to the given token rows.

    Every one of these depends only on its own row of H (and all of W), so a
    sample of rows can be checked at any T.  Returns (loss, lse, dH) for the
    rows, in the order given."""
    rows = np.asarray(rows, dtype=np.int64)
    loss, lse, dH, _ = forward_backward(_f64(H[rows]), W, np.asarray(target)[rows],
                                        ignore_index, grad_scale, need_dW=False)
    return loss, lse, dH
