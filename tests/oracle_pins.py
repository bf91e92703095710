"""Pins that tie the CPU oracle to facts other than its own code.

Each pin takes the oracle module as an argument so that the mutation test
can run the same pins against deliberately broken copies of the oracle.
Every pin compares against something the pages or mathematics fix:
closed forms, invariants, finite differences, or torch's own float64
cross-entropy and autograd (an independent library implementation).
"""
from __future__ import annotations

import math

import numpy as np

IGN = -100


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny(seed, T=6, d=5, V=7, sigma_w=0.5, n_ignored=1):
    g = _rng(seed)
    H = g.standard_normal((T, d))
    W = sigma_w * g.standard_normal((V, d))
    y = g.integers(0, V, T)
    y[:n_ignored] = IGN
    return H, W, y


def pin_hand_example(orc):
    """T=1, d=1, V=2, h=1, W=[0, ln 3]: Z=[0, ln 3], softmax=[1/4, 3/4].

    target 0: loss = ln 4, dZ = [-3/4, 3/4], dH = (3/4) ln 3, dW = [-3/4, 3/4]."""
    H = np.array([[1.0]])
    W = np.array([[0.0], [math.log(3.0)]])
    y = np.array([0])
    loss, lse, dH, dW = orc.forward_backward(H, W, y, IGN, 1.0)
    assert abs(loss[0] - math.log(4.0)) < 1e-14
    assert abs(lse[0] - math.log(4.0)) < 1e-14
    assert abs(dH[0, 0] - 0.75 * math.log(3.0)) < 1e-14
    assert np.allclose(dW[:, 0], [-0.75, 0.75], atol=1e-15, rtol=0)
    # target 1: loss = ln 4 - ln 3 = ln(4/3), dZ = [1/4, -1/4], dH = -(1/4) ln 3
    loss, lse, dH, dW = orc.forward_backward(H, W, np.array([1]), IGN, 2.0)
    assert abs(loss[0] - math.log(4.0 / 3.0)) < 1e-14
    assert abs(dH[0, 0] + 2.0 * 0.25 * math.log(3.0)) < 1e-14
    assert np.allclose(dW[:, 0], [0.5, -0.5], atol=1e-15, rtol=0)


def pin_zero_weights(orc):
    """W = 0: z = 0, lse = ln V, loss = ln V on valid rows, dH = 0 and
    dW_j = g * sum over valid i of (1/V - [y_i = j]) h_i."""
    T, d, V, g = 9, 4, 11, 0.37
    H, _, y = _tiny(1, T, d, V, n_ignored=2)
    W = np.zeros((V, d))
    loss, lse, dH, dW = orc.forward_backward(H, W, y, IGN, g)
    assert np.allclose(lse, math.log(V), atol=1e-14, rtol=0)
    valid = y != IGN
    assert np.allclose(loss[valid], math.log(V), atol=1e-14, rtol=0)
    assert np.all(loss[~valid] == 0.0)
    assert np.all(dH == 0.0)
    expect = np.zeros((V, d))
    for i in range(T):
        if y[i] == IGN:
            continue
        for j in range(V):
            expect[j] += g * ((1.0 / V) - (1.0 if y[i] == j else 0.0)) * H[i]
    assert np.allclose(dW, expect, atol=1e-13, rtol=0)
    f_loss, f_lse = orc.forward(H, W, y, IGN)
    assert np.allclose(f_loss, loss, atol=1e-14, rtol=0)
    assert np.allclose(f_lse, lse, atol=1e-14, rtol=0)


def pin_single_class(orc):
    """V = 1: the only class has probability 1, so loss = 0 and dZ = 0."""
    H, W, y = _tiny(2, 5, 3, 1, n_ignored=0)
    y[:] = 0
    loss, lse, dH, dW = orc.forward_backward(H, W, y, IGN, 1.0)
    assert np.allclose(loss, 0.0, atol=1e-14)
    assert np.allclose(lse, H @ W[0], atol=1e-13, rtol=0)
    assert np.allclose(dH, 0.0, atol=1e-14)
    assert np.allclose(dW, 0.0, atol=1e-14)


def _softplus(x):
    return max(x, 0.0) + math.log1p(math.exp(-abs(x)))


def _sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


def pin_two_classes(orc):
    """V = 2 is logistic regression: loss = softplus(z_other - z_target) and
    dZ_other = g * sigmoid(z_other - z_target) = -dZ_target."""
    T, d, g = 7, 3, 0.5
    H, W, y = _tiny(3, T, d, 2, sigma_w=1.5, n_ignored=1)
    loss, lse, dH, dW = orc.forward_backward(H, W, y, IGN, g)
    eH = np.zeros((T, d))
    eW = np.zeros((2, d))
    for i in range(T):
        if y[i] == IGN:
            assert loss[i] == 0.0
            continue
        t, o = int(y[i]), 1 - int(y[i])
        zt = sum(H[i, k] * W[t, k] for k in range(d))
        zo = sum(H[i, k] * W[o, k] for k in range(d))
        assert abs(loss[i] - _softplus(zo - zt)) < 1e-13
        s = g * _sigmoid(zo - zt)
        eH[i] = s * (W[o] - W[t])
        eW[o] += s * H[i]
        eW[t] -= s * H[i]
    assert np.allclose(dH, eH, atol=1e-13, rtol=0)
    assert np.allclose(dW, eW, atol=1e-13, rtol=0)


def pin_equal_rows(orc):
    """All rows of W equal: every class is equally likely, loss = ln V, dH = 0."""
    T, d, V = 6, 4, 13
    H, W, y = _tiny(4, T, d, V, n_ignored=0)
    W[:] = W[0]
    loss, lse, dH, dW = orc.forward_backward(H, W, y, IGN, 1.0)
    assert np.allclose(loss, math.log(V), atol=1e-12, rtol=0)
    assert np.allclose(dH, 0.0, atol=1e-12)


def pin_translation(orc, shift=None):
    """w_j -> w_j + c for every j shifts lse_i by h_i . c and leaves loss, dH
    and dW unchanged.  With h . c near 1000 the shifted logits overflow exp()
    in float64 unless the row maximum is subtracted first."""
    T, d, V, g = 8, 6, 9, 0.8
    H, W, y = _tiny(5, T, d, V, n_ignored=2)
    c = np.full(d, 1.0)
    hc = H @ c
    # scale c so that the largest |h.c| is 1000: exp(1000) overflows float64
    c = c * (1000.0 / np.abs(hc).max()) if shift is None else c * shift
    loss0, lse0, dH0, dW0 = orc.forward_backward(H, W, y, IGN, g)
    loss1, lse1, dH1, dW1 = orc.forward_backward(H, W + c, y, IGN, g)
    assert np.all(np.isfinite(lse1)) and np.all(np.isfinite(loss1))
    assert np.allclose(lse1, lse0 + H @ c, atol=1e-9, rtol=0)
    assert np.allclose(loss1, loss0, atol=1e-9, rtol=0)
    assert np.allclose(dH1, dH0, atol=1e-9, rtol=0)
    assert np.allclose(dW1, dW0, atol=1e-9, rtol=0)


def pin_rows_sum_to_zero(orc):
    """Each dZ row sums to 0 (softmax sums to 1, onehot sums to 1), hence the
    rows of dW sum to the zero vector."""
    T, d, V, g = 10, 5, 17, 1.3
    H, W, y = _tiny(6, T, d, V, sigma_w=2.0, n_ignored=3)
    _, _, _, dW = orc.forward_backward(H, W, y, IGN, g)
    assert np.allclose(dW.sum(axis=0), 0.0, atol=1e-12)
    Z = orc.logits(H, W)
    lse = orc.log_sum_exp_rows(Z)
    dZ = orc.grad_logits(Z, lse, y, y != IGN, g)
    assert np.allclose(dZ.sum(axis=1), 0.0, atol=1e-14)


def pin_finite_differences(orc):
    """Central differences of g * sum_i loss_i in H and W match dH and dW."""
    T, d, V, g, eps = 3, 4, 5, 0.7, 1e-6
    H, W, y = _tiny(7, T, d, V, sigma_w=0.8, n_ignored=1)
    _, _, dH, dW = orc.forward_backward(H, W, y, IGN, g)

    def L(Hx, Wx):
        loss, _ = orc.forward(Hx, Wx, y, IGN)
        return g * math.fsum(loss)

    nH = np.zeros_like(H)
    for i in range(T):
        for k in range(d):
            Hp, Hm = H.copy(), H.copy()
            Hp[i, k] += eps
            Hm[i, k] -= eps
            nH[i, k] = (L(Hp, W) - L(Hm, W)) / (2 * eps)
    nW = np.zeros_like(W)
    for j in range(V):
        for k in range(d):
            Wp, Wm = W.copy(), W.copy()
            Wp[j, k] += eps
            Wm[j, k] -= eps
            nW[j, k] = (L(H, Wp) - L(H, Wm)) / (2 * eps)
    assert np.allclose(dH, nH, atol=1e-8, rtol=1e-6)
    assert np.allclose(dW, nW, atol=1e-8, rtol=1e-6)


def pin_torch_library(orc, T=37, d=16, V=101, seed=8):
    """torch.nn.functional.cross_entropy and autograd in float64 on the CPU
    (an independent library implementation) give the same loss, lse, dH, dW."""
    import torch
    H, W, y = _tiny(seed, T, d, V, sigma_w=0.7, n_ignored=5)
    g = 0.25
    loss, lse, dH, dW = orc.forward_backward(H, W, y, IGN, g, row_chunk=8)
    tH = torch.tensor(H, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    ty = torch.tensor(y, dtype=torch.int64)
    Z = tH @ tW.T
    tl = torch.nn.functional.cross_entropy(Z, ty, reduction="none", ignore_index=IGN)
    (g * tl.sum()).backward()
    assert np.allclose(loss, tl.detach().numpy(), atol=1e-12, rtol=0)
    assert np.allclose(lse, torch.logsumexp(Z.detach(), dim=1).numpy(), atol=1e-12, rtol=0)
    assert np.allclose(dH, tH.grad.numpy(), atol=1e-12, rtol=0)
    assert np.allclose(dW, tW.grad.numpy(), atol=1e-12, rtol=0)


def pin_sampled_rows(orc):
    """rows_forward_dH on a row subset equals the same rows of the full result."""
    H, W, y = _tiny(9, 20, 6, 12, n_ignored=4)
    loss, lse, dH, _ = orc.forward_backward(H, W, y, IGN, 0.3)
    rows = np.array([0, 3, 4, 11, 19])
    l2, s2, h2 = orc.rows_forward_dH(H, W, y, rows, IGN, 0.3)
    assert np.allclose(l2, loss[rows], atol=1e-14, rtol=0)
    assert np.allclose(s2, lse[rows], atol=1e-14, rtol=0)
    assert np.allclose(h2, dH[rows], atol=1e-14, rtol=0)


def pin_reduced_loss(orc):
    """scale * sum: a mean with scale 1/N equals the arithmetic mean."""
    vals = np.array([0.5, 1.25, 2.0, 0.25])
    assert orc.reduced_loss(vals, 1.0 / 4) == 1.0
    assert orc.reduced_loss(vals, 2.0) == 8.0


def pin_rejects_bad_target(orc):
    """A target outside [0, V) that is not ignore_index is rejected."""
    H, W, y = _tiny(10, 4, 3, 5, n_ignored=0)
    y[2] = 5
    try:
        orc.forward(H, W, y, IGN)
    except ValueError:
        return
    raise AssertionError("out-of-range target was accepted")


def pin_backward(orc):
    """backward() returns (dH, dW) of g * sum_i loss_i, in that order: checked
    against central differences of the loss (T != V != d, so a swapped pair
    fails on shape alone), against the W = 0 closed form of dW, and for its
    linearity in g (dZ = g (softmax - onehot), first page section 3)."""
    T, d, V, g, eps = 4, 3, 6, 0.6, 1e-6
    H, W, y = _tiny(11, T, d, V, sigma_w=0.9, n_ignored=1)
    dH, dW = orc.backward(H, W, y, IGN, g)
    assert dH.shape == (T, d) and dW.shape == (V, d)

    def L(Hx, Wx):
        loss, _ = orc.forward(Hx, Wx, y, IGN)
        return g * math.fsum(loss)

    for i in range(T):
        for k in range(d):
            Hp, Hm = H.copy(), H.copy()
            Hp[i, k] += eps
            Hm[i, k] -= eps
            assert abs(dH[i, k] - (L(Hp, W) - L(Hm, W)) / (2 * eps)) < 1e-7
    for j in range(V):
        for k in range(d):
            Wp, Wm = W.copy(), W.copy()
            Wp[j, k] += eps
            Wm[j, k] -= eps
            assert abs(dW[j, k] - (L(H, Wp) - L(H, Wm)) / (2 * eps)) < 1e-7
    # linear in g: twice the scale, twice the gradients
    dH2, dW2 = orc.backward(H, W, y, IGN, 2 * g)
    assert np.allclose(dH2, 2 * dH, atol=1e-14, rtol=1e-12)
    assert np.allclose(dW2, 2 * dW, atol=1e-14, rtol=1e-12)
    # W = 0: dH = 0 and dW_j = g * sum over valid i of (1/V - [y_i = j]) h_i
    dH0, dW0 = orc.backward(H, np.zeros((V, d)), y, IGN, g)
    assert np.all(dH0 == 0.0)
    for j in range(V):
        e = sum(g * ((1.0 / V) - (1.0 if y[i] == j else 0.0)) * H[i]
                for i in range(T) if y[i] != IGN)
        assert np.allclose(dW0[j], e, atol=1e-13, rtol=0)


ALL_PINS = [pin_hand_example, pin_zero_weights, pin_single_class, pin_two_classes,
            pin_equal_rows, pin_translation, pin_rows_sum_to_zero, pin_finite_differences,
            pin_torch_library, pin_sampled_rows, pin_reduced_loss, pin_rejects_bad_target,
            pin_backward]
