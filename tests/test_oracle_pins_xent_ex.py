"""Pins of the oracle's cross-entropy with options (ignore_index, label
smoothing, sum / mean reduction, gradient scale).

The gradient is checked against central finite differences of the oracle's
own loss in double ("NexusGrad", Verified VJP Operators), the losses and
gradients against torch CPU float64 `cross_entropy` with autograd, and both
against closed forms (uniform logits) and the plain cross-entropy without
options.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(4242)
EPS_FD = 1e-6


@pytest.mark.parametrize("C", [2, 3, 6])
@pytest.mark.parametrize("eps", [0.0, 0.1, 0.3])
def test_gradient_is_derivative_of_summed_loss(C, eps):
    x = RNG.normal(0, 2, size=(3, C))
    y = RNG.integers(0, C, size=3).astype(np.int32)
    _, g, _, tot = oracle.softmax_xent_ex(x, y, label_smoothing=eps, reduction="sum")
    for r in range(3):
        for j in range(C):
            xp, xm = x.copy(), x.copy()
            xp[r, j] += EPS_FD
            xm[r, j] -= EPS_FD
            fp = oracle.softmax_xent_ex(xp, y, label_smoothing=eps, reduction="sum")[3]
            fm = oracle.softmax_xent_ex(xm, y, label_smoothing=eps, reduction="sum")[3]
            assert abs((fp - fm) / (2 * EPS_FD) - g[r, j]) <= 1e-8


def test_mean_with_ignored_rows_gradient_is_derivative():
    C = 5
    x = RNG.normal(0, 1.5, size=(6, C))
    y = np.array([1, -100, 4, 0, -100, 2], np.int32)
    kw = dict(ignore_index=-100, label_smoothing=0.2, reduction="mean", grad_scale=0.75)
    loss, g, _, tot = oracle.softmax_xent_ex(x, y, **kw)
    assert np.all(loss[[1, 4]] == 0) and np.all(g[[1, 4]] == 0)
    assert tot == pytest.approx(loss.sum() / 4, rel=1e-15)
    for r in range(6):
        for j in range(C):
            xp, xm = x.copy(), x.copy()
            xp[r, j] += EPS_FD
            xm[r, j] -= EPS_FD
            d = (oracle.softmax_xent_ex(xp, y, **kw)[3] - oracle.softmax_xent_ex(xm, y, **kw)[3])
            assert abs(0.75 * d / (2 * EPS_FD) - g[r, j]) <= 1e-8


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
@pytest.mark.parametrize("eps", [0.0, 0.1])
def test_torch_float64(reduction, eps):
    R, C = 40, 1000
    x = RNG.normal(0, 2, size=(R, C))
    y = RNG.integers(0, C, size=R).astype(np.int32)
    y[::7] = -100
    scale = 0.5
    loss, g, _, tot = oracle.softmax_xent_ex(x, y, ignore_index=-100, label_smoothing=eps,
                                             reduction=reduction, grad_scale=scale)
    xt = torch.from_numpy(x).requires_grad_(True)
    out = F.cross_entropy(xt, torch.from_numpy(y.astype(np.int64)), ignore_index=-100,
                          label_smoothing=eps, reduction=reduction)
    if reduction == "none":
        assert np.max(np.abs(loss - out.detach().numpy())) <= 1e-12
        out.backward(torch.full((R,), scale, dtype=torch.float64))
    else:
        assert abs(tot - float(out.detach())) <= 1e-12 * max(1.0, abs(tot))
        (scale * out).backward()
    assert np.max(np.abs(g - xt.grad.numpy())) <= 1e-14


@pytest.mark.parametrize("eps", [0.0, 0.05, 1.0])
def test_uniform_logits_closed_form(eps):
    C = 16
    x = np.full((3, C), 2.5)
    y = np.array([0, 7, 15], np.int32)
    loss, g, _, _ = oracle.softmax_xent_ex(x, y, label_smoothing=eps)
    assert np.allclose(loss, np.log(C), rtol=0, atol=1e-14)
    q = np.full((3, C), eps / C)
    q[np.arange(3), y] += 1 - eps
    assert np.allclose(g, 1.0 / C - q, rtol=0, atol=1e-16)


def test_no_options_is_plain_cross_entropy():
    x = RNG.normal(0, 2, size=(8, 300)).astype(np.float32)
    y = RNG.integers(0, 300, size=8).astype(np.int32)
    l0, g0, a0 = oracle.softmax_xent(x, y)
    l1, g1, a1, t = oracle.softmax_xent_ex(x, y)
    assert np.array_equal(a0, a1) and t is None
    assert np.max(np.abs(l0 - l1)) <= 1e-13 * np.max(np.abs(l0))
    assert np.max(np.abs(g0 - g1)) <= 1e-16


def test_invalid_label_and_all_ignored():
    C = 10
    x = RNG.normal(size=(3, C))
    y = np.array([C, -1, 3], np.int32)            # out of range, not the ignore value
    loss, g, _, tot = oracle.softmax_xent_ex(x, y, ignore_index=-100, label_smoothing=0.1,
                                             reduction="sum")
    p = oracle.softmax(x)
    assert np.isnan(loss[0]) and np.isnan(loss[1]) and np.isnan(tot)
    assert np.max(np.abs(g[:2] - (p[:2] - 0.1 / C))) <= 1e-16
    y = np.full(3, -100, np.int32)
    loss, g, _, tot = oracle.softmax_xent_ex(x, y, ignore_index=-100, reduction="mean")
    assert np.all(loss == 0) and np.all(g == 0) and np.isnan(tot)   # 0 / 0, as torch


def test_masked_logits_zero_weight_terms():
    # a -inf logit (masked class) has zero target weight without smoothing:
    # the loss is the plain one and finite; with smoothing it is +inf
    x = np.array([[1.0, -np.inf, 0.5, 2.0]])
    y = np.array([0], np.int32)
    l0, g0, _ = oracle.softmax_xent(x, y)
    l, g, _, _ = oracle.softmax_xent_ex(x, y)
    assert np.isfinite(l[0]) and l[0] == pytest.approx(l0[0], rel=1e-15)
    assert np.array_equal(g, g0) and g[0, 1] == 0.0
    l, _, _, _ = oracle.softmax_xent_ex(x, y, label_smoothing=0.1)
    assert l[0] == np.inf
