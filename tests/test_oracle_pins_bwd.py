"""Pins of the oracle's backward definitions (vector-Jacobian products).

Each backward is checked against central finite differences of the scalar
L = sum(dy * forward(inputs)) computed with the oracle's own forward in double
("NexusGrad", Verified VJP Operators: df/dx ~ (f(x+e) - f(x-e)) / 2e), against
torch CPU float64 autograd, and against invariants (softmax and LayerNorm
input gradients sum to zero over a row).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(777)
EPS_FD = 1e-6


def fd(fun, a, idx):
    ap, am = a.copy(), a.copy()
    ap[idx] += EPS_FD
    am[idx] -= EPS_FD
    return (fun(ap) - fun(am)) / (2 * EPS_FD)


# ------------------------------------------------------------- softmax

@pytest.mark.parametrize("C", [1, 2, 3, 5, 8])
def test_softmax_bwd_finite_differences(C):
    x = RNG.normal(0, 2, size=(3, C))
    dy = RNG.normal(0, 1, size=(3, C))
    dx = oracle.softmax_bwd(oracle.softmax(x), dy)
    loss = lambda xx: float(np.sum(dy * oracle.softmax(xx)))
    for r in range(3):
        for j in range(C):
            assert abs(fd(loss, x, (r, j)) - dx[r, j]) <= 1e-8
    assert np.max(np.abs(dx.sum(1))) <= 1e-15 * 8


def test_softmax_bwd_torch():
    x = RNG.normal(0, 4, size=(16, 1000))
    dy = RNG.normal(0, 1, size=(16, 1000))
    xt = torch.from_numpy(x).requires_grad_(True)
    torch.softmax(xt, 1).backward(torch.from_numpy(dy))
    dx = oracle.softmax_bwd(oracle.softmax(x), dy)
    assert np.max(np.abs(dx - xt.grad.numpy())) <= 1e-15 * 4
    # stored fp32 inputs decode exactly: same result as their values in double
    p32, dy32 = oracle.softmax(x).astype(np.float32), dy.astype(np.float32)
    assert np.array_equal(oracle.softmax_bwd(p32, dy32),
                          oracle.softmax_bwd(p32.astype(np.float64), dy32.astype(np.float64)))


# ------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("C", [1, 2, 3, 6])
def test_rmsnorm_bwd_finite_differences(C):
    h = RNG.normal(0, 1, size=(3, C))
    w = RNG.uniform(0.5, 1.5, size=C)
    dy = RNG.normal(0, 1, size=(3, C))
    eps = np.float32(1e-3)
    dh, dw = oracle.rmsnorm_bwd(h, dy, w, eps)
    z = np.zeros_like(h)

    def loss_h(hh):
        return float(np.sum(dy * oracle.add_rmsnorm(hh, z, w, eps)[0]))

    def loss_w(ww):
        return float(np.sum(dy * oracle.add_rmsnorm(h, z, ww, eps)[0]))

    for r in range(3):
        for j in range(C):
            assert abs(fd(loss_h, h, (r, j)) - dh[r, j]) <= 1e-8
    for j in range(C):
        assert abs(fd(loss_w, w, (j,)) - dw[j]) <= 1e-8


@pytest.mark.parametrize("C", [1, 4])
def test_add_rmsnorm_bwd_residual_gradient(C):
    """With h = x + residual also an output, L = sum(dy * y) + sum(dres * h):
    dL/dx and dL/dresidual are both the returned dh (finite differences in x
    and in residual separately)."""
    x = RNG.normal(0, 1, size=(3, C))
    res = RNG.normal(0, 1, size=(3, C))
    w = RNG.uniform(0.5, 1.5, size=C)
    dy = RNG.normal(0, 1, size=(3, C))
    dres = RNG.normal(0, 1, size=(3, C))
    eps = np.float32(1e-3)
    dh, dw = oracle.rmsnorm_bwd(x + res, dy, w, eps, dres=dres)
    _, dw0 = oracle.rmsnorm_bwd(x + res, dy, w, eps)
    assert np.array_equal(dw, dw0)  # dres does not reach the weight

    def loss(xx, rr):
        y, h, _ = oracle.add_rmsnorm(xx, rr, w, eps)
        return float(np.sum(dy * y) + np.sum(dres * h))

    for r in range(3):
        for j in range(C):
            assert abs(fd(lambda xx: loss(xx, res), x, (r, j)) - dh[r, j]) <= 1e-8
            assert abs(fd(lambda rr: loss(x, rr), res, (r, j)) - dh[r, j]) <= 1e-8


def test_rmsnorm_bwd_torch():
    h = RNG.normal(0, 1, size=(12, 2048))
    w = RNG.uniform(0.8, 1.2, size=2048)
    dy = RNG.normal(0, 1, size=(12, 2048))
    eps = float(np.float32(1e-6))
    ht = torch.from_numpy(h).requires_grad_(True)
    wt = torch.from_numpy(w).requires_grad_(True)
    F.rms_norm(ht, (2048,), wt, eps=eps).backward(torch.from_numpy(dy))
    dh, dw = oracle.rmsnorm_bwd(h, dy, w, np.float32(1e-6))
    assert np.max(np.abs(dh - ht.grad.numpy())) <= 1e-12
    assert np.max(np.abs(dw - wt.grad.numpy())) <= 1e-11


# ------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("C", [2, 3, 4, 7])
def test_layernorm_bwd_finite_differences(C):
    x = RNG.normal(3, 2, size=(3, C))
    g = RNG.uniform(0.5, 1.5, size=C)
    b = RNG.normal(0, 0.3, size=C)
    dy = RNG.normal(0, 1, size=(3, C))
    eps = np.float32(1e-3)
    _, mean, rstd = oracle.layernorm(x, g, b, eps)
    dx, dg, db = oracle.layernorm_bwd(x, dy, g, mean, rstd)
    loss_x = lambda xx: float(np.sum(dy * oracle.layernorm(xx, g, b, eps)[0]))
    loss_g = lambda gg: float(np.sum(dy * oracle.layernorm(x, gg, b, eps)[0]))
    loss_b = lambda bb: float(np.sum(dy * oracle.layernorm(x, g, bb, eps)[0]))
    for r in range(3):
        for j in range(C):
            assert abs(fd(loss_x, x, (r, j)) - dx[r, j]) <= 1e-7
    for j in range(C):
        assert abs(fd(loss_g, g, (j,)) - dg[j]) <= 1e-7
        assert abs(fd(loss_b, b, (j,)) - db[j]) <= 1e-7
    assert np.max(np.abs(dx.sum(1))) <= 1e-12


def test_layernorm_bwd_torch():
    x = RNG.normal(3, 2, size=(10, 1024))
    g = RNG.uniform(0.5, 1.5, size=1024)
    b = RNG.normal(0, 0.3, size=1024)
    dy = RNG.normal(0, 1, size=(10, 1024))
    eps = float(np.float32(1e-5))
    xt = torch.from_numpy(x).requires_grad_(True)
    gt = torch.from_numpy(g).requires_grad_(True)
    bt = torch.from_numpy(b).requires_grad_(True)
    F.layer_norm(xt, (1024,), gt, bt, eps=eps).backward(torch.from_numpy(dy))
    _, mean, rstd = oracle.layernorm(x, g, b, np.float32(1e-5))
    dx, dg, db = oracle.layernorm_bwd(x, dy, g, mean, rstd)
    assert np.max(np.abs(dx - xt.grad.numpy())) <= 1e-12
    assert np.max(np.abs(dg - gt.grad.numpy())) <= 1e-11
    assert np.max(np.abs(db - bt.grad.numpy())) <= 1e-11
