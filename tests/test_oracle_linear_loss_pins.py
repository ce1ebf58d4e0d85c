"""Pins of the generic linear-loss oracle (CPU only).

* central finite differences of the total loss with respect to every entry of
  X and W (autograd-free) for the written-out ``mse_sum``;
* ``W = I`` (V = D): the logits are the inputs, so grad_inputs = 2 (X - Y) and
  grad_weight = 2 (X - Y)^T X;
* the cross-entropy case: with the CE oracle's row function as the loss
  (reduction 'sum'), it reproduces ``oracle.linear_cross_entropy``.
A planted mistake (grad_weight transposed, the gradient's factor 2 dropped) is
caught by the finite differences.
"""
import torch

import oracle
from oracle import generic as oll

torch.set_default_dtype(torch.float64)


def _data(BT=4, D=3, V=5, seed=21):
    g = torch.Generator().manual_seed(seed)
    X = torch.randn(BT, D, generator=g)
    W = torch.randn(V, D, generator=g)
    Y = torch.randn(BT, V, generator=g)
    return X, W, Y


def _fd_error(fn):
    X, W, Y = _data()
    out = fn(X, W, oll.mse_sum, Y)
    h = 1e-6

    def L(XX, WW):
        return oll.linear_loss(XX, WW, oll.mse_sum, Y)["loss"]
    errs, scale = [], 0.0
    for M, key in ((X, "grad_inputs"), (W, "grad_weight")):
        fd = torch.empty_like(M)
        for i in range(M.shape[0]):
            for j in range(M.shape[1]):
                P = M.clone(); P[i, j] += h
                Q = M.clone(); Q[i, j] -= h
                args = (P, W) if key == "grad_inputs" else (X, P)
                argm = (Q, W) if key == "grad_inputs" else (X, Q)
                fd[i, j] = (L(*args) - L(*argm)) / (2 * h)
        errs.append(float((fd - out[key]).abs().max()))
        scale = max(scale, float(fd.abs().max()))
    return max(errs), 1e-8 + 1e-7 * scale


def test_mse_gradients_match_central_differences():
    err, tol = _fd_error(oll.linear_loss)
    assert err <= tol


def test_identity_weight_closed_form():
    X, _, Y = _data(V=3)
    W = torch.eye(3)
    out = oll.linear_loss(X, W, oll.mse_sum, Y)
    assert abs(out["loss"] - float(((X - Y) ** 2).sum())) < 1e-12
    assert torch.allclose(out["grad_inputs"], 2 * (X - Y), atol=1e-14)
    assert torch.allclose(out["grad_weight"], 2 * (X - Y).T @ X, atol=1e-13)


def test_cross_entropy_case_matches_linear_ce_oracle():
    g = torch.Generator().manual_seed(5)
    X = torch.randn(12, 6, generator=g)
    W = torch.randn(9, 6, generator=g) * 0.5
    t = torch.randint(0, 9, (12,), generator=g)
    t[3] = -100

    def ce_sum(Z, tt):
        r = oracle.cross_entropy(Z, tt, -100, "sum", 0.0)
        return r["loss"], r["grad"]
    got = oll.linear_loss(X, W, ce_sum, t)
    ref = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0)
    assert abs(got["loss"] - ref["loss"]) < 1e-12
    assert torch.allclose(got["grad_inputs"], ref["grad_inputs"], atol=1e-13)
    assert torch.allclose(got["grad_weight"], ref["grad_weight"], atol=1e-13)


def test_planted_mistakes_are_caught():
    def transposed(X, W, fn, Y):
        out = dict(oll.linear_loss(X, W, fn, Y))
        gw = out["grad_weight"]
        out["grad_weight"] = gw.flip(0)          # rows of grad_weight permuted
        return out

    def half_grad(X, W, fn, Y):
        def f(Z, YY):
            loss, G = fn(Z, YY)
            return loss, G / 2
        return oll.linear_loss(X, W, f, Y)
    for mutant in (transposed, half_grad):
        err, tol = _fd_error(mutant)
        assert err > tol, mutant.__name__
