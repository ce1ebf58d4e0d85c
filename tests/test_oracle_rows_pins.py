"""Pins of the per-row oracle functions (CPU only): ``selective_log_softmax``,
the unreduced per-row cross-entropy and its vector-Jacobian product.

Sources of truth, none of them the oracle itself:

* ``torch.gather(log_softmax(x), index)`` in fp64, which the greyhound page's
  ``selective_log_softmax`` entry states as its equivalent;
* ``torch.nn.functional.cross_entropy(reduction='none')`` in fp64 for the
  per-row loss (the FastOp page's ``logsumexp(logits) - logits[target]``);
* autograd-free central finite differences of ``sum_i g_i loss_i`` for the VJP;
* closed forms: uniform logits give ``-log V`` / ``log V``; V = 2 gives a
  softplus; invariants: VJP rows sum to zero, are linear in ``g``, ignored rows
  are zero.

``test_planted_vjp_mistakes_are_caught`` plants slips in a copy of the VJP and
shows the finite-difference pin catches each.
"""
import math

import pytest
import torch
import torch.nn.functional as F

from oracle import rows as orows

torch.set_default_dtype(torch.float64)


def _tiny(B=5, V=7, seed=11, ignored=(1,)):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, V, generator=g, dtype=torch.float64) * 2.0
    t = torch.randint(0, V, (B,), generator=g)
    for r in ignored:
        t[r] = -100
    gr = torch.randn(B, generator=g, dtype=torch.float64)
    return x, t, gr


def test_selective_log_softmax_equals_gather_of_log_softmax():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(6, 50, generator=g, dtype=torch.float64) * 3
    idx = torch.randint(0, 50, (6,), generator=g)
    ref = torch.gather(F.log_softmax(x, dim=-1), -1, idx.unsqueeze(-1)).squeeze(-1)
    assert torch.allclose(orows.selective_log_softmax(x, idx), ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("V", (2, 1000, 128256))
def test_selective_log_softmax_uniform_logits(V):
    x = torch.full((2, V), 0.25, dtype=torch.float64)
    out = orows.selective_log_softmax(x, torch.tensor([0, V - 1]))
    assert torch.allclose(out, torch.full((2,), -math.log(V)), rtol=1e-13, atol=0)


def test_selective_log_softmax_two_classes_is_negative_softplus():
    x = torch.tensor([[1.5, -0.25], [-3.0, 2.0]])
    idx = torch.tensor([0, 0])
    other = torch.tensor([-0.25, 2.0])
    ref = -F.softplus(other - x[:, 0])
    assert torch.allclose(orows.selective_log_softmax(x, idx), ref, rtol=1e-14, atol=1e-15)


def test_selective_log_softmax_rejects_out_of_range_index():
    x = torch.zeros(2, 4)
    with pytest.raises(ValueError):
        orows.selective_log_softmax(x, torch.tensor([0, 4]))


def test_per_row_loss_equals_torch_cross_entropy_none():
    x, t, _ = _tiny(B=9, V=13)
    ref = F.cross_entropy(x, t, ignore_index=-100, reduction="none")
    assert torch.allclose(orows.cross_entropy_per_row(x, t, -100), ref, rtol=1e-14, atol=1e-15)


def test_per_row_loss_uniform_and_ignored():
    V = 50257
    x = torch.full((3, V), -1.75, dtype=torch.float64)
    t = torch.tensor([0, -100, V - 1])
    out = orows.cross_entropy_per_row(x, t, -100)
    assert out[1] == 0.0
    assert math.isclose(float(out[0]), math.log(V), rel_tol=1e-13)
    assert math.isclose(float(out[2]), math.log(V), rel_tol=1e-13)


def _fd_vjp_error(vjp):
    x, t, gr = _tiny()
    h = 1e-6

    def f(xx):
        return float((gr * orows.cross_entropy_per_row(xx, t, -100)).sum())
    fd = torch.empty_like(x)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            xp = x.clone(); xp[i, j] += h
            xm = x.clone(); xm[i, j] -= h
            fd[i, j] = (f(xp) - f(xm)) / (2 * h)
    err = float((fd - vjp(x, t, gr, -100)).abs().max())
    return err, 1e-8 + 1e-7 * float(fd.abs().max())


def test_vjp_matches_central_differences():
    err, tol = _fd_vjp_error(orows.cross_entropy_per_row_vjp)
    assert err <= tol


def test_vjp_invariants():
    x, t, gr = _tiny(B=6, V=11)
    G = orows.cross_entropy_per_row_vjp(x, t, gr, -100)
    valid = t != -100
    assert torch.all(G[~valid] == 0)
    assert torch.allclose(G[valid].sum(dim=1), torch.zeros(int(valid.sum())), atol=1e-15)
    G2 = orows.cross_entropy_per_row_vjp(x, t, 2.5 * gr, -100)
    assert torch.allclose(G2, 2.5 * G, rtol=1e-14, atol=1e-16)
    # with g = 1 on every valid row, the VJP is the 'sum' reduction's gradient
    ones = torch.ones_like(gr)
    ref = torch.autograd.functional.jacobian(
        lambda xx: F.cross_entropy(xx, t, ignore_index=-100, reduction="sum"), x)
    assert torch.allclose(orows.cross_entropy_per_row_vjp(x, t, ones, -100), ref,
                          rtol=1e-13, atol=1e-15)


def test_planted_vjp_mistakes_are_caught():
    real = orows.cross_entropy_per_row_vjp

    def sign(x, t, g, ii):                    # onehot added instead of subtracted
        out = real(x, t, g, ii)
        valid = t != ii
        rows = torch.arange(x.shape[0])[valid]
        out[rows, t[valid]] += 2 * g[valid]
        return out

    def no_g(x, t, g, ii):                    # upstream gradient ignored
        return real(x, t, torch.ones_like(g), ii)

    def shifted_index(x, t, g, ii):           # one-hot at t + 1
        tt = t.clone()
        valid = tt != ii
        tt[valid] = (tt[valid] + 1) % x.shape[1]
        return real(x, tt, g, ii)

    for mutant in (sign, no_g, shifted_index):
        err, tol = _fd_vjp_error(mutant)
        assert err > tol, mutant.__name__
