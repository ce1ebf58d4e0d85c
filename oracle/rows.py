"""Per-row cross-entropy operations, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* ``selective_log_softmax`` -- greyhound functional API page,
  ``selective_log_softmax``: the log-softmax of each row taken at one index,
  i.e. ``gather(log_softmax(x), index)``, returned per row.
* ``cross_entropy_per_row`` -- nuvec ``FastOp`` page, ``CrossEntropy``: per row
  ``logsumexp(x_i) - x_i[t_i]`` (no reduction).
* ``cross_entropy_per_row_vjp`` -- nuvec ``FastOp`` page, ``CrossEntropyVjp``:
  the gradient with respect to the logits of ``sum_i g_i * CrossEntropy_i``,
  i.e. ``g_i * (softmax(x_i) - onehot(t_i))`` for each row. (The page's VJP
  also receives the forward's loss; it does not change the value, so the
  definition here does not use it.)

Readings where the pages are silent:

* ``ignore_index`` as in ``cross_entropy``: a row whose target equals it has
  loss 0 and a zero gradient row (the FastOp page has no ignore index; any
  value that no target takes reproduces it);
* an index or valid target outside [0, V) is a precondition violation: raise;
* outputs are float (fp64 here), whatever the logits dtype.
"""
from __future__ import annotations

import torch


def _check_index(index: torch.Tensor, V: int, valid: torch.Tensor) -> torch.Tensor:
    t = index.to(torch.int64)
    if bool((valid & ((t < 0) | (t >= V))).any()):
        raise ValueError("an index lies outside [0, V)")
    return t


def _row_logsumexp(x: torch.Tensor) -> torch.Tensor:
    """log(sum_j exp(x[i, j])) per row, shifted by the row max for range."""
    m = x.max(dim=1, keepdim=True).values
    return (m + torch.log(torch.exp(x - m).sum(dim=1, keepdim=True))).squeeze(1)


def selective_log_softmax(logits: torch.Tensor, index: torch.Tensor) -> torch.Tensor:
    """``log_softmax(x_i)[index_i]`` per row, fp64 [B]."""
    x = logits.to(torch.float64)
    B, V = x.shape
    t = _check_index(index, V, torch.ones(B, dtype=torch.bool))
    x_t = x.gather(1, t.unsqueeze(1)).squeeze(1)
    return x_t - _row_logsumexp(x)


def cross_entropy_per_row(logits: torch.Tensor, target: torch.Tensor,
                          ignore_index: int = -100) -> torch.Tensor:
    """``logsumexp(x_i) - x_i[t_i]`` per row (0 on ignored rows), fp64 [B]."""
    x = logits.to(torch.float64)
    B, V = x.shape
    valid = target.to(torch.int64) != ignore_index
    t = _check_index(target, V, valid).clamp(0, V - 1)
    x_t = x.gather(1, t.unsqueeze(1)).squeeze(1)
    loss = _row_logsumexp(x) - x_t
    return torch.where(valid, loss, torch.zeros_like(loss))


def cross_entropy_per_row_vjp(logits: torch.Tensor, target: torch.Tensor, g: torch.Tensor,
                              ignore_index: int = -100) -> torch.Tensor:
    """``g_i * (softmax(x_i) - onehot(t_i))`` per row (zero rows where ignored), fp64 [B, V]."""
    x = logits.to(torch.float64)
    B, V = x.shape
    valid = target.to(torch.int64) != ignore_index
    t = _check_index(target, V, valid).clamp(0, V - 1)
    p = torch.exp(x - _row_logsumexp(x).unsqueeze(1))          # softmax
    p[torch.arange(B), t] -= 1.0                               # minus one-hot
    grad = g.to(torch.float64).unsqueeze(1) * p
    grad[~valid] = 0.0
    return grad
