"""Cross-entropy with optional z-loss, loss and logits gradient, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed follows the greyhound functional API page, ``cross_entropy``
(signature, Parameters and Returns):

* each row ``i`` with ``target[i] != ignore_index`` contributes
  ``lse_i - x[i, t_i] + z * lse_i**2`` where ``lse_i = log(sum_j exp(x[i, j]))``
  is the natural-log log-sum-exp of the raw logits (the z-loss penalises the
  log-partition value; ``z`` is ``z_loss_multiplier``);
* rows whose target equals ``ignore_index`` contribute neither loss nor gradient;
* ``reduction='sum'`` returns the summed loss, ``'mean'`` divides it by the
  number N of valid tokens;
* the gradient of that scalar with respect to the logits is
  ``scale * ((1 + 2 z lse_i) * softmax(x_i) - onehot(t_i))`` on valid rows and
  zero on ignored rows, with ``scale = 1/N`` for mean and 1 for sum.

The per-row term ``logsumexp(logits) - logits[target]`` is also how the nuvec
``FastOp::CrossEntropy`` variant defines cross-entropy, and the negated per-row
loss at ``z = 0`` equals ``gather(log_softmax(x), t)`` as on the greyhound page's
``selective_log_softmax`` entry; both serve as pins in the tests.

Readings where the page is silent:

* ``mean`` with N = 0 gives ``0/0 = nan`` and all-zero gradients;
* a row is ignored exactly when ``target == ignore_index``, even when
  ``ignore_index`` lies in [0, V);
* a valid target outside [0, V) is a precondition violation: the oracle raises;
* the z-loss is inside the reduction, so ``mean`` divides it by N as well.
"""
from __future__ import annotations

import math
from typing import Optional

import torch


def count_valid(target: torch.Tensor, ignore_index: int, V: int):
    """N = #{i : target[i] != ignore_index}; raise if a valid target is outside [0, V).

    Greyhound functional API page, ``cross_entropy`` Parameters: targets are class
    indices in [0, V) and ``ignore_index`` tokens do not contribute.
    """
    t = target.to(torch.int64)
    valid = t != ignore_index
    bad = valid & ((t < 0) | (t >= V))
    if bool(bad.any()):
        raise ValueError("a valid target lies outside [0, V)")
    return int(valid.sum()), valid


def cross_entropy_rows(x: torch.Tensor, target: torch.Tensor, valid: torch.Tensor,
                       scale: float, z: float, want_grad: bool = True):
    """Per-row lse, loss term and gradient rows for a block of rows, in fp64.

    ``x`` is any float tensor [R, V]; it is upcast exactly to fp64. ``scale`` is the
    reduction factor of the whole batch (1/N for mean, 1 for sum), so a block of
    rows taken out of a larger batch gets exactly its rows of the full gradient.
    Returns ``(lse [R], row_loss [R], grad [R, V] or None)``; ignored rows have
    ``row_loss = 0`` and a zero gradient row (their lse is still reported).
    """
    x = x.to(torch.float64)
    R, V = x.shape
    m = x.max(dim=1, keepdim=True).values                      # row max
    s = torch.exp(x - m).sum(dim=1, keepdim=True)               # sum of shifted exps
    lse = (m + torch.log(s)).squeeze(1)                         # log-sum-exp
    t = target.to(torch.int64).clamp(0, max(V - 1, 0))
    x_t = x.gather(1, t.unsqueeze(1)).squeeze(1) if V > 0 else torch.zeros(R, dtype=torch.float64)
    row_loss = torch.where(valid, lse - x_t + z * lse * lse, torch.zeros_like(lse))
    grad = None
    if want_grad:
        p = torch.exp(x - lse.unsqueeze(1))                     # softmax
        grad = (1.0 + 2.0 * z * lse).unsqueeze(1) * p
        rows = torch.arange(R)
        grad[rows, t] -= 1.0                                    # minus one-hot
        grad *= scale
        grad[~valid] = 0.0
    return lse, row_loss, grad


def reduction_scale(n_valid: int, reduction: str) -> float:
    """1/N for mean (inf when N = 0, unused then since every row is ignored), 1 for sum."""
    if reduction == "mean":
        return math.inf if n_valid == 0 else 1.0 / n_valid
    if reduction == "sum":
        return 1.0
    raise ValueError(f"unknown reduction {reduction!r}")


def cross_entropy(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100,
                  reduction: str = "mean", z_loss_multiplier: float = 0.0,
                  want_grad: bool = True, block_rows: Optional[int] = None):
    """Loss and logits gradient of the greyhound ``cross_entropy`` definition, in fp64.

    Returns a dict with ``loss`` (Python float), ``grad`` (fp64 [B, V] or None),
    ``n_valid`` (int), ``lse`` (fp64 [B]) and ``row_loss`` (fp64 [B]).
    Rows are processed in blocks of ``block_rows`` to bound host memory; the
    rows are independent, so the blocking does not change any value.
    """
    B, V = logits.shape
    n_valid, valid = count_valid(target, ignore_index, V)
    scale = reduction_scale(n_valid, reduction)
    if block_rows is None:
        block_rows = max(1, (1 << 24) // max(V, 1))
    lse = torch.empty(B, dtype=torch.float64)
    row_loss = torch.empty(B, dtype=torch.float64)
    grad = torch.empty((B, V), dtype=torch.float64) if want_grad else None
    for r0 in range(0, B, block_rows):
        r1 = min(B, r0 + block_rows)
        l, rl, g = cross_entropy_rows(logits[r0:r1], target[r0:r1], valid[r0:r1],
                                      scale, z_loss_multiplier, want_grad)
        lse[r0:r1] = l
        row_loss[r0:r1] = rl
        if want_grad:
            grad[r0:r1] = g
    total = math.fsum(row_loss.tolist())
    if reduction == "mean":
        loss = total / n_valid if n_valid > 0 else math.nan
    else:
        loss = total
    return {"loss": loss, "grad": grad, "n_valid": n_valid, "lse": lse,
            "row_loss": row_loss}
