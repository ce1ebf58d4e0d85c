"""Generic linear loss: a per-row-chunk loss on ``inputs @ weight.T``, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed follows the greyhound functional API page, ``chunked_linear_loss``
(Returns: the sum of the scalar losses of the chunks; gradients of inputs and weight
accumulated from each chunk's logits gradient) with a loss whose chunk losses add up
to the loss of the whole batch (sums over rows, as ``mse_loss(reduction='sum')`` or
``cross_entropy(reduction='sum')``). For such a loss the sum over chunks is the loss
of all rows at once, and the gradients are the plain chain rule:

    Z = X W^T,   (loss, G) = loss_and_grad(Z),   dX = G W,   dW = G^T X.

The oracle evaluates that definition in one piece (no chunking), in fp64.

``mse_sum`` is one such loss written out: ``sum((Z - Y)^2)`` with gradient
``2 (Z - Y)``.
"""
from __future__ import annotations

import torch


def mse_sum(Z: torch.Tensor, Y: torch.Tensor):
    """sum((Z - Y)^2) and its gradient with respect to Z, fp64."""
    d = Z.to(torch.float64) - Y.to(torch.float64)
    return float((d * d).sum()), 2.0 * d


def linear_loss(inputs: torch.Tensor, weight: torch.Tensor, loss_and_grad, *loss_args):
    """Loss, grad_inputs and grad_weight of ``loss_and_grad(inputs @ weight.T, *loss_args)``."""
    X = inputs.to(torch.float64)
    W = weight.to(torch.float64)
    Z = X @ W.T
    loss, G = loss_and_grad(Z, *loss_args)
    return {"loss": loss, "grad_inputs": G @ W, "grad_weight": G.T @ X}
