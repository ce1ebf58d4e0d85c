"""Linear cross-entropy (``inputs @ weight.T`` then cross-entropy), in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows the greyhound functional API page, ``chunked_linear_loss`` and
``chunked_linear_cross_entropy``:

* the logits are ``inputs [BT, D] @ weight[V, D].T``;
* the loss is the ``cross_entropy`` of those logits (``oracle.ce``), with
  ``mean`` dividing by the number of valid tokens of the whole batch (the
  plain reading: one global N, not a mean of per-chunk means);
* ``grad_inputs = G @ weight`` and ``grad_weight = G.T @ inputs`` where ``G`` is
  the logits gradient; chunking the rows changes neither in exact arithmetic,
  so the fp32-accumulation mode is the exact product;
* ``grad_weight_accum_dtype='weight'`` accumulates directly in the parameter
  dtype and rounds between chunks. It is emulated chunk by chunk, in the
  order of the rows, as ``dW <- bf16(dW + G_c.T @ X_c)`` starting from zero,
  with the partial product exact and one round-to-nearest-even per chunk.

No intermediate rounding of the logits or of ``G`` is modelled: the oracle is
the exact value; the GPU path's bf16 matmul inputs and outputs are covered by
the tolerances.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import torch

from oracle.bf16 import round_to_bf16
from oracle.fp16 import round_to_fp16
from oracle.ce import count_valid, cross_entropy_rows, reduction_scale


def _finish_loss(row_loss_sum_terms, n_valid: int, reduction: str) -> float:
    total = math.fsum(row_loss_sum_terms)
    if reduction == "mean":
        return total / n_valid if n_valid > 0 else math.nan
    return total


def linear_cross_entropy_chunks(inputs: torch.Tensor, weight: torch.Tensor,
                                target: torch.Tensor, ignore_index: int = -100,
                                reduction: str = "mean", z_loss_multiplier: float = 0.0,
                                chunk_rows: int = 256):
    """The linear cross-entropy chunk by chunk, in fp64, in the order of the rows.

    Yields one dict per chunk of ``chunk_rows`` rows (the last one may be shorter):
    ``r0``, ``r1`` (the rows), ``lse`` and ``row_loss`` of those rows, their
    ``grad_inputs`` rows ``G_c @ weight`` and the chunk's product
    ``partial = G_c.T @ inputs[r0:r1]`` (its share of grad_weight); ``n_valid``
    and ``scale`` are those of the whole batch (one global N for the mean).
    """
    BT, D = inputs.shape
    V = weight.shape[0]
    n_valid, valid = count_valid(target, ignore_index, V)
    scale = reduction_scale(n_valid, reduction)
    W = weight.to(torch.float64)
    for r0 in range(0, BT, chunk_rows):
        r1 = min(BT, r0 + chunk_rows)
        Xc = inputs[r0:r1].to(torch.float64)
        logits = Xc @ W.T                                        # [rows, V]
        lse, rl, G = cross_entropy_rows(logits, target[r0:r1], valid[r0:r1],
                                        scale, z_loss_multiplier)
        del logits
        yield {"r0": r0, "r1": r1, "lse": lse, "row_loss": rl, "grad_inputs": G @ W,
               "partial": G.T @ Xc, "n_valid": n_valid, "scale": scale}


def _rowwise(fn, M: torch.Tensor, workers: int) -> torch.Tensor:
    """fn applied to row blocks of M (fn is element-wise: the blocking does not
    change any value), on up to ``workers`` threads."""
    if workers <= 1 or M.shape[0] < 2 * workers:
        return fn(M)
    import concurrent.futures as cf
    out = torch.empty_like(M)
    bounds = [(i * M.shape[0] // workers, (i + 1) * M.shape[0] // workers) for i in range(workers)]

    def run(b):
        out[b[0]:b[1]] = fn(M[b[0]:b[1]])
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(run, bounds))
    return out


def accumulate_weight_dtype(dW: torch.Tensor, partial: torch.Tensor, weight_dtype: torch.dtype,
                            workers: int = 1) -> torch.Tensor:
    """One chunk of the ``'weight'`` accumulation: ``rnd(dW + partial)``.

    The running weight gradient is held in the parameter's dtype, so after each
    chunk the exact sum of the previous value and the chunk's exact product is
    rounded to nearest even in that dtype (bf16, or fp16 for an fp16 weight).
    """
    rnd = round_to_fp16 if weight_dtype == torch.float16 else round_to_bf16
    return _rowwise(rnd, dW + partial, workers)


def linear_cross_entropy(inputs: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                         ignore_index: int = -100, reduction: str = "mean",
                         z_loss_multiplier: float = 0.0,
                         grad_weight_accum_dtype: str = "fp32",
                         chunk_size: Optional[int] = None,
                         block_rows: int = 256):
    """Loss, grad_inputs and grad_weight of the linear cross-entropy, in fp64.

    ``grad_weight_accum_dtype='fp32'`` returns the exact fp64 gradients (chunking
    does not change them); ``'weight'`` returns the chunk-by-chunk emulation of
    the weight gradient in the weight's dtype (bf16, or fp16 for an fp16
    weight; ``chunk_size`` rows per chunk) and the exact ``grad_inputs``. Returns a dict with ``loss``, ``grad_inputs``,
    ``grad_weight``, ``n_valid``, ``lse`` and ``row_loss``.
    """
    BT, D = inputs.shape
    V = weight.shape[0]
    if grad_weight_accum_dtype == "fp32":
        step = block_rows
    elif grad_weight_accum_dtype == "weight":
        if chunk_size is None or chunk_size <= 0:
            raise ValueError("the weight-dtype emulation needs the chunk size")
        step = chunk_size
    else:
        raise ValueError(f"unknown grad_weight_accum_dtype {grad_weight_accum_dtype!r}")
    dX = torch.zeros((BT, D), dtype=torch.float64)
    dW = torch.zeros((V, D), dtype=torch.float64)
    lse = torch.empty(BT, dtype=torch.float64)
    row_loss = torch.empty(BT, dtype=torch.float64)
    n_valid = count_valid(target, ignore_index, V)[0]
    for ch in linear_cross_entropy_chunks(inputs, weight, target, ignore_index, reduction,
                                          z_loss_multiplier, step):
        r0, r1 = ch["r0"], ch["r1"]
        lse[r0:r1] = ch["lse"]
        row_loss[r0:r1] = ch["row_loss"]
        dX[r0:r1] = ch["grad_inputs"]
        if grad_weight_accum_dtype == "fp32":
            dW += ch["partial"]                                  # exact sum over chunks
        else:
            dW = accumulate_weight_dtype(dW, ch["partial"], weight.dtype)   # rounds between chunks
    loss = _finish_loss(row_loss.tolist(), n_valid, reduction)
    return {"loss": loss, "grad_inputs": dX, "grad_weight": dW, "n_valid": n_valid,
            "lse": lse, "row_loss": row_loss}


def linear_cross_entropy_sampled(inputs: torch.Tensor, weight: torch.Tensor,
                                 target: torch.Tensor, rows: Sequence[int],
                                 vocab_rows: Sequence[int], ignore_index: int = -100,
                                 reduction: str = "mean", z_loss_multiplier: float = 0.0,
                                 block_rows: int = 512):
    """Exact fp64 loss plus selected rows of grad_inputs and of grad_weight.

    The same definition as ``linear_cross_entropy`` (fp32-accumulation mode),
    evaluated only where asked so that it stays affordable at full sizes: the
    loss needs every row's lse; ``grad_inputs[r] = G[r] @ weight`` needs row r of
    G; ``grad_weight[v] = G[:, v] @ inputs`` needs column v of G for all rows.
    """
    BT, D = inputs.shape
    V = weight.shape[0]
    n_valid, valid = count_valid(target, ignore_index, V)
    scale = reduction_scale(n_valid, reduction)
    W = weight.to(torch.float64)
    rows_t = torch.as_tensor(list(rows), dtype=torch.int64)
    cols_t = torch.as_tensor(list(vocab_rows), dtype=torch.int64)
    dX_rows = torch.zeros((len(rows_t), D), dtype=torch.float64)
    dW_rows = torch.zeros((len(cols_t), D), dtype=torch.float64)
    row_loss = torch.empty(BT, dtype=torch.float64)
    z = z_loss_multiplier
    for r0 in range(0, BT, block_rows):
        r1 = min(BT, r0 + block_rows)
        Xb = inputs[r0:r1].to(torch.float64)
        logits = Xb @ W.T
        lse, rl, _ = cross_entropy_rows(logits, target[r0:r1], valid[r0:r1], scale, z,
                                        want_grad=False)
        row_loss[r0:r1] = rl
        # column block of G for the sampled vocabulary rows: scale*((1+2z lse) p - onehot)
        pc = torch.exp(logits[:, cols_t] - lse.unsqueeze(1)) * (1.0 + 2.0 * z * lse).unsqueeze(1)
        tb = target[r0:r1].to(torch.int64)
        pc -= (tb.unsqueeze(1) == cols_t.unsqueeze(0)).to(torch.float64)
        pc *= scale
        pc[~valid[r0:r1]] = 0.0
        dW_rows += pc.T @ Xb
        # full rows of G for the sampled token rows that fall in this block
        sel = ((rows_t >= r0) & (rows_t < r1)).nonzero().flatten()
        if len(sel):
            loc = rows_t[sel] - r0
            _, _, G = cross_entropy_rows(logits[loc], tb[loc], valid[r0:r1][loc], scale, z)
            dX_rows[sel] = G @ W
    loss = _finish_loss(row_loss.tolist(), n_valid, reduction)
    return {"loss": loss, "grad_inputs_rows": dX_rows, "grad_weight_rows": dW_rows,
            "n_valid": n_valid, "row_loss": row_loss}
