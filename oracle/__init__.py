"""Plain fp64 CPU oracle for the cross-entropy paths.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never calls it, and the two share no
code: the oracle is the plain definition written out in float64 with PyTorch
CPU tensor operations, slow and obvious, so that a reader can check it against
the pages by eye.

Modules:

* ``oracle.ce``        -- cross-entropy loss and logits gradient from
  materialized logits (greyhound functional API page, ``cross_entropy``).
* ``oracle.linear_ce`` -- linear cross-entropy: logits ``inputs @ weight.T``,
  the same loss, and the gradients of ``inputs`` and ``weight``, plus the
  chunk-by-chunk weight-dtype accumulation (greyhound functional API page,
  ``chunked_linear_loss`` and ``chunked_linear_cross_entropy``).
* ``oracle.generic`` -- the generic chunked linear loss (greyhound
  functional API page, ``chunked_linear_loss``) for losses that are sums over
  rows, with ``mse_sum`` as the written-out example.
* ``oracle.rows``      -- per-row operations: ``selective_log_softmax``
  (greyhound functional API page) and the unreduced per-row cross-entropy
  with its vector-Jacobian product (nuvec ``FastOp`` page, ``CrossEntropy`` and
  ``CrossEntropyVjp``).
* ``oracle.bf16``, ``oracle.fp16`` -- round-to-nearest-even to bfloat16 and to
  IEEE binary16, written from the formats' definitions; used only by the
  weight-dtype accumulation emulation.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (finite differences, closed forms, invariants and
reductions to library routines).
"""
from oracle.ce import cross_entropy, cross_entropy_rows, count_valid  # noqa: F401
from oracle.linear_ce import linear_cross_entropy  # noqa: F401
from oracle.bf16 import round_to_bf16  # noqa: F401
from oracle.fp16 import round_to_fp16  # noqa: F401
from oracle.generic import linear_loss, mse_sum  # noqa: F401
from oracle.rows import (cross_entropy_per_row, cross_entropy_per_row_vjp,  # noqa: F401
                         selective_log_softmax)
