"""Seeded synthetic inputs for the cross-entropy paths.

This module only draws tensors on the host. It holds none of the method's
arithmetic, so the fp64 oracle, the GPU parity tests and the benchmark can all
take their inputs from it without sharing any computation.

Shapes and distributions follow the pages:

* the GPT-2 vocabulary of 50257 and hidden size 768, with the LM head tied to
  the token embedding so that logits are ``h @ wte^T`` (forge-ml ``Gpt2`` page,
  ``from_safetensors`` / ``forward``), and the (1, 128, 50257) logits example
  (lucid ``CausalLMOutput`` page, Examples);
* weights drawn from N(0, 0.02), read as a standard deviation of 0.02
  (forge-ml ``Gpt2`` page, ``init_random``);
* targets are class indices in [0, V), with ``ignore_index`` rows mixed in
  (greyhound functional API page, ``cross_entropy`` parameters).

Recipe (one ``torch.Generator('cpu')`` seeded once per workload, draws in this
order):

1. ``target = randint(0, V, (B,))``;
2. ``ignored = randperm(B)[:k]`` with ``k = floor(p*B + 0.5)``, or the explicit
   row list, and ``target[ignored] = ignore_index``;
3. only for boosted workloads: ``boost_col = randint(0, V, (B,))``;
4. the data, ``randn`` times sigma in fp32, drawn in blocks of rows (the
   stream does not depend on the block size), boost added in fp32, then cast
   to the workload dtype with round-to-nearest-even.

For the linear workloads step 4 draws ``inputs`` [BT, D] and then ``weight``
[V, D].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

IGNORE_INDEX = -100
_BLOCK_ELEMS = 1 << 26  # rows are drawn in blocks of about this many elements


@dataclasses.dataclass(frozen=True)
class CEWorkload:
    """A logits-level cross-entropy workload."""
    name: str
    B: int
    V: int
    dtype: torch.dtype
    sigma: float
    ignore_frac: float = 0.0
    ignore_rows: Optional[Sequence[int]] = None
    boost: float = 0.0
    z_loss: Sequence[float] = (0.0,)
    reductions: Sequence[str] = ("mean",)
    in_place: bool = False
    seed: int = 0

    @property
    def n_ignored(self) -> int:
        if self.ignore_rows is not None:
            return len(self.ignore_rows)
        return int(math.floor(self.ignore_frac * self.B + 0.5))


@dataclasses.dataclass(frozen=True)
class LinearCEWorkload:
    """A chunked linear cross-entropy workload (``inputs @ weight.T`` then CE)."""
    name: str
    BT: int
    D: int
    V: int
    chunk_size: int
    sigma_x: float = 1.0
    sigma_w: float = 0.02
    ignore_frac: float = 0.0
    z_loss: float = 0.0
    reduction: str = "mean"
    accums: Sequence[str] = ("fp32",)
    dtype: torch.dtype = torch.bfloat16
    seed: int = 0

    @property
    def n_ignored(self) -> int:
        return int(math.floor(self.ignore_frac * self.BT + 0.5))


# The five workloads of this path, named by what they are.
CE_B8_V1000_F32 = CEWorkload(
    name="ce_b8_v1000_f32", B=8, V=1000, dtype=torch.float32, sigma=2.0,
    ignore_rows=(3, 6), z_loss=(0.0, 1e-4), reductions=("mean", "sum"))
CE_B4096_V50257_BF16 = CEWorkload(
    name="ce_b4096_v50257_bf16_mean_z1e-4", B=4096, V=50257, dtype=torch.bfloat16,
    sigma=3.0, ignore_frac=0.05, boost=8.0, z_loss=(1e-4,), reductions=("mean",))
CE_B16384_V128256_BF16 = CEWorkload(
    name="ce_b16384_v128256_bf16_sum_inplace", B=16384, V=128256, dtype=torch.bfloat16,
    sigma=3.0, ignore_frac=0.02, z_loss=(0.0,), reductions=("sum",), in_place=True)
LCE_BT8192_D768_V50257 = LinearCEWorkload(
    name="linear_ce_bt8192_d768_v50257_c1024", BT=8192, D=768, V=50257, chunk_size=1024,
    ignore_frac=0.05, z_loss=1e-4, reduction="mean", accums=("fp32",))
LCE_BT16384_D4096_V128256 = LinearCEWorkload(
    name="linear_ce_bt16384_d4096_v128256_c2048", BT=16384, D=4096, V=128256,
    chunk_size=2048, ignore_frac=0.02, z_loss=0.0, reduction="mean",
    accums=("fp32", "weight"))

CE_WORKLOADS = (CE_B8_V1000_F32, CE_B4096_V50257_BF16, CE_B16384_V128256_BF16)
LINEAR_WORKLOADS = (LCE_BT8192_D768_V50257, LCE_BT16384_D4096_V128256)


def _targets(g: torch.Generator, B: int, V: int, n_ignored: int,
             ignore_rows: Optional[Sequence[int]], ignore_index: int) -> torch.Tensor:
    target = torch.randint(0, V, (B,), generator=g, dtype=torch.int64)
    if ignore_rows is not None:
        rows = torch.tensor(list(ignore_rows), dtype=torch.int64)
    else:
        rows = torch.randperm(B, generator=g)[:n_ignored]
    target[rows] = ignore_index
    return target


def _normal_rows(g: torch.Generator, rows: int, cols: int, sigma: float,
                 dtype: torch.dtype, boost_col: Optional[torch.Tensor] = None,
                 boost: float = 0.0) -> torch.Tensor:
    """``rows x cols`` of N(0, sigma) drawn in fp32 row blocks, cast to ``dtype``."""
    out = torch.empty((rows, cols), dtype=dtype)
    blk = max(1, _BLOCK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, blk):
        r1 = min(rows, r0 + blk)
        x = torch.randn((r1 - r0, cols), generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        if boost_col is not None and boost != 0.0:
            idx = torch.arange(r1 - r0)
            x[idx, boost_col[r0:r1]] += boost
        out[r0:r1].copy_(x)
    return out


def ce_inputs(w: CEWorkload, seed: Optional[int] = None):
    """(logits [B, V] in ``w.dtype``, target [B] int64) on the host."""
    g = torch.Generator(device="cpu").manual_seed(w.seed if seed is None else seed)
    target = _targets(g, w.B, w.V, w.n_ignored, w.ignore_rows, IGNORE_INDEX)
    boost_col = None
    if w.boost != 0.0:
        boost_col = torch.randint(0, w.V, (w.B,), generator=g, dtype=torch.int64)
    logits = _normal_rows(g, w.B, w.V, w.sigma, w.dtype, boost_col, w.boost)
    return logits, target


def linear_ce_inputs(w: LinearCEWorkload, seed: Optional[int] = None):
    """(inputs [BT, D], weight [V, D], target [BT]) on the host."""
    g = torch.Generator(device="cpu").manual_seed(w.seed if seed is None else seed)
    target = _targets(g, w.BT, w.V, w.n_ignored, None, IGNORE_INDEX)
    x = _normal_rows(g, w.BT, w.D, w.sigma_x, w.dtype)
    wt = _normal_rows(g, w.V, w.D, w.sigma_w, w.dtype)
    return x, wt, target


def small_ce(B: int, V: int, dtype=torch.float32, sigma: float = 2.0,
             n_ignored: int = 0, seed: int = 0, boost: float = 0.0):
    """Ad-hoc CE inputs with the same recipe, for tests at arbitrary sizes."""
    w = CEWorkload(name=f"ce_b{B}_v{V}", B=B, V=V, dtype=dtype, sigma=sigma,
                   ignore_rows=None, ignore_frac=0.0, boost=boost, seed=seed)
    g = torch.Generator(device="cpu").manual_seed(seed)
    target = _targets(g, B, V, n_ignored, None, IGNORE_INDEX)
    boost_col = torch.randint(0, V, (B,), generator=g, dtype=torch.int64) if boost else None
    logits = _normal_rows(g, B, V, sigma, dtype, boost_col, boost)
    return logits, target


def small_linear_ce(BT: int, D: int, V: int, dtype=torch.bfloat16, sigma_x: float = 1.0,
                    sigma_w: float = 0.02, n_ignored: int = 0, seed: int = 0):
    """Ad-hoc linear-CE inputs with the same recipe, for tests at arbitrary sizes."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    target = _targets(g, BT, V, n_ignored, None, IGNORE_INDEX)
    x = _normal_rows(g, BT, D, sigma_x, dtype)
    wt = _normal_rows(g, V, D, sigma_w, dtype)
    return x, wt, target


def row_upstream(B: int, seed: int = 0) -> torch.Tensor:
    """A per-row upstream gradient g [B] fp32 ~ N(0, 1) (for the per-row VJP tests)."""
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    return torch.randn(B, generator=g, dtype=torch.float32)
