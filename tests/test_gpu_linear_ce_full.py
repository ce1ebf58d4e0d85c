"""Full-size GPU parity of linear_ce on the inputs [16384, 4096] x weight
[128256, 4096] bf16 workload (chunk 2048, mean, z = 0), needs an MI355X.

Both accumulation modes run once on the GPU; the fp64 oracle then walks the
same row chunks in order (``oracle.linear_ce.linear_cross_entropy_chunks``),
one test per chunk so that no single test holds the host for long:

* every grad_inputs row of both modes against the exact value (relative
  Frobenius norm per chunk and over the whole tensor, 1e-2);
* grad_weight in 'fp32' mode against the exact sum of the chunk products, and
  in 'weight' mode against the chunk-by-chunk emulation
  ``rnd(dW + G_c^T X_c)`` (``oracle.linear_ce.accumulate_weight_dtype``), both
  over the whole [128256, 4096] tensor at 1e-2 relative Frobenius; the 'weight'
  result must also lie closer to the emulation than to the exact value;
* the loss (2e-3 relative) and N (exact).

The chunks of the oracle are the GPU's chunks (2048 rows), so the emulation
rounds where the GPU does.
"""
import math

import pytest
import torch

import workloads
from oracle import linear_ce as olce
from lm_head_cross_pass_amd import functional as F

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = torch.device("cuda:0")
W5 = workloads.LCE_BT16384_D4096_V128256
NCHUNKS = (W5.BT + W5.chunk_size - 1) // W5.chunk_size


class _Walk:
    """GPU results of both modes, and the oracle's chunk walk with its running sums."""

    def __init__(self):
        X, W, t = workloads.linear_ce_inputs(W5)
        self.gpu = {}
        Xd, Wd, td = X.to(DEV), W.to(DEV), t.to(DEV)
        for accum in ("fp32", "weight"):
            loss, gx, gw, n, bad = F.linear_ce(Xd, Wd, td, -100, W5.reduction, W5.z_loss,
                                               W5.chunk_size, accum)
            torch.cuda.synchronize()
            self.gpu[accum] = {"loss": float(loss), "n": int(n), "bad": int(bad),
                               "gx": gx.cpu(), "gw": gw.cpu()}
            del gx, gw
        del Xd, Wd, td
        torch.cuda.empty_cache()
        self.steps = olce.linear_cross_entropy_chunks(X, W, t, -100, W5.reduction, W5.z_loss,
                                                      W5.chunk_size)
        self.done = 0
        self.row_loss = []
        self.n_valid = None
        self.dw_exact = torch.zeros(W5.V, W5.D, dtype=torch.float64)
        self.dw_emu = torch.zeros(W5.V, W5.D, dtype=torch.float64)
        self.gx_num2 = {"fp32": 0.0, "weight": 0.0}
        self.gx_den2 = 0.0
        self.workers = max(1, torch.get_num_threads())

    def advance(self, upto):
        """Walks the oracle through chunk `upto - 1`; returns the per-chunk
        grad_inputs errors of the chunks walked now."""
        errs = []
        while self.done < upto:
            ch = next(self.steps)
            r0, r1 = ch["r0"], ch["r1"]
            self.n_valid = ch["n_valid"]
            self.row_loss += ch["row_loss"].tolist()
            ref = ch["grad_inputs"]
            den = float((ref * ref).sum())
            self.gx_den2 += den
            for accum in ("fp32", "weight"):
                d = self.gpu[accum]["gx"][r0:r1].double() - ref
                num = float((d * d).sum())
                self.gx_num2[accum] += num
                errs.append((accum, math.sqrt(num / den)))
            self.dw_exact += ch["partial"]
            self.dw_emu = olce.accumulate_weight_dtype(self.dw_emu, ch["partial"], torch.bfloat16,
                                                       self.workers)
            self.done += 1
        return errs


@pytest.fixture(scope="module")
def walk():
    return _Walk()


@pytest.mark.parametrize("c", range(NCHUNKS))
def test_grad_inputs_rows_of_chunk(walk, c):
    for accum, err in walk.advance(c + 1):
        assert err <= 1e-2, (c, accum, err)


def test_loss_count_and_whole_grad_inputs(walk):
    walk.advance(NCHUNKS)
    ref = math.fsum(walk.row_loss) / walk.n_valid
    for accum in ("fp32", "weight"):
        g = walk.gpu[accum]
        assert g["n"] == walk.n_valid == 16056 and g["bad"] == 0
        assert g["loss"] == pytest.approx(ref, rel=2e-3)
        assert math.sqrt(walk.gx_num2[accum] / walk.gx_den2) <= 1e-2


def _rel(a, b):
    d = a.double() - b
    return math.sqrt(float((d * d).sum()) / float((b * b).sum()))


def test_grad_weight_fp32_against_exact(walk):
    walk.advance(NCHUNKS)
    assert _rel(walk.gpu["fp32"]["gw"], walk.dw_exact) <= 1e-2


def test_grad_weight_weight_mode_against_emulation(walk):
    walk.advance(NCHUNKS)
    gw = walk.gpu["weight"]["gw"]
    e_emu = _rel(gw, walk.dw_emu)
    assert e_emu <= 1e-2
    # rounding after each of the 8 chunks moves the result toward the emulation
    assert e_emu < _rel(gw, walk.dw_exact)
