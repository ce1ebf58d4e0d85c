"""GPU parity of the per-row entry points against the fp64 oracle (needs an MI355X):
selective_log_softmax, ce_loss_rows and ce_loss_rows_vjp.

Tolerances:
* per-row values (log-probabilities, losses): |got - ref| <= 1e-5 max(1, |ref|)
  for fp32 and bf16 logits alike (the arithmetic is fp32 from the exact input
  values; 1e-5 relative is the loss bar of the reduced cross-entropy);
* the VJP gradient, fp32 logits: |got - ref| <= 1e-6 max(1, |g_i|) per element
  (the reduced path's 1e-6 absolute bar, scaled by the row's upstream
  gradient); bf16 logits: relative Frobenius error <= 1e-2 and element-wise
  one bf16 rounding on top of fp32 arithmetic (2^-8 |ref| + 1e-7 |g_i|);
  fp16 logits: the same with the fp16 unit roundoff, relative Frobenius error
  <= 1e-3 and element-wise 2^-10 |ref| + 2^-25 + 1e-7 |g_i| (2^-25 is half the
  spacing of fp16 subnormals, where the smallest probabilities land);
* ignored rows exactly 0; N and the out-of-range flag exactly.
The VJP's loss input is the oracle's per-row loss rounded to fp32 (never a GPU
value); g comes from the seeded ``workloads.row_upstream``.
"""
import pytest
import torch

import oracle
import workloads
from lm_head_cross_pass_amd import functional as F

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SHAPES = [
    (3, 1, torch.float32), (5, 7, torch.bfloat16), (9, 2049, torch.bfloat16),
    (130, 1000, torch.float32), (33, 50257, torch.bfloat16), (17, 50257, torch.float32),
    (4, 131073, torch.bfloat16), (6, 70001, torch.float32), (5, 128256, torch.bfloat16),
    (5, 7, torch.float16), (9, 2049, torch.float16), (33, 50257, torch.float16),
    (5, 128256, torch.float16),
]


def _rows_close(got, ref):
    got = got.double().cpu()
    bound = 1e-5 * torch.clamp(ref.abs(), min=1.0)
    assert bool(((got - ref).abs() <= bound).all()), float(((got - ref).abs() - bound).max())


def _vjp_close(got, ref, g, dtype):
    got = got.double().cpu()
    gi = g.double().abs().unsqueeze(1)
    if dtype == torch.float32:
        bound = 1e-6 * torch.clamp(gi, min=1.0)
        assert bool(((got - ref).abs() <= bound).all()), float(((got - ref).abs() - bound).max())
    else:
        fp16 = dtype == torch.float16
        n = float(ref.norm())
        if n > 0:
            assert float((got - ref).norm()) / n <= (1e-3 if fp16 else 1e-2)
        if fp16:
            bound = 2.0 ** -10 * ref.abs() + 2.0 ** -25 + 1e-7 * gi
        else:
            bound = 2.0 ** -8 * ref.abs() + 1e-7 * gi
        assert bool(((got - ref).abs() <= bound).all()), float(((got - ref).abs() - bound).max())


@pytest.mark.parametrize("B,V,dtype", SHAPES)
def test_selective_log_softmax(B, V, dtype):
    logits, index = workloads.small_ce(B, V, dtype, sigma=2.0, seed=B + V)
    out = F.selective_log_softmax(logits.to(DEV), index.to(DEV))
    torch.cuda.synchronize()
    assert out.dtype == torch.float32 and out.shape == (B,)
    _rows_close(out, oracle.selective_log_softmax(logits, index))


@pytest.mark.parametrize("B,V,dtype", SHAPES)
def test_ce_loss_rows(B, V, dtype):
    logits, target = workloads.small_ce(B, V, dtype, sigma=2.0, n_ignored=B // 3, seed=B * V)
    loss, n, bad = F.ce_loss_rows(logits.to(DEV), target.to(DEV), -100)
    torch.cuda.synchronize()
    ref = oracle.cross_entropy_per_row(logits, target, -100)
    _rows_close(loss, ref)
    ignored = target == -100
    assert bool((loss.cpu()[ignored] == 0).all())
    assert int(n) == int((~ignored).sum()) and int(bad) == 0


@pytest.mark.parametrize("in_place", (False, True))
@pytest.mark.parametrize("B,V,dtype", SHAPES)
def test_ce_loss_rows_vjp(B, V, dtype, in_place):
    logits, target = workloads.small_ce(B, V, dtype, sigma=2.0, n_ignored=B // 3, seed=B + 2 * V)
    g = workloads.row_upstream(B, seed=V)
    loss_in = oracle.cross_entropy_per_row(logits, target, -100).float()
    x = logits.to(DEV)
    grad = F.ce_loss_rows_vjp(x, target.to(DEV), loss_in.to(DEV), g.to(DEV), -100,
                              in_place=in_place)
    torch.cuda.synchronize()
    assert grad.dtype == dtype and (grad.data_ptr() == x.data_ptr()) == in_place
    ref = oracle.cross_entropy_per_row_vjp(logits, target, g.double(), -100)
    _vjp_close(grad, ref, g, dtype)
    assert bool((grad.cpu()[target == -100] == 0).all())


@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16, torch.float32))
@pytest.mark.parametrize("in_place", (False, True))
def test_vjp_many_rows_per_workgroup(dtype, in_place):
    """More rows than resident workgroups (each walks several rows, reading the
    next row's target, g, loss and x[t] while the current one streams), odd V
    so that rows start at every offset inside a 16-byte chunk, and (in place)
    a logits base 2 elements past a 16-byte boundary; every row is compared,
    and the elements around the tensor are left alone."""
    B, V = 1100, 3001
    logits, target = workloads.small_ce(B, V, dtype, sigma=2.0, n_ignored=97, seed=77)
    g = workloads.row_upstream(B, seed=5)
    loss_in = oracle.cross_entropy_per_row(logits, target, -100).float()
    off = 2 if in_place else 0
    buf = torch.full((B * V + 8,), 7.0, dtype=dtype, device=DEV)
    x = buf[off:off + B * V].view(B, V)
    x.copy_(logits.to(DEV))
    assert (x.data_ptr() % 16 != 0) == in_place
    grad = F.ce_loss_rows_vjp(x, target.to(DEV), loss_in.to(DEV), g.to(DEV), -100,
                              in_place=in_place)
    torch.cuda.synchronize()
    assert (grad.data_ptr() == x.data_ptr()) == in_place
    ref = oracle.cross_entropy_per_row_vjp(logits, target, g.double(), -100)
    _vjp_close(grad, ref, g, dtype)
    assert bool((grad.cpu()[target == -100] == 0).all())
    outside = torch.cat([buf[:off], buf[off + B * V:]]).cpu()
    assert bool((outside == 7.0).all())


def test_forward_then_vjp_and_autograd():
    B, V = 24, 3001
    logits, target = workloads.small_ce(B, V, torch.float32, sigma=2.0, n_ignored=5, seed=4)
    g = workloads.row_upstream(B, seed=4)
    x = logits.to(DEV).requires_grad_(True)
    loss = F.cross_entropy_per_row(x, target.to(DEV), -100)
    (loss * g.to(DEV)).sum().backward()
    torch.cuda.synchronize()
    _rows_close(loss.detach(), oracle.cross_entropy_per_row(logits, target, -100))
    _vjp_close(x.grad, oracle.cross_entropy_per_row_vjp(logits, target, g.double(), -100), g,
               torch.float32)


def test_edge_cases():
    # an out-of-range index flags and gives 0; B = 0 is a no-op
    logits, index = workloads.small_ce(4, 100, torch.bfloat16, seed=1)
    index[2] = 100
    out = F.selective_log_softmax(logits.to(DEV), index.to(DEV))
    torch.cuda.synchronize()
    assert float(out[2]) == 0.0
    keep = torch.tensor([0, 1, 3])
    _rows_close(out.cpu()[keep], oracle.selective_log_softmax(logits[keep], index[keep]))
    empty = torch.empty(0, 100, dtype=torch.bfloat16, device=DEV)
    assert F.selective_log_softmax(empty, torch.empty(0, dtype=torch.int64)).shape == (0,)
    # all rows ignored: zero losses, zero gradient rows
    t = torch.full((4,), -100, dtype=torch.int64)
    loss, n, bad = F.ce_loss_rows(logits.to(DEV), t.to(DEV), -100)
    grad = F.ce_loss_rows_vjp(logits.to(DEV), t.to(DEV), loss, torch.ones(4, device=DEV), -100)
    torch.cuda.synchronize()
    assert int(n) == 0 and bool((loss == 0).all()) and bool((grad == 0).all())


@pytest.mark.slow
def test_full_size_rows_sampled():
    """[16384, 128256] bf16 with 2% ignored rows: all three entry points on the
    whole batch (the VJP in place), checked on sampled rows."""
    w = workloads.CE_B16384_V128256_BF16
    logits, target = workloads.ce_inputs(w)
    rows = torch.tensor([0, 1, 777, 4095, 8191, 12000, 16383]
                        + torch.nonzero(target == -100)[:3, 0].tolist())
    x = logits.to(DEV)
    t = target.to(DEV)
    lp = F.selective_log_softmax(x, torch.clamp(t, min=0))
    loss, n, bad = F.ce_loss_rows(x, t, -100)
    g = workloads.row_upstream(w.B, seed=1)
    loss_in = oracle.cross_entropy_per_row(logits[rows], target[rows], -100).float()
    full_loss_in = torch.zeros(w.B, dtype=torch.float32)
    full_loss_in[rows] = loss_in
    F.ce_loss_rows_vjp(x, t, full_loss_in.to(DEV), g.to(DEV), -100, in_place=True)
    torch.cuda.synchronize()
    assert int(n) == w.B - w.n_ignored and int(bad) == 0
    _rows_close(lp.cpu()[rows], oracle.selective_log_softmax(logits[rows],
                                                              torch.clamp(target[rows], min=0)))
    _rows_close(loss.cpu()[rows], oracle.cross_entropy_per_row(logits[rows], target[rows], -100))
    ref = oracle.cross_entropy_per_row_vjp(logits[rows], target[rows], g[rows].double(), -100)
    _vjp_close(x[rows.to(DEV)], ref, g[rows], torch.bfloat16)


def test_selective_log_softmax_any_leading_shape():
    # the page's entry takes logits [..., V] and index [...]
    logits, index = workloads.small_ce(24, 1001, torch.bfloat16, sigma=2.0, seed=31)
    ref = oracle.selective_log_softmax(logits, index)
    out3 = F.selective_log_softmax(logits.view(2, 3, 4, 1001).to(DEV), index.view(2, 3, 4).to(DEV))
    out1 = F.selective_log_softmax(logits[5].to(DEV), index[5].to(DEV))
    torch.cuda.synchronize()
    assert out3.shape == (2, 3, 4) and out1.shape == ()
    _rows_close(out3.reshape(-1), ref)
    _rows_close(out1.reshape(1), ref[5:6])
    with pytest.raises(ValueError):
        F.selective_log_softmax(logits.view(2, 12, 1001).to(DEV), index.to(DEV))
