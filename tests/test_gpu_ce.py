"""GPU parity of ce_fwd_bwd against the fp64 oracle (needs an MI355X).

Tolerances (stated with the method's workloads):
* fp32 logits: loss within 1e-5 relative, gradient within 1e-6 absolute;
* bf16 logits: loss within 2e-3 relative, gradient within 1e-2 relative
  Frobenius norm ||g - g*|| / ||g*||, plus an element-wise bound of one bf16
  rounding on top of the fp32 arithmetic: |g - g*| <= (2^-8 + delta) |g*|,
  plus delta c at the target entry, delta the relative error of the kernel's
  fp32 exponent argument (about 2^-22 times the size of its parts: the row
  max, log2 of the scale and of V) and c = scale (1 + 2 z lse) (see
  _elementwise_bound);
* fp16 logits: the loss is fp32 arithmetic on exact inputs, so within 1e-5
  relative as for fp32; the gradient is rounded once to fp16, so within 1e-3
  relative Frobenius plus ||fp16(g*) - g*|| (the format's own rounding, which
  dominates when a mean over many rows puts most p/N among fp16's subnormals)
  and |g - g*| <= (2^-10 + delta) |g*| + 2^-25 (+ delta c at the target entry)
  element-wise (2^-25 is half the spacing of fp16 subnormals);
* the valid-token count N is compared exactly.
Inputs are the seeded workloads of ``workloads.py``; the oracle computes on the
same host bit patterns.
"""
import math

import pytest
import torch

import oracle
import workloads
from lm_head_cross_pass_amd import _lib
from lm_head_cross_pass_amd import functional as F

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check(logits, target, red, z, got_loss, got_grad, got_n, rows=None, ref=None):
    if ref is None:
        ref = oracle.cross_entropy(logits, target, -100, red, z)
    assert int(got_n) == ref["n_valid"]
    rl = float(got_loss)
    if math.isnan(ref["loss"]):
        assert math.isnan(rl)
    elif logits.dtype in (torch.float32, torch.float16):
        assert rl == pytest.approx(ref["loss"], rel=1e-5, abs=1e-30)
    else:
        assert rl == pytest.approx(ref["loss"], rel=2e-3, abs=1e-30)
    if got_grad is None:
        return
    g = got_grad.double().cpu()
    gs = ref["grad"]
    if rows is not None:
        g = g[rows]
    if logits.dtype == torch.float32:
        assert float((g - gs).abs().max()) <= 1e-6
    else:
        fp16 = logits.dtype == torch.float16
        n = float(gs.norm())
        if n > 0:
            # fp16: plus the output format's own rounding of the oracle's values
            # (a mean over many rows puts most p / N below fp16's normal range)
            fmt = float((gs.to(torch.float16).double() - gs).norm()) if fp16 else 0.0
            assert float((g - gs).norm()) <= (1e-3 if fp16 else 1e-2) * n + fmt
        scale = 1.0 / max(ref["n_valid"], 1) if red == "mean" else 1.0
        bound = _elementwise_bound(gs, logits if rows is None else logits[rows],
                                   target if rows is None else target[rows], scale, z, fp16)
        assert bool(((g - gs).abs() <= bound).all()), float(((g - gs).abs() - bound).max())


def _elementwise_bound(gs, logits, target, scale, z, fp16):
    """|g - g*| allowed per entry: one rounding to the output format on top of
    the fp32 arithmetic. The kernel takes p c = exp2(x log2 e - (m log2 e +
    log2 s - log2 c)) (c = scale (1 + 2 z lse), m the row max, s the sum of
    exponentials): the argument's fp32 rounding gives p c a relative error of
    about 2^-24 ln 2 times the size of its parts, delta below (with a factor
    of 4 to spare). That error enters every entry relative to its value (it can
    move a value across a rounding midpoint), and at the target entry, where
    p c - scale cancels when p is near 1, relative to p c, i.e. up to delta c."""
    x = logits.double()
    m = x.max(dim=1).values.abs()
    lse = torch.logsumexp(x, dim=1)
    c = (scale * (1.0 + 2.0 * z * lse)).abs()
    V = x.shape[1]
    delta = 2.0 ** -22 * (1.0 + m / math.log(2.0) + abs(math.log2(scale)) + math.log2(V))
    bound = ((2.0 ** -10 if fp16 else 2.0 ** -8) + delta[:, None]) * gs.abs()
    if fp16:
        bound = bound + 2.0 ** -25
    rows = ((target >= 0) & (target < V)).nonzero().flatten()
    bound[rows, target[rows]] += (delta * c)[rows]
    return bound


def _run(logits, target, red, z, in_place=False, want_grad=True):
    x = logits.to(DEV)
    loss, grad, n, bad = F.ce_fwd_bwd(x, target.to(DEV), -100, red, z, want_grad=want_grad,
                                      in_place=in_place)
    torch.cuda.synchronize()
    return loss, grad, n, bad, x


@pytest.mark.parametrize("z", (0.0, 1e-4))
@pytest.mark.parametrize("red", ("mean", "sum"))
def test_small_fp32_workload(z, red):
    w = workloads.CE_B8_V1000_F32
    logits, target = workloads.ce_inputs(w)
    loss, grad, n, bad, _ = _run(logits, target, red, z)
    _check(logits, target, red, z, loss, grad, n)
    assert int(bad) == 0
    loss2, grad2, n2, _, x = _run(logits, target, red, z, in_place=True)
    assert torch.equal(grad2, grad) and float(loss2) == float(loss)


SHAPES = [
    (3, 1, torch.float32), (5, 7, torch.bfloat16), (5, 9, torch.float32),
    (7, 2041, torch.bfloat16), (7, 2048, torch.bfloat16), (9, 2049, torch.bfloat16),
    (64, 4097, torch.bfloat16), (130, 1000, torch.float32), (33, 50257, torch.bfloat16),
    (17, 50257, torch.float32), (11, 65536, torch.float32), (4, 131073, torch.bfloat16),
    (6, 70001, torch.float32), (5, 128256, torch.bfloat16),
    (5, 7, torch.float16), (7, 2041, torch.float16), (9, 2049, torch.float16),
    (33, 50257, torch.float16), (4, 131073, torch.float16), (5, 128256, torch.float16),
]


@pytest.mark.parametrize("B,V,dtype", SHAPES)
def test_shapes_against_oracle(B, V, dtype):
    logits, target = workloads.small_ce(B, V, dtype=dtype, sigma=3.0,
                                        n_ignored=min(2, B - 1), seed=B * 7 + V, boost=8.0)
    for red, z in (("mean", 1e-4), ("sum", 0.0)):
        ref = oracle.cross_entropy(logits, target, -100, red, z)
        loss, grad, n, bad, _ = _run(logits, target, red, z)
        _check(logits, target, red, z, loss, grad, n, ref=ref)
        assert int(bad) == 0
        loss2, grad2, _, _, _ = _run(logits, target, red, z, in_place=True)
        assert torch.equal(grad2, grad), "in place differs from out of place"
        assert float(loss2) == float(loss)
        # the loss-only path folds each chunk into a running max / rescaled sum
        # (one sweep), so it matches the two-sweep value up to fp32 rounding
        loss3, g3, _, _, _ = _run(logits, target, red, z, want_grad=False)
        assert g3 is None
        _check(logits, target, red, z, loss3, None, n, ref=ref)
        assert float(loss3) == pytest.approx(float(loss), rel=2e-6, abs=1e-30)


@pytest.mark.parametrize("B,V,dtype", ((1000, 50257, torch.bfloat16),
                                        (1000, 50257, torch.float16),
                                        (1000, 20000, torch.float32)))
def test_more_rows_than_resident_workgroups(B, V, dtype):
    """1000 rows of up to 6656 16-byte chunks: the row kernel of this width
    runs two 512-thread workgroups per CU (512 on 256 CUs), so some workgroups
    walk a second row; every row against the oracle, in place and out of place,
    both reductions. (The linear-CE chunk rows take its instance with three
    workgroups per CU; the linear-CE tests at V = 50257 cover it.)"""
    logits, target = workloads.small_ce(B, V, dtype=dtype, sigma=3.0, n_ignored=50,
                                        seed=17, boost=8.0)
    for red, z in (("mean", 1e-4), ("sum", 0.0)):
        ref = oracle.cross_entropy(logits, target, -100, red, z)
        loss, grad, n, bad, _ = _run(logits, target, red, z)
        _check(logits, target, red, z, loss, grad, n, ref=ref)
        assert int(bad) == 0
        loss2, grad2, _, _, _ = _run(logits, target, red, z, in_place=True)
        assert torch.equal(grad2, grad) and float(loss2) == float(loss)


@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16, torch.float32))
def test_many_short_rows(dtype):
    """100000 rows of 7 classes: far more rows than resident workgroups, so
    each workgroup walks a hundred rows or more; every row against the
    oracle, in place and out of place, both reductions."""
    logits, target = workloads.small_ce(100000, 7, dtype=dtype, sigma=3.0, n_ignored=5000,
                                        seed=23)
    for red, z in (("mean", 1e-4), ("sum", 0.0)):
        ref = oracle.cross_entropy(logits, target, -100, red, z)
        loss, grad, n, bad, _ = _run(logits, target, red, z)
        _check(logits, target, red, z, loss, grad, n, ref=ref)
        assert int(bad) == 0
        loss2, grad2, _, _, _ = _run(logits, target, red, z, in_place=True)
        assert torch.equal(grad2, grad) and float(loss2) == float(loss)


@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16))
def test_misaligned_rows_and_base(dtype):
    # 16-bit rows of odd width, starting 2 bytes past a 16-byte boundary
    B, V = 12, 50257
    logits, target = workloads.small_ce(B + 1, V, dtype=dtype, sigma=3.0, n_ignored=2,
                                        seed=3)
    full = logits.to(DEV)
    view = full.view(-1)[1:1 + B * V].view(B, V)           # base offset of one element
    t = target[:B].to(DEV)
    ref_logits = full.view(-1)[1:1 + B * V].view(B, V).cpu()
    grad = torch.empty((B * V + 8,), dtype=dtype, device=DEV)[1:1 + B * V].view(B, V)
    loss, g, n, bad = F.ce_fwd_bwd(view, t, -100, "mean", 1e-4, grad=grad)
    _check(ref_logits, target[:B], "mean", 1e-4, loss, g, n)
    before = full.clone()
    loss2, g2, _, _ = F.ce_fwd_bwd(view, t, -100, "mean", 1e-4, in_place=True)
    assert torch.equal(view, g)
    # the element before the view was not touched
    assert torch.equal(full.view(-1)[:1], before.view(-1)[:1])


def test_edge_cases():
    V = 300
    logits, _ = workloads.small_ce(4, V, dtype=torch.float32, seed=11)
    allign = torch.full((4,), -100)
    loss, grad, n, bad, _ = _run(logits, allign, "mean", 0.0)
    assert math.isnan(float(loss)) and int(n) == 0 and bool((grad == 0).all())
    loss, grad, n, bad, _ = _run(logits, allign, "sum", 0.0)
    assert float(loss) == 0.0 and bool((grad == 0).all())
    # ignore_index inside [0, V) takes precedence over being a class
    t = torch.tensor([5, 7, 5, 2])
    x = logits.to(DEV)
    loss, grad, n, bad = F.ce_fwd_bwd(x, t.to(DEV), 5, "mean", 0.0)
    ref = oracle.cross_entropy(logits, t, 5, "mean", 0.0)
    assert int(n) == ref["n_valid"] == 2
    assert float(loss) == pytest.approx(ref["loss"], rel=1e-5)
    assert float((grad.double().cpu() - ref["grad"]).abs().max()) <= 1e-6
    # out-of-range valid targets: flagged, treated as ignored
    t = torch.tensor([1, V, -3, 2])
    loss, grad, n, bad = F.ce_fwd_bwd(x, t.to(DEV), -100, "sum", 0.0)
    assert int(bad) == 1 and int(n) == 2
    assert bool((grad[1] == 0).all()) and bool((grad[2] == 0).all())
    tt = torch.tensor([1, -100, -100, 2])
    ref = oracle.cross_entropy(logits, tt, -100, "sum", 0.0)
    assert float(loss) == pytest.approx(ref["loss"], rel=1e-5)


def test_empty_batch():
    x = torch.empty((0, 17), dtype=torch.bfloat16, device=DEV)
    t = torch.empty((0,), dtype=torch.int64, device=DEV)
    loss, grad, n, bad = F.ce_fwd_bwd(x, t, -100, "mean", 0.0)
    assert math.isnan(float(loss)) and int(n) == 0 and int(bad) == 0
    loss, grad, n, bad = F.ce_fwd_bwd(x, t, -100, "sum", 0.0)
    assert float(loss) == 0.0


def test_extreme_logits():
    # large offsets, -inf entries, and one dominant logit (closed form)
    V = 5000
    x = torch.zeros(4, V)
    x[0] += 3.0e4                      # shift: lse - x_t is log V
    x[1, 10] = 12.0                    # one dominant logit
    x[2, ::2] = -float("inf")          # half the row impossible
    x[3] = torch.linspace(-80, 80, V)
    t = torch.tensor([3, 10, 1, 4999])
    for dtype in (torch.float32, torch.bfloat16, torch.float16):
        xl = x.to(dtype)
        loss, grad, n, bad, _ = _run(xl, t, "sum", 0.0)
        ref = oracle.cross_entropy(xl, t, -100, "sum", 0.0)
        assert math.isfinite(float(loss))
        tol = 2e-3 if dtype == torch.bfloat16 else 1e-5
        assert float(loss) == pytest.approx(ref["loss"], rel=tol)
        assert bool(torch.isfinite(grad).all())
        assert bool((grad[2, ::2] == 0).all())


def test_autograd_wrappers():
    from lm_head_cross_pass_amd import cross_entropy, cross_entropy_
    logits, target = workloads.small_ce(16, 3001, dtype=torch.float32, n_ignored=3, seed=5)
    x = logits.to(DEV).requires_grad_(True)
    loss = cross_entropy(x, target.to(DEV), -100, "mean", 1e-4)
    (2.5 * loss).backward()
    ref = oracle.cross_entropy(logits, target, -100, "mean", 1e-4)
    assert float(loss.detach()) == pytest.approx(ref["loss"], rel=1e-5)
    assert float((x.grad.double().cpu() - 2.5 * ref["grad"]).abs().max()) <= 3e-6
    assert torch.equal(x.detach().cpu(), logits)          # not mutated
    y = logits.to(DEV)
    l2 = cross_entropy_(y, target.to(DEV), -100, "mean", 1e-4)
    assert float(l2) == float(loss.detach())
    assert float((y.double().cpu() - ref["grad"]).abs().max()) <= 1e-6


def test_repeatable_bitwise():
    logits, target = workloads.small_ce(257, 32001, dtype=torch.bfloat16, n_ignored=9, seed=8)
    a = _run(logits, target, "mean", 1e-4)
    b = _run(logits, target, "mean", 1e-4)
    assert float(a[0]) == float(b[0]) and torch.equal(a[1], b[1])


def test_workload_b4096_v50257_bf16_full():
    w = workloads.CE_B4096_V50257_BF16
    logits, target = workloads.ce_inputs(w)
    z, red = w.z_loss[0], w.reductions[0]
    loss, grad, n, bad, _ = _run(logits, target, red, z)
    assert int(n) == w.B - w.n_ignored == 3891
    _check(logits, target, red, z, loss, grad, n)


@pytest.mark.slow
def test_workload_b16384_v128256_bf16_inplace_full():
    """The headline workload, gradient written over the logits, compared with the
    oracle on every row: element-wise (one bf16 rounding on top of the fp32
    arithmetic) and by the relative Frobenius norm over the whole gradient;
    ignored rows exactly zero; loss and N over all rows."""
    w = workloads.CE_B16384_V128256_BF16
    logits, target = workloads.ce_inputs(w)
    z, red = w.z_loss[0], w.reductions[0]
    x = logits.to(DEV)
    loss, grad, n, bad = F.ce_fwd_bwd(x, target.to(DEV), -100, red, z, in_place=True)
    torch.cuda.synchronize()
    assert grad.data_ptr() == x.data_ptr()
    assert int(n) == 16056 and int(bad) == 0
    g_host = grad.cpu()
    del x, grad
    n_valid, valid = oracle.count_valid(target, -100, w.V)
    scale = 1.0 / n_valid if red == "mean" else 1.0
    num2 = den2 = 0.0
    row_loss = []
    for r0 in range(0, w.B, 1024):
        r1 = min(w.B, r0 + 1024)
        _, rl, gref = oracle.cross_entropy_rows(logits[r0:r1], target[r0:r1], valid[r0:r1],
                                                scale, z)
        row_loss += rl.tolist()
        d = g_host[r0:r1].double() - gref
        num2 += float((d * d).sum())
        den2 += float((gref * gref).sum())
        bound = _elementwise_bound(gref, logits[r0:r1], target[r0:r1], scale, z, False)
        assert bool((d.abs() <= bound).all()), (r0, float((d.abs() - bound).max()))
        ign = ~valid[r0:r1]
        assert bool((g_host[r0:r1][ign] == 0).all())
    assert math.sqrt(num2 / den2) <= 1e-2
    ref_loss = math.fsum(row_loss)
    assert float(loss) == pytest.approx(ref_loss / (n_valid if red == "mean" else 1), rel=2e-3)
