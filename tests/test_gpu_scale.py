"""GPU checks of lmx_scale, the upstream-gradient step of the reduced losses'
autograd wrappers (needs an MI355X).

lmx_scale computes RNE_dtype(fp32(x * s)): the expected values are formed on
the host in fp64 (the product of two fp32 values is exact there), rounded to
fp32, then to the 16-bit format with the oracle's round-to-nearest-even
functions, so the comparison is bitwise. The autograd cases check that an fp16
loss scale of 2^16 (above fp16's largest finite value) reaches the gradients
intact.
"""
import pytest
import torch

import oracle
import workloads
from lm_head_cross_pass_amd import _lib
from lm_head_cross_pass_amd import functional as F

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CODES = {torch.float32: _lib.LMX_F32, torch.bfloat16: _lib.LMX_BF16, torch.float16: _lib.LMX_F16}


def _expected(x: torch.Tensor, s: float) -> torch.Tensor:
    p = (x.double() * torch.tensor(s, dtype=torch.float32).double()).float().double()
    if x.dtype == torch.bfloat16:
        return oracle.round_to_bf16(p)
    if x.dtype == torch.float16:
        return oracle.round_to_fp16(p)
    return p


@pytest.mark.parametrize("dtype", (torch.float32, torch.bfloat16, torch.float16))
@pytest.mark.parametrize("n,offset", ((1, 0), (7, 0), (4099, 0), (4099, 1), (100003, 3)))
@pytest.mark.parametrize("s", (1.0 / 3.0, 65536.0, -2.5e-3))
def test_scale_bitwise(dtype, n, offset, s):
    g = torch.Generator().manual_seed(n + offset)
    x = (torch.randn(n + offset, generator=g) * 3.0).to(dtype)
    xd = x.to(DEV)
    src = xd[offset:]
    out = torch.empty(n + 5, dtype=dtype, device=DEV)[offset:offset + n]   # misaligned too
    sc = torch.tensor(s, dtype=torch.float32, device=DEV)
    st = _lib.lmx_scale(src.data_ptr(), out.data_ptr(), n, CODES[dtype], sc.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    assert st == _lib.LMX_OK
    torch.cuda.synchronize()
    exp = _expected(x[offset:], s)
    got = out.double().cpu()
    same = (got == exp) | (torch.isinf(got) & torch.isinf(exp) & (torch.sign(got) == torch.sign(exp)))
    assert bool(same.all()), int((~same).sum())
    # in place gives the same values
    st = _lib.lmx_scale(src.data_ptr(), src.data_ptr(), n, CODES[dtype], sc.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(src, out)


def test_fp16_loss_scale_reaches_the_linear_gradients():
    from lm_head_cross_pass_amd import linear_cross_entropy
    X, W, t = workloads.small_linear_ce(128, 64, 500, dtype=torch.float16, n_ignored=3, seed=17)
    scale = 65536.0
    Xd = X.to(DEV).requires_grad_(True)
    Wd = W.to(DEV).requires_grad_(True)
    # mean over 125 tokens keeps every scaled gradient well inside fp16's range;
    # the scale itself is not an fp16 value
    loss = linear_cross_entropy(Xd, Wd, t.to(DEV), -100, "mean", 0.0, chunk_size=32)
    (loss * scale).backward()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Xd.grad).all()) and bool(torch.isfinite(Wd.grad).all())
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 0.0)
    for got, exact in ((Xd.grad, ref["grad_inputs"]), (Wd.grad, ref["grad_weight"])):
        e = scale * exact
        rel = float((got.double().cpu() - e).norm() / e.norm())
        assert rel <= 2e-3, rel


def test_fp16_loss_scale_reaches_the_ce_gradient():
    from lm_head_cross_pass_amd import cross_entropy
    logits, target = workloads.small_ce(16, 3001, dtype=torch.float16, n_ignored=2, seed=9)
    x = logits.to(DEV).requires_grad_(True)
    loss = cross_entropy(x, target.to(DEV), -100, "mean", 0.0)
    (loss * 65536.0).backward()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(x.grad).all())
    ref = oracle.cross_entropy(logits, target, -100, "mean", 0.0)
    e = 65536.0 * ref["grad"]
    rel = float((x.grad.double().cpu() - e).norm() / e.norm())
    assert rel <= 1e-3, rel
