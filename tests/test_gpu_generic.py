"""GPU parity of the generic chunked linear loss (linear_loss_logits /
linear_loss_grads through ``chunked_linear_loss``) against the fp64 oracle.

The loss-and-gradient functions are the caller's: a sum-of-squares loss through
``autograd_loss_and_logits_grad`` (torch autograd on the chunk), torch's
cross-entropy the same way, and the library's own cross-entropy
(``cross_entropy_loss_and_grad``). The logits are bf16 (the matmuls' dtype), so
the bars are those of the bf16 linear path: loss within 5e-3 relative (2e-3 for
cross-entropy), each gradient within 1e-2 relative Frobenius norm; the same
bars hold for fp16 logits, whose rounding is finer. Y (the regression targets)
and the other inputs come from the seeded generators.
"""
import pytest
import torch
import torch.nn.functional as TF

import oracle
from oracle import generic as ogen
import workloads
from lm_head_cross_pass_amd import functional as F

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _rel(got, ref):
    got = got.double().cpu()
    n = float(ref.norm())
    return float((got - ref).norm()) / n if n > 0 else float(got.norm())


def _mse(z, y):
    return TF.mse_loss(z.float(), y, reduction="sum")


@pytest.mark.parametrize("BT,D,V,chunk", [(96, 64, 512, 32), (100, 72, 336, 37),
                                          (257, 128, 4096, 100), (64, 64, 1000, 0)])
@pytest.mark.parametrize("accum", ("fp32", "weight"))
@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16))
def test_sum_of_squares_loss(BT, D, V, chunk, accum, dtype):
    X, W, _ = workloads.small_linear_ce(BT, D, V, dtype=dtype, seed=BT + V, sigma_w=0.1)
    Y = workloads.row_upstream(BT * V, seed=V).reshape(BT, V) * 0.5
    loss, gx, gw = F.chunked_linear_loss_fwd(X.to(DEV), W.to(DEV),
                                             F.autograd_loss_and_logits_grad(_mse), (Y.to(DEV),),
                                             chunk_size=chunk or None,
                                             grad_weight_accum_dtype=accum)
    torch.cuda.synchronize()
    ref = ogen.linear_loss(X, W, ogen.mse_sum, Y)
    assert float(loss) == pytest.approx(ref["loss"], rel=5e-3)
    assert _rel(gx, ref["grad_inputs"]) <= 1e-2
    assert _rel(gw, ref["grad_weight"]) <= 1e-2


@pytest.mark.parametrize("how", ("library", "torch"))
@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16))
def test_cross_entropy_through_the_generic_path(how, dtype):
    BT, D, V = 300, 96, 2048
    X, W, t = workloads.small_linear_ce(BT, D, V, dtype=dtype, n_ignored=15, seed=9)
    if how == "library":
        fn = F.cross_entropy_loss_and_grad
    else:
        fn = F.autograd_loss_and_logits_grad(
            lambda z, tt: TF.cross_entropy(z.float(), tt, ignore_index=-100, reduction="sum"))
    loss, gx, gw = F.chunked_linear_loss_fwd(X.to(DEV), W.to(DEV), fn, (t.to(DEV),),
                                             chunk_size=64)
    torch.cuda.synchronize()
    ref = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0)
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx, ref["grad_inputs"]) <= 1e-2
    assert _rel(gw, ref["grad_weight"]) <= 1e-2


def test_generic_matches_fused_linear_ce():
    # the library's CE through the generic path against the fused linear_ce
    BT, D, V = 512, 128, 4096
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=20, seed=3)
    Xd, Wd, td = X.to(DEV), W.to(DEV), t.to(DEV)
    loss_g, gx_g, gw_g = F.chunked_linear_loss_fwd(Xd, Wd, F.cross_entropy_loss_and_grad, (td,),
                                                   chunk_size=128)
    loss_f, gx_f, gw_f, _, _ = F.linear_ce(Xd, Wd, td, -100, "sum", 0.0, 128, "fp32")
    torch.cuda.synchronize()
    assert float(loss_g) == pytest.approx(float(loss_f), rel=1e-5)
    assert _rel(gx_g, gx_f.double().cpu()) <= 1e-2
    assert _rel(gw_g, gw_f.double().cpu()) <= 1e-2


def test_autograd_and_argument_slicing():
    BT, D, V = 128, 64, 256
    X, W, _ = workloads.small_linear_ce(BT, D, V, seed=2, sigma_w=0.1)
    Y = workloads.row_upstream(BT * V, seed=2).reshape(BT, V)
    scale = 0.5
    Xd = X.to(DEV).requires_grad_(True)
    Wd = W.to(DEV).requires_grad_(True)
    loss = F.chunked_linear_loss(Xd, Wd, F.autograd_loss_and_logits_grad(_mse), Y.to(DEV),
                                 chunk_size=48)
    (loss * scale).backward()
    torch.cuda.synchronize()
    ref = ogen.linear_loss(X, W, ogen.mse_sum, Y)
    assert float(loss.detach()) == pytest.approx(ref["loss"], rel=5e-3)
    assert _rel(Xd.grad, scale * ref["grad_inputs"]) <= 1e-2
    assert _rel(Wd.grad, scale * ref["grad_weight"]) <= 1e-2


def test_vocabulary_must_give_16_byte_gradient_rows():
    X, W, _ = workloads.small_linear_ce(32, 64, 1001, seed=1)
    with pytest.raises(ValueError):
        F.chunked_linear_loss_fwd(X.to(DEV), W.to(DEV), F.cross_entropy_loss_and_grad,
                                  (torch.zeros(32, dtype=torch.int64, device=DEV),))


def test_grouped_grad_weight_products_generic():
    """Nine chunks of 2048 rows at V = 128256 through the generic path: fp32
    accumulation takes the grad_weight product once per group of four chunks
    (the group's G^T columns wait in the workspace between calls): a first
    group, a middle group, then the last chunk alone; checked against the
    oracle on sampled rows and against the fused linear_ce on everything."""
    from oracle import linear_ce as olce
    BT, D, V, C = 9 * 2048, 64, 128256, 2048
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=200, seed=13)
    Xd, Wd, td = X.to(DEV), W.to(DEV), t.to(DEV)
    loss, gx, gw = F.chunked_linear_loss_fwd(Xd, Wd, F.cross_entropy_loss_and_grad, (td,),
                                             chunk_size=C)
    loss_f, gx_f, gw_f, _, _ = F.linear_ce(Xd, Wd, td, -100, "sum", 0.0, C, "fp32")
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(5)
    rows = torch.randperm(BT, generator=g)[:16].tolist()
    vrows = torch.randperm(V, generator=g)[:16].tolist() + [int(t[rows[0]]), V - 1]
    ref = olce.linear_cross_entropy_sampled(X, W, t, rows, vrows, -100, "sum", 0.0,
                                            block_rows=1024)
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx.cpu()[rows], ref["grad_inputs_rows"]) <= 1e-2
    assert _rel(gw.cpu()[vrows], ref["grad_weight_rows"]) <= 1e-2
    assert float(loss) == pytest.approx(float(loss_f), rel=1e-5)
    assert _rel(gx, gx_f.double().cpu()) <= 1e-2
    assert _rel(gw, gw_f.double().cpu()) <= 1e-2


@pytest.mark.parametrize("accum", ("fp32", "weight"))
def test_workspace_contents_do_not_matter_generic(accum):
    # three chunks, the last ragged: a workspace full of NaN bit patterns gives
    # the same bits as a zeroed one (every padding entry read is written first)
    from lm_head_cross_pass_amd import _lib
    BT, D, V, C = 250, 72, 776, 100
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=6, seed=29)
    Xd, Wd, td = X.to(DEV), W.to(DEV), t.to(DEV)
    nbytes = _lib.linear_loss_workspace_bytes(BT, D, V, _lib.LMX_BF16, C,
                                              0 if accum == "fp32" else 1)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        outs.append(F.chunked_linear_loss_fwd(Xd, Wd, F.cross_entropy_loss_and_grad, (td,),
                                              chunk_size=C, grad_weight_accum_dtype=accum,
                                              workspace=ws))
    torch.cuda.synchronize()
    a, b = outs
    assert float(a[0]) == float(b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert not bool(torch.isnan(a[2].float()).any())


@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16))
def test_split_tail_launches_generic(dtype):
    # D = 768 and V = 50256: the chunk's logits product has 4 x 197 large tiles,
    # so its last columns go to a second launch on small tiles; grad_weight is
    # one product over both chunks (K = 2048) whose last wave of rows runs as
    # large tiles with K split in three, summed by the tail reduction
    BT, D, V = 2048, 768, 50256
    X, W, t = workloads.small_linear_ce(BT, D, V, dtype=dtype, n_ignored=30, seed=41)
    loss, gx, gw = F.chunked_linear_loss_fwd(X.to(DEV), W.to(DEV), F.cross_entropy_loss_and_grad,
                                             (t.to(DEV),), chunk_size=1024)
    torch.cuda.synchronize()
    ref = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0, block_rows=512)
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx, ref["grad_inputs"]) <= 1e-2
    assert _rel(gw, ref["grad_weight"]) <= 1e-2


@pytest.mark.parametrize("rows,D,V,ld,offset", [
    (37, 64, 1000, 1000, 0),     # 16-byte rows: the packed product, staged stores
    (300, 136, 2000, 2008, 0),   # staged, padding columns past V
    (37, 64, 1001, 1001, 0),     # odd V: element stores through the LDS product
    (130, 72, 777, 784, 0),      # odd V with padding columns
    (300, 136, 1000, 1000, 1),   # logits two bytes past a 16-byte boundary
])
@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16))
def test_chunk_logits_through_the_c_abi(rows, D, V, ld, offset, dtype):
    """linear_loss_logits called directly: every logit of the chunk against
    inputs @ weight.T in fp64, element by element. The kernel's products of
    16-bit operands are exact in fp32 and the fp32 sum over D errs by at most
    D * 2^-24 * (|x| @ |w|^T); rounding to the output format then adds half an
    ulp (2^-8 relative for bf16, 2^-11 for fp16). Columns past V keep their
    sentinel."""
    from lm_head_cross_pass_amd import _lib
    X, W, _ = workloads.small_linear_ce(rows, D, V, dtype=dtype, seed=rows + V)
    code = _lib.LMX_BF16 if dtype == torch.bfloat16 else _lib.LMX_F16
    half_ulp = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    Xd, Wd = X.to(DEV), W.to(DEV)
    sentinel = -7.0
    buf = torch.full((rows * ld + offset,), sentinel, dtype=dtype, device=DEV)
    out = buf[offset:].view(rows, ld)
    nbytes = _lib.linear_loss_logits_workspace_bytes(rows, D, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    _lib.check("linear_loss_logits", _lib.linear_loss_logits(
        Xd.data_ptr(), Wd.data_ptr(), rows, D, V, code, out.data_ptr(), ld,
        ws.data_ptr(), nbytes, stream))
    torch.cuda.synchronize()
    got = out.double().cpu()
    Xf, Wf = X.double(), W.double()
    ref = Xf @ Wf.T
    acc_err = D * 2.0 ** -24 * (Xf.abs() @ Wf.abs().T)
    bound = acc_err + half_ulp * (ref.abs() + acc_err)
    err = (got[:, :V] - ref).abs()
    assert bool((err <= bound).all()), float((err - bound).max())
    assert bool((got[:, V:] == sentinel).all())
    assert bool((buf[:offset].double().cpu() == sentinel).all())
