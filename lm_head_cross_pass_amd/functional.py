"""PyTorch-facing functions over liblmx.so (greyhound functional API page).

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's kernels. The functions:

* ``cross_entropy``  -- loss from materialized logits with normal autograd
  behaviour; the logits are not modified (page entry ``cross_entropy``);
* ``cross_entropy_`` -- the raw helper: returns the loss and overwrites the
  logits with their gradient (upstream gradient 1);
* ``linear_cross_entropy`` -- chunked ``inputs @ weight.T`` cross-entropy with
  gradients for inputs and weight (page entries ``chunked_linear_loss`` and
  ``chunked_linear_cross_entropy``; ``chunk_size`` as in the former), and
  ``chunked_linear_cross_entropy`` with that entry's own signature;
* ``chunked_linear_loss`` with ``autograd_loss_and_logits_grad`` -- the
  generic chunked linear loss: the library computes each chunk's logits and,
  from the caller's logits gradient, the chunk's grad_inputs rows and its
  share of grad_weight (page entries ``chunked_linear_loss`` and
  ``autograd_loss_and_logits_grad``); ``cross_entropy_loss_and_grad`` is the
  library's cross-entropy in that loss-and-gradient form;
* ``selective_log_softmax`` -- one log-probability per row of ``[..., V]``
  logits (page entry ``selective_log_softmax``);
* ``cross_entropy_per_row`` -- the unreduced per-row cross-entropy whose
  backward is the separate vector-Jacobian product call (nuvec ``FastOp``
  page, ``CrossEntropy`` / ``CrossEntropyVjp``).

For the reduced losses the gradients are produced in the forward call (one
pass) and backward only scales them by the upstream scalar gradient; the
per-row loss instead runs its own backward pass, since its upstream gradient
is a vector.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from lm_head_cross_pass_amd import _lib

_DTYPES = {torch.float32: _lib.LMX_F32, torch.bfloat16: _lib.LMX_BF16,
           torch.float16: _lib.LMX_F16}
_LINEAR_DTYPES = {torch.bfloat16: _lib.LMX_BF16, torch.float16: _lib.LMX_F16}
_REDUCTIONS = {"mean": _lib.LMX_MEAN, "sum": _lib.LMX_SUM}
_ACCUMS = {"fp32": _lib.LMX_ACC_F32, "weight": _lib.LMX_ACC_WEIGHT}


def _require_device(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    # the caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _scaled(t: torch.Tensor, g: torch.Tensor) -> torch.Tensor:
    """``t * g`` for the upstream scalar gradient ``g`` of a reduced loss: a new
    tensor, the product taken in fp32 by the library (so a large fp16 loss scale
    does not overflow and ``g`` is not first rounded to 16 bits)."""
    out = torch.empty_like(t)
    if t.numel() == 0:
        return out
    s = g.detach().to(device=t.device, dtype=torch.float32).reshape(()).contiguous()
    with torch.cuda.device(t.device):
        st = _lib.lmx_scale(t.data_ptr(), out.data_ptr(), t.numel(), _DTYPES[t.dtype],
                            s.data_ptr(), _stream_handle(t.device))
    _lib.check("lmx_scale", st)
    return out


def ce_fwd_bwd(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100,
               reduction: str = "mean", z_loss_multiplier: float = 0.0,
               grad: Optional[torch.Tensor] = None, want_grad: bool = True,
               in_place: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor],
                                                torch.Tensor, torch.Tensor]:
    """One library call: (loss fp32 scalar, grad or None, n_valid int64, bad_target int32).

    ``in_place=True`` writes the gradient over ``logits``; otherwise a gradient
    buffer is allocated (or ``grad`` is used) when ``want_grad``.
    """
    _require_device(logits, "logits")
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [B, V] tensor")
    if logits.dtype not in _DTYPES:
        raise ValueError(f"unsupported logits dtype {logits.dtype}")
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'sum', not {reduction!r}")
    B, V = logits.shape
    target = target.to(device=logits.device, dtype=torch.int64).contiguous()
    if target.shape != (B,):
        raise ValueError("target must have shape [B]")
    dev = logits.device
    if in_place:
        grad = logits
    elif want_grad and grad is None:
        grad = torch.empty_like(logits)
    elif not want_grad:
        grad = None
    loss = torch.empty((), dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int64, device=dev)
    bad = torch.empty((), dtype=torch.int32, device=dev)
    dtype = _DTYPES[logits.dtype]
    nbytes = _lib.ce_workspace_bytes(B, V, dtype)
    ws = _workspace(nbytes, dev)
    with torch.cuda.device(dev):
        st = _lib.ce_fwd_bwd(logits.data_ptr(), grad.data_ptr() if grad is not None else None,
                             target.data_ptr(), B, V, dtype, int(ignore_index),
                             _REDUCTIONS[reduction], float(z_loss_multiplier), loss.data_ptr(),
                             n_valid.data_ptr(), bad.data_ptr(), ws.data_ptr(), ws.numel(),
                             _stream_handle(dev))
    _lib.check("ce_fwd_bwd", st)
    return loss, grad, n_valid, bad


class _CrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, target, ignore_index, reduction, z):
        loss, grad, _, _ = ce_fwd_bwd(logits.detach(), target, ignore_index, reduction, z,
                                      want_grad=logits.requires_grad)
        ctx.save_for_backward(grad if grad is not None else logits.new_empty(0))
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        (grad,) = ctx.saved_tensors
        return _scaled(grad, grad_out), None, None, None, None


def cross_entropy(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100,
                  reduction: str = "mean", z_loss_multiplier: float = 0.0) -> torch.Tensor:
    """Cross-entropy plus z-loss from materialized logits [B, V]; does not mutate logits."""
    return _CrossEntropy.apply(logits, target, ignore_index, reduction, z_loss_multiplier)


def cross_entropy_(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100,
                   reduction: str = "mean", z_loss_multiplier: float = 0.0) -> torch.Tensor:
    """Raw helper: returns the loss and overwrites ``logits`` with d(loss)/d(logits)."""
    loss, _, _, _ = ce_fwd_bwd(logits, target, ignore_index, reduction, z_loss_multiplier,
                               in_place=True)
    return loss


def linear_ce(inputs: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
              ignore_index: int = -100, reduction: str = "mean",
              z_loss_multiplier: float = 0.0, chunk_size: Optional[int] = None,
              grad_weight_accum_dtype: str = "fp32",
              workspace: Optional[torch.Tensor] = None,
              group_bytes: Optional[int] = None):
    """One library call: (loss, grad_inputs, grad_weight, n_valid, bad_target).

    ``group_bytes`` bounds the workspace bytes of transposed logits gradient
    that one grad_weight product covers (None: the library's default, 2 GiB)."""
    for t, n in ((inputs, "inputs"), (weight, "weight")):
        _require_device(t, n)
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous 2-D tensor")
        if t.dtype not in _LINEAR_DTYPES:
            raise ValueError(f"{n} must be bfloat16 or float16 (the matmuls' input formats)")
    if inputs.dtype != weight.dtype:
        raise ValueError("inputs and weight must have the same dtype")
    BT, D = inputs.shape
    V, D2 = weight.shape
    if D2 != D:
        raise ValueError("inputs [BT, D] and weight [V, D] disagree on D")
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'sum', not {reduction!r}")
    if grad_weight_accum_dtype not in _ACCUMS:
        raise ValueError("grad_weight_accum_dtype must be 'fp32' or 'weight'")
    dev = inputs.device
    target = target.to(device=dev, dtype=torch.int64).contiguous()
    if target.shape != (BT,):
        raise ValueError("target must have shape [BT]")
    cs = 0 if chunk_size is None else int(chunk_size)
    acc = _ACCUMS[grad_weight_accum_dtype]
    ldt = _LINEAR_DTYPES[inputs.dtype]
    gb = 0 if group_bytes is None else int(group_bytes)
    if gb < 0:
        raise ValueError("group_bytes must be >= 0")
    nbytes = _lib.linear_ce_workspace_bytes(BT, D, V, ldt, cs, acc, gb)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int64, device=dev)
    bad = torch.empty((), dtype=torch.int32, device=dev)
    gx = torch.empty_like(inputs)
    gw = torch.empty_like(weight)
    with torch.cuda.device(dev):
        st = _lib.linear_ce(inputs.data_ptr(), weight.data_ptr(), target.data_ptr(), BT, D, V,
                            ldt, int(ignore_index), _REDUCTIONS[reduction],
                            float(z_loss_multiplier), cs, acc, gb, loss.data_ptr(), gx.data_ptr(),
                            gw.data_ptr(), n_valid.data_ptr(), bad.data_ptr(),
                            workspace.data_ptr(), workspace.numel(), _stream_handle(dev))
    _lib.check("linear_ce", st)
    return loss, gx, gw, n_valid, bad


class _LinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, inputs, weight, target, ignore_index, reduction, z, chunk_size, accum):
        loss, gx, gw, _, _ = linear_ce(inputs.detach(), weight.detach(), target, ignore_index,
                                       reduction, z, chunk_size, accum)
        ctx.save_for_backward(gx, gw)
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        gx, gw = ctx.saved_tensors
        return _scaled(gx, grad_out), _scaled(gw, grad_out), None, None, None, None, None, None


def linear_cross_entropy(inputs: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                         ignore_index: int = -100, reduction: str = "mean",
                         z_loss_multiplier: float = 0.0, chunk_size: Optional[int] = None,
                         grad_weight_accum_dtype: str = "fp32") -> torch.Tensor:
    """Chunked linear cross-entropy with z-loss; gradients flow to inputs and weight."""
    return _LinearCrossEntropy.apply(inputs, weight, target, ignore_index, reduction,
                                     z_loss_multiplier, chunk_size, grad_weight_accum_dtype)


def chunked_linear_cross_entropy(inputs: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                                 ignore_index: int = -100, reduction: str = "mean",
                                 z_loss_multiplier: float = 0.0,
                                 grad_weight_accum_dtype: str = "fp32", *,
                                 chunk_size: Optional[int] = None) -> torch.Tensor:
    """The page's ``chunked_linear_cross_entropy``, argument for argument (the
    row-chunk size, which that entry leaves to the library, may be given by
    keyword); the same computation as ``linear_cross_entropy``."""
    return _LinearCrossEntropy.apply(inputs, weight, target, ignore_index, reduction,
                                     z_loss_multiplier, chunk_size, grad_weight_accum_dtype)


def _rows_args(logits: torch.Tensor, index: torch.Tensor, what: str):
    _require_device(logits, "logits")
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [B, V] tensor")
    if logits.dtype not in _DTYPES:
        raise ValueError(f"unsupported logits dtype {logits.dtype}")
    B, V = logits.shape
    index = index.to(device=logits.device, dtype=torch.int64).contiguous()
    if index.shape != (B,):
        raise ValueError(f"{what} must have shape [B]")
    return B, V, index


def selective_log_softmax(logits: torch.Tensor, index: torch.Tensor) -> torch.Tensor:
    """``log_softmax(logits, -1).gather(-1, index[..., None])[..., 0]`` in fp32; no autograd.

    ``logits`` is ``[..., V]`` (contiguous) and ``index`` has its leading shape
    ``[...]``; the result has that shape too."""
    if logits.dim() != 2:
        if logits.dim() < 1 or not logits.is_contiguous():
            raise ValueError("logits must be a contiguous [..., V] tensor")
        lead = logits.shape[:-1]
        if tuple(index.shape) != tuple(lead):
            raise ValueError("index must have the leading shape of logits")
        return selective_log_softmax(logits.reshape(-1, logits.shape[-1]),
                                     index.reshape(-1)).reshape(lead)
    B, V, index = _rows_args(logits, index, "index")
    dev = logits.device
    out = torch.empty(B, dtype=torch.float32, device=dev)
    bad = torch.empty((), dtype=torch.int32, device=dev)
    dtype = _DTYPES[logits.dtype]
    ws = _workspace(_lib.ce_workspace_bytes(B, V, dtype), dev)
    with torch.cuda.device(dev):
        st = _lib.selective_log_softmax(logits.data_ptr(), index.data_ptr(), B, V, dtype,
                                        out.data_ptr(), bad.data_ptr(), ws.data_ptr(),
                                        ws.numel(), _stream_handle(dev))
    _lib.check("selective_log_softmax", st)
    return out


def ce_loss_rows(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100):
    """One library call: (per-row losses fp32 [B], n_valid, bad_target)."""
    B, V, target = _rows_args(logits, target, "target")
    dev = logits.device
    out = torch.empty(B, dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int64, device=dev)
    bad = torch.empty((), dtype=torch.int32, device=dev)
    dtype = _DTYPES[logits.dtype]
    ws = _workspace(_lib.ce_workspace_bytes(B, V, dtype), dev)
    with torch.cuda.device(dev):
        st = _lib.ce_loss_rows(logits.data_ptr(), target.data_ptr(), B, V, dtype,
                               int(ignore_index), out.data_ptr(), n_valid.data_ptr(),
                               bad.data_ptr(), ws.data_ptr(), ws.numel(), _stream_handle(dev))
    _lib.check("ce_loss_rows", st)
    return out, n_valid, bad


def ce_loss_rows_vjp(logits: torch.Tensor, target: torch.Tensor, loss_rows: torch.Tensor,
                     g: torch.Tensor, ignore_index: int = -100,
                     in_place: bool = False) -> torch.Tensor:
    """One library call: d(sum_i g_i loss_i)/d(logits), in the logits dtype."""
    B, V, target = _rows_args(logits, target, "target")
    dev = logits.device
    loss_rows = loss_rows.to(device=dev, dtype=torch.float32).contiguous()
    g = g.to(device=dev, dtype=torch.float32).contiguous()
    if loss_rows.shape != (B,) or g.shape != (B,):
        raise ValueError("loss_rows and g must have shape [B]")
    grad = logits if in_place else torch.empty_like(logits)
    with torch.cuda.device(dev):
        st = _lib.ce_loss_rows_vjp(logits.data_ptr(), target.data_ptr(), loss_rows.data_ptr(),
                                   g.data_ptr(), grad.data_ptr(), B, V, _DTYPES[logits.dtype],
                                   int(ignore_index), _stream_handle(dev))
    _lib.check("ce_loss_rows_vjp", st)
    return grad


class _CrossEntropyPerRow(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, target, ignore_index):
        loss, _, _ = ce_loss_rows(logits.detach(), target, ignore_index)
        ctx.ignore_index = ignore_index
        ctx.save_for_backward(logits.detach(), target, loss)
        return loss

    @staticmethod
    def backward(ctx, g):
        logits, target, loss = ctx.saved_tensors
        return ce_loss_rows_vjp(logits, target, loss, g, ctx.ignore_index), None, None


def cross_entropy_per_row(logits: torch.Tensor, target: torch.Tensor,
                          ignore_index: int = -100) -> torch.Tensor:
    """Unreduced cross-entropy ``logsumexp(x_i) - x_i[t_i]`` per row (fp32 [B], 0 where
    ignored); its backward is one ``ce_loss_rows_vjp`` pass over the logits."""
    return _CrossEntropyPerRow.apply(logits, target, ignore_index)


def autograd_loss_and_logits_grad(loss_fn):
    """Adapts a scalar loss ``loss_fn(logits_chunk, *args, **kwargs)`` to return
    ``(loss, grad_logits)`` by running autograd on the logits chunk (page entry
    ``autograd_loss_and_logits_grad``)."""
    def loss_and_grad(logits_chunk, *args, **kwargs):
        x = logits_chunk.detach().requires_grad_(True)
        with torch.enable_grad():
            loss = loss_fn(x, *args, **kwargs)
            (g,) = torch.autograd.grad(loss, x)
        return loss.detach(), g
    return loss_and_grad


def cross_entropy_loss_and_grad(logits_chunk: torch.Tensor, target: torch.Tensor,
                                ignore_index: int = -100, z_loss_multiplier: float = 0.0):
    """The library's cross-entropy (sum over the chunk's valid rows) as a
    loss-and-gradient function for ``chunked_linear_loss``; the gradient is
    written over the logits chunk, which ``chunked_linear_loss`` allows."""
    loss, _, _, _ = ce_fwd_bwd(logits_chunk, target, ignore_index, "sum", z_loss_multiplier,
                               in_place=True)
    return loss, logits_chunk


def _slice_rows(v, BT: int, r0: int, r1: int):
    if isinstance(v, torch.Tensor) and v.dim() > 0 and v.shape[0] == BT:
        return v[r0:r1]
    return v


def chunked_linear_loss_fwd(inputs: torch.Tensor, weight: torch.Tensor, loss_and_grad_fn,
                            loss_args=(), loss_kwargs=None, chunk_size: Optional[int] = None,
                            grad_weight_accum_dtype: str = "fp32", workspace=None):
    """One pass: (sum of the chunk losses, grad_inputs, grad_weight) for an upstream
    gradient of 1. The logits chunk handed to ``loss_and_grad_fn`` is a fresh
    [rows, V] tensor in the inputs' dtype (bf16 or fp16), which the function
    may overwrite with its gradient."""
    loss_kwargs = loss_kwargs or {}
    for t, n in ((inputs, "inputs"), (weight, "weight")):
        _require_device(t, n)
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous 2-D tensor")
        if t.dtype not in _LINEAR_DTYPES:
            raise ValueError(f"{n} must be bfloat16 or float16 (the matmuls' input formats)")
    if inputs.dtype != weight.dtype:
        raise ValueError("inputs and weight must have the same dtype")
    BT, D = inputs.shape
    V, D2 = weight.shape
    if D2 != D:
        raise ValueError("inputs [BT, D] and weight [V, D] disagree on D")
    if V % 8 != 0:
        raise ValueError("the generic chunked loss needs V % 8 == 0 (16-byte gradient rows)")
    if grad_weight_accum_dtype not in _ACCUMS:
        raise ValueError("grad_weight_accum_dtype must be 'fp32' or 'weight'")
    dev = inputs.device
    cs = 0 if chunk_size is None else int(chunk_size)
    acc = _ACCUMS[grad_weight_accum_dtype]
    gx = torch.empty_like(inputs)
    gw = torch.empty_like(weight)
    total = torch.zeros((), dtype=torch.float32, device=dev)
    if BT == 0:
        gw.zero_()
        return total, gx, gw
    ldt = _LINEAR_DTYPES[inputs.dtype]
    C = _lib.linear_ce_chunk_rows(BT, V, cs)
    nbytes = _lib.linear_loss_workspace_bytes(BT, D, V, ldt, cs, acc)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, dev)
    lws = _workspace(_lib.linear_loss_logits_workspace_bytes(C, D, ldt), dev)
    stream = _stream_handle(dev)
    with torch.cuda.device(dev):
        for ci, r0 in enumerate(range(0, BT, C)):
            r1 = min(BT, r0 + C)
            rows = r1 - r0
            logits = torch.empty((rows, V), dtype=inputs.dtype, device=dev)
            _lib.check("linear_loss_logits", _lib.linear_loss_logits(
                inputs[r0:r1].data_ptr(), weight.data_ptr(), rows, D, V, ldt,
                logits.data_ptr(), V, lws.data_ptr(), lws.numel(), stream))
            args = [_slice_rows(a, BT, r0, r1) for a in loss_args]
            kwargs = {k: _slice_rows(v, BT, r0, r1) for k, v in loss_kwargs.items()}
            loss_c, g = loss_and_grad_fn(logits, *args, **kwargs)
            if g.shape != (rows, V):
                raise ValueError("loss_and_grad_fn must return a gradient shaped like the logits")
            g = g.to(inputs.dtype).contiguous()
            total += loss_c.detach().to(torch.float32)
            _lib.check("linear_loss_grads", _lib.linear_loss_grads(
                inputs[r0:r1].data_ptr(), weight.data_ptr(), g.data_ptr(), V, rows, BT, D, V,
                ldt, cs, acc, ci, gx[r0:r1].data_ptr(), gw.data_ptr(),
                workspace.data_ptr(), workspace.numel(), stream))
    return total, gx, gw


class _ChunkedLinearLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, inputs, weight, fn, args, kwargs, chunk_size, accum):
        loss, gx, gw = chunked_linear_loss_fwd(inputs.detach(), weight.detach(), fn, args, kwargs,
                                               chunk_size, accum)
        ctx.save_for_backward(gx, gw)
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        gx, gw = ctx.saved_tensors
        return _scaled(gx, grad_out), _scaled(gw, grad_out), None, None, None, None, None


def chunked_linear_loss(inputs: torch.Tensor, weight: torch.Tensor, loss_and_grad_fn,
                        *loss_args, chunk_size: Optional[int] = None,
                        grad_weight_accum_dtype: str = "fp32", **loss_kwargs) -> torch.Tensor:
    """Sum over row chunks of ``loss_and_grad_fn(inputs_c @ weight.T, *args_c, **kwargs_c)[0]``,
    with gradients for inputs and weight accumulated chunk by chunk (tensor
    arguments whose leading dimension is BT are sliced to the chunk's rows)."""
    return _ChunkedLinearLoss.apply(inputs, weight, loss_and_grad_fn, loss_args, loss_kwargs,
                                    chunk_size, grad_weight_accum_dtype)
