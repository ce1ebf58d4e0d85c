"""ctypes binding of liblmx.so: the C ABI of ``include/lmx.h``, one Python
function per C entry point with the same name and argument order.

Arguments are plain integers (device addresses, sizes, enum values) and the
HIP stream handle; this module only marshals them. Loading fails loudly when
the library has not been built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblmx.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "lmx.h")

# enums of lmx.h
LMX_F32, LMX_BF16, LMX_F16 = 0, 1, 2
LMX_MEAN, LMX_SUM = 0, 1
LMX_ACC_F32, LMX_ACC_WEIGHT = 0, 1

STATUS = {
    0: "LMX_OK", -1: "LMX_ERR_NULL", -2: "LMX_ERR_SIZE", -3: "LMX_ERR_ENUM",
    -4: "LMX_ERR_WORKSPACE", -5: "LMX_ERR_ALIAS", -6: "LMX_ERR_ALIGN",
    -7: "LMX_ERR_CHUNK", -8: "LMX_ERR_UNSUPPORTED", -9: "LMX_ERR_HIP",
    -10: "LMX_ERR_SCRATCH",
}
for _code, _name in STATUS.items():
    globals()[_name] = _code

_vp, _i64, _i32, _sz, _f32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                              ctypes.c_size_t, ctypes.c_float)

_SIGNATURES = {
    "ce_fwd_bwd": (_i32, [_vp, _vp, _vp, _i64, _i64, _i32, _i64, _i32, _f32,
                          _vp, _vp, _vp, _vp, _sz, _vp]),
    "ce_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "ce_fwd_bwd_noalloc": (_i32, [_vp, _vp, _vp, _i64, _i64, _i32, _i64, _i32, _f32,
                                  _vp, _vp, _vp, _vp]),
    "linear_ce": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _i32, _f32,
                         _i64, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "linear_ce_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i64, _i32, _i64]),
    "linear_ce_chunk_rows": (_i64, [_i64, _i64, _i64]),
    "lmx_status_string": (ctypes.c_char_p, [_i32]),
    "lmx_copy": (_i32, [_vp, _vp, _sz, _vp]),
    "lmx_stream_probe": (_i32, [_vp, _vp, _sz, _sz, _i32, _vp]),
    "lmx_scale": (_i32, [_vp, _vp, _i64, _i32, _vp, _vp]),
    "selective_log_softmax": (_i32, [_vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp, _sz, _vp]),
    "ce_loss_rows": (_i32, [_vp, _vp, _i64, _i64, _i32, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ce_loss_rows_vjp": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i64, _vp]),
    "linear_loss_logits": (_i32, [_vp, _vp, _i64, _i64, _i64, _i32, _vp, _i64, _vp, _sz, _vp]),
    "linear_loss_logits_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "linear_loss_grads": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i32, _i64, _i32,
                                 _i64, _vp, _vp, _vp, _sz, _vp]),
    "linear_loss_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i64, _i32]),
}

_lib = None


class LmxError(RuntimeError):
    """A liblmx.so entry point returned a negative status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_string(status)})")


def load() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m lm_head_cross_pass_amd.build` "
                "(or __graft_entry__.build()). There is no CPU fallback.")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions declared in lmx.h (for export checks)."""
    text = open(path).read()
    return re.findall(r"LMX_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def status_string(status: int) -> str:
    return load().lmx_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != 0:
        raise LmxError(fn, status)


def ce_fwd_bwd(logits, grad_logits, target, B, V, dtype, ignore_index, reduction,
               z_loss_multiplier, loss, n_valid, bad_target, workspace, workspace_bytes,
               stream) -> int:
    return load().ce_fwd_bwd(logits, grad_logits, target, B, V, dtype, ignore_index,
                             reduction, z_loss_multiplier, loss, n_valid, bad_target,
                             workspace, workspace_bytes, stream)


def ce_fwd_bwd_noalloc(logits, grad_logits, target, B, V, dtype, ignore_index, reduction,
                       z_loss_multiplier, loss, n_valid, bad_target, stream) -> int:
    return load().ce_fwd_bwd_noalloc(logits, grad_logits, target, B, V, dtype, ignore_index,
                                     reduction, z_loss_multiplier, loss, n_valid, bad_target,
                                     stream)


def ce_workspace_bytes(B, V, dtype) -> int:
    return load().ce_workspace_bytes(B, V, dtype)


def linear_ce(inputs, weight, target, BT, D, V, dtype, ignore_index, reduction,
              z_loss_multiplier, chunk_size, accum, group_bytes, loss, grad_inputs, grad_weight,
              n_valid, bad_target, workspace, workspace_bytes, stream) -> int:
    return load().linear_ce(inputs, weight, target, BT, D, V, dtype, ignore_index, reduction,
                            z_loss_multiplier, chunk_size, accum, group_bytes, loss, grad_inputs,
                            grad_weight, n_valid, bad_target, workspace, workspace_bytes,
                            stream)


def linear_ce_workspace_bytes(BT, D, V, dtype, chunk_size, accum, group_bytes) -> int:
    return load().linear_ce_workspace_bytes(BT, D, V, dtype, chunk_size, accum, group_bytes)


def linear_ce_chunk_rows(BT, V, chunk_size) -> int:
    return load().linear_ce_chunk_rows(BT, V, chunk_size)


def lmx_copy(src, dst, nbytes, stream) -> int:
    return load().lmx_copy(src, dst, nbytes, stream)


# lmx_stream_probe modes
(LMX_PROBE_READ, LMX_PROBE_WRITE, LMX_PROBE_COPY, LMX_PROBE_COPY_BATCHED,
 LMX_PROBE_ROWS_INTERLEAVED, LMX_PROBE_ROWS_PHASED) = range(6)


def lmx_stream_probe(src, dst, nbytes, row_bytes, mode, stream) -> int:
    return load().lmx_stream_probe(src, dst, nbytes, row_bytes, mode, stream)


def lmx_scale(src, dst, n, dtype, scale, stream) -> int:
    return load().lmx_scale(src, dst, n, dtype, scale, stream)


def selective_log_softmax(logits, index, B, V, dtype, out, bad_index, workspace,
                          workspace_bytes, stream) -> int:
    return load().selective_log_softmax(logits, index, B, V, dtype, out, bad_index, workspace,
                                        workspace_bytes, stream)


def ce_loss_rows(logits, target, B, V, dtype, ignore_index, loss_rows, n_valid, bad_target,
                 workspace, workspace_bytes, stream) -> int:
    return load().ce_loss_rows(logits, target, B, V, dtype, ignore_index, loss_rows, n_valid,
                               bad_target, workspace, workspace_bytes, stream)


def ce_loss_rows_vjp(logits, target, loss_rows, g, grad_logits, B, V, dtype, ignore_index,
                     stream) -> int:
    return load().ce_loss_rows_vjp(logits, target, loss_rows, g, grad_logits, B, V, dtype,
                                   ignore_index, stream)


def linear_loss_logits(inputs_c, weight, rows, D, V, dtype, logits, ld_logits, workspace,
                       workspace_bytes, stream) -> int:
    return load().linear_loss_logits(inputs_c, weight, rows, D, V, dtype, logits, ld_logits,
                                     workspace, workspace_bytes, stream)


def linear_loss_logits_workspace_bytes(rows, D, dtype) -> int:
    return load().linear_loss_logits_workspace_bytes(rows, D, dtype)


def linear_loss_grads(inputs_c, weight, grad_logits, ld_grad, rows, BT, D, V, dtype, chunk_size,
                      accum, chunk_index, grad_inputs_c, grad_weight, workspace, workspace_bytes,
                      stream) -> int:
    return load().linear_loss_grads(inputs_c, weight, grad_logits, ld_grad, rows, BT, D, V, dtype,
                                    chunk_size, accum, chunk_index, grad_inputs_c, grad_weight,
                                    workspace, workspace_bytes, stream)


def linear_loss_workspace_bytes(BT, D, V, dtype, chunk_size, accum) -> int:
    return load().linear_loss_workspace_bytes(BT, D, V, dtype, chunk_size, accum)
