"""MI355X-native large-vocabulary cross-entropy.

The computation lives in ``liblmx.so`` (hand-written HIP kernels for gfx950,
C ABI in ``include/lmx.h``); this package is its ctypes binding (``_lib``) and
the PyTorch-facing functions (``functional``).
"""
from lm_head_cross_pass_amd.functional import (  # noqa: F401
    autograd_loss_and_logits_grad, ce_fwd_bwd, ce_loss_rows, ce_loss_rows_vjp,
    chunked_linear_cross_entropy, chunked_linear_loss, cross_entropy, cross_entropy_,
    cross_entropy_loss_and_grad,
    cross_entropy_per_row, linear_ce, linear_cross_entropy, selective_log_softmax)
