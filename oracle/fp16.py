"""Round-to-nearest-even from fp64 to IEEE binary16 (half), written from the format.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

binary16 has an 11-bit significand (10 stored bits plus the implicit one),
normal numbers down to 2**-14 and subnormals spaced 2**-24; the largest finite
value is 65504. A finite value ``v = m * 2**e`` with ``m`` in [0.5, 1) is rounded
to the nearest multiple of ``2**(e - 11)`` (of ``2**-24`` in the subnormal range),
ties to the even multiple; a result of 2**16 or more becomes infinity (so values
from 65520 up overflow, as the format prescribes). Returned as fp64.

Used only by the emulation of the weight-dtype gradient accumulation for fp16
weights (greyhound functional API page, ``chunked_linear_cross_entropy``: the
matmuls run in bf16 or fp16 and ``grad_weight_accum_dtype='weight'`` rounds
between chunks).
"""
from __future__ import annotations

import numpy as np
import torch

_SUB_QUANTUM = 2.0 ** -24
_OVERFLOW = 2.0 ** 16


def round_to_fp16(v: torch.Tensor) -> torch.Tensor:
    """Nearest binary16 value (ties to even) of each element, returned as fp64."""
    a = v.to(torch.float64).numpy()
    out = np.array(a, dtype=np.float64, copy=True)
    finite = np.isfinite(a) & (a != 0.0)
    x = a[finite]
    _, e = np.frexp(x)                                  # x = m * 2**e, 0.5 <= |m| < 1
    q = np.ldexp(np.ones_like(x), e - 11)               # spacing of 11-bit significands
    q = np.maximum(q, _SUB_QUANTUM)                     # subnormal spacing floor
    r = np.rint(x / q) * q                              # rint rounds half to even
    r = np.where(np.abs(r) >= _OVERFLOW, np.copysign(np.inf, r), r)
    out[finite] = r
    return torch.from_numpy(out)
