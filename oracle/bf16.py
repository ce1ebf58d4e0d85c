"""Round-to-nearest-even from fp64 to bfloat16, written from the format's definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

bfloat16 keeps the fp32 exponent range (normal numbers down to 2**-126,
subnormals spaced 2**-133) with an 8-bit significand (7 stored bits plus the
implicit one). A finite value ``v = m * 2**e`` with ``m`` in [0.5, 1) is rounded
to the nearest multiple of ``2**(e - 8)`` (of ``2**-133`` in the subnormal
range), ties to the even multiple; a result at or above ``2**128`` becomes
infinity. The value is returned as fp64 (every bfloat16 is exactly an fp64).

Used only by the emulation of the weight-dtype gradient accumulation, which
rounds the running weight gradient between chunks (greyhound functional API
page, ``chunked_linear_cross_entropy``, ``grad_weight_accum_dtype``).
"""
from __future__ import annotations

import numpy as np
import torch

_SUB_QUANTUM = 2.0 ** -133
_OVERFLOW = 2.0 ** 128


def round_to_bf16(v: torch.Tensor) -> torch.Tensor:
    """Nearest bfloat16 value (ties to even) of each element, returned as fp64."""
    a = v.to(torch.float64).numpy()
    out = np.array(a, dtype=np.float64, copy=True)
    finite = np.isfinite(a) & (a != 0.0)
    x = a[finite]
    _, e = np.frexp(x)                                  # x = m * 2**e, 0.5 <= |m| < 1
    q = np.ldexp(np.ones_like(x), e - 8)                # spacing of 8-bit significands
    q = np.maximum(q, _SUB_QUANTUM)                     # subnormal spacing floor
    r = np.rint(x / q) * q                              # rint rounds half to even
    r = np.where(np.abs(r) >= _OVERFLOW, np.copysign(np.inf, r), r)
    out[finite] = r
    return torch.from_numpy(out)
