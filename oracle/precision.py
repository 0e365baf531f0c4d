"""Precision policy of the backbone.

[P2 section 3] gives the backbone precision as BF16 and the mHC routing
parameters as FP32; [P1 section 5] says the backbone is stored in BF16 while
the mHC routing and the computation of the mixing matrix stay in FP32 so that
they take no half-precision rounding.

Reading taken for the oracle's ``bf16=True`` mode: every tensor that the
backbone hands from one operation to the next is stored in bf16 -- the
normed inputs of the projections (pre-norm outputs), the projection outputs,
q and k after QK-norm and rotary, the attention probabilities that multiply
V, the gated mixer output that enters W_o, the SwiGLU activation that enters
W_down, and the final normed hidden state that enters the head -- while the
residual stream, the mHC streams and routing, softmax statistics,
normalisation statistics, the Gated-DeltaNet state and recurrence, and every
accumulation stay fp32.  Rounding is to nearest even.

With ``bf16=False`` (the default) the oracle is the plain fp32 (or fp64)
definition with no intermediate rounding.
"""

from __future__ import annotations

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); returns float32."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    u = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def maybe_bf16(x: np.ndarray, on: bool) -> np.ndarray:
    return round_bf16(x) if on else x
