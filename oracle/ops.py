"""Row operations: RMSNorm, activations, softmax, rotary embedding, SwiGLU FFN.

Readings (the pages name these components but do not define them):
* RMSNorm ``y = x / sqrt(mean(x^2) + eps) * g`` with a learned gain, eps 1e-6,
  pre-norm before the mixer and before the FFN, and a final norm before the
  head.  [P4 section 01] gives the backbone type of the configuration as a
  Qwen3.5-style text decoder, whose norms are RMSNorms.
* SwiGLU FFN with three matrices and no biases, [P1 section 2].
* Rotary embedding on the first ``rotary_dim`` dims only (factor 0.25 of 256:
  64 dims), [P1 section 3]; "interleaved" read as adjacent pairs (2i, 2i+1);
  base 10000; text-only positions so the multi-axis variant collapses to one
  axis.  Angles in float64, cos/sin rounded to the working precision.
"""

from __future__ import annotations

import numpy as np


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * g


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def silu(x: np.ndarray) -> np.ndarray:
    return x * sigmoid(x)


def softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(x.dtype.type(0), x)


def logsumexp(x: np.ndarray, axis: int) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    return m + np.log(np.sum(np.exp(x - m), axis=axis, keepdims=True))


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def rope_cos_sin(positions: np.ndarray, rotary_dim: int, theta: float, dtype):
    """cos, sin of shape [T, rotary_dim/2]: angle pos * theta^(-2i/rotary_dim)."""
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / rotary_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def apply_rope(x: np.ndarray, positions: np.ndarray, rotary_dim: int, theta: float) -> np.ndarray:
    """Rotate the adjacent pairs (2i, 2i+1), i < rotary_dim/2, of the last axis.
    ``x``: [T, heads, D]; dims >= rotary_dim pass through."""
    if rotary_dim == 0:
        return x.copy()
    c, s = rope_cos_sin(positions, rotary_dim, theta, x.dtype)
    c, s = c[:, None, :], s[:, None, :]
    out = x.copy()
    x0 = x[..., 0:rotary_dim:2]
    x1 = x[..., 1:rotary_dim:2]
    out[..., 0:rotary_dim:2] = x0 * c - x1 * s
    out[..., 1:rotary_dim:2] = x0 * s + x1 * c
    return out


def swiglu_ffn(hn: np.ndarray, w_gateup: np.ndarray, w_down: np.ndarray,
               bf16: bool = False) -> np.ndarray:
    """``(silu(hn W_gate^T) * (hn W_up^T)) W_down^T``; ``w_gateup`` = [gate; up].
    ``bf16``: the activation entering W_down is stored in bf16."""
    from .precision import maybe_bf16
    F = w_down.shape[1]
    gu = hn @ w_gateup.T
    return maybe_bf16(silu(gu[:, :F]) * gu[:, F:], bf16) @ w_down.T
