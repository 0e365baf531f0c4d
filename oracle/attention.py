"""Full-attention layer: GQA with QK-norm, partial rotary and an output gate.

[P1 section 3], [P2 section 3]: 16 query heads share 4 KV heads (GQA), head
dim 256, QK normalisation, an attention output gate, rotary on a quarter of
the dims.  [P1 section 4]: the cache holds K and V of every KV head in bf16.

Readings: one fused input projection ``[W_q; W_g; W_k; W_v]`` of the normed
input, no biases; QK-norm = RMSNorm over the head dim with one gain vector for
q and one for k shared across heads, applied before rotary; the cache stores
post-norm, post-rotary K and raw V; scale 1/sqrt(D); query head j reads KV head
``j // (Hq / Hkv)``; causal on absolute positions; the gate is an elementwise
sigmoid of ``xn W_g^T`` over all Hq*D outputs, applied before ``W_o``.
"""

from __future__ import annotations

import numpy as np

from .ops import rmsnorm, apply_rope, softmax, sigmoid
from .precision import maybe_bf16, round_bf16


class KVCache:
    """K, V of one sequence for one full-attention execution: [Hkv, L, D]."""

    def __init__(self, n_kv_heads: int, head_dim: int, dtype):
        self.k = np.zeros((n_kv_heads, 0, head_dim), dtype)
        self.v = np.zeros((n_kv_heads, 0, head_dim), dtype)

    @property
    def length(self) -> int:
        return self.k.shape[1]

    def append(self, k: np.ndarray, v: np.ndarray) -> None:
        """``k``, ``v``: [T, Hkv, D]."""
        self.k = np.concatenate([self.k, k.transpose(1, 0, 2)], axis=1)
        self.v = np.concatenate([self.v, v.transpose(1, 0, 2)], axis=1)


def attention_core(q: np.ndarray, K: np.ndarray, V: np.ndarray, q_pos: np.ndarray,
                   bf16: bool = False) -> np.ndarray:
    """softmax(q K^T / sqrt(D), keys at positions <= q_pos) V per query head.
    ``q``: [T, Hq, D]; ``K``, ``V``: [Hkv, L, D] for key positions 0..L-1.
    ``bf16``: the (unnormalised) probabilities exp(s - max) that multiply V
    are stored in bf16; the normaliser is summed in full precision."""
    T, Hq, D = q.shape
    Hkv, L, _ = K.shape
    group = Hq // Hkv
    scale = q.dtype.type(1.0 / np.sqrt(D))
    keypos = np.arange(L)
    mask = keypos[None, :] <= np.asarray(q_pos)[:, None]          # [T, L]
    out = np.empty_like(q)
    for j in range(Hq):
        kv = j // group
        s = (q[:, j, :] @ K[kv].T) * scale                        # [T, L]
        s = np.where(mask, s, -np.inf)
        if not bf16:
            out[:, j, :] = softmax(s, axis=-1) @ V[kv]
        else:
            e = np.exp(s - np.max(s, axis=-1, keepdims=True))
            out[:, j, :] = (round_bf16(e) @ V[kv]) / np.sum(e, axis=-1, keepdims=True)
    return out


def attention_mixer(proj: np.ndarray, w: dict, cache: KVCache, pos0: int, cfg,
                    bf16: bool = False) -> np.ndarray:
    """The mixer between the two projections: from the input projection's
    output ``proj`` [T, 2 Hq D + 2 Hkv D] (columns q | g | k | v) of one
    sequence whose new tokens sit at positions pos0 .. pos0+T-1, the gated
    attention output [T, Hq*D] that enters ``W_o``; appends the new K, V to
    ``cache``.  ``bf16``: the backbone precision policy of
    ``oracle.precision`` (``proj`` is then already bf16-valued)."""
    T = proj.shape[0]
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = proj[:, :Hq * D].reshape(T, Hq, D)
    g = proj[:, Hq * D:2 * Hq * D]
    k = proj[:, 2 * Hq * D:2 * Hq * D + Hkv * D].reshape(T, Hkv, D)
    v = proj[:, 2 * Hq * D + Hkv * D:].reshape(T, Hkv, D)
    q = rmsnorm(q, w["q_norm"], cfg.eps)
    k = rmsnorm(k, w["k_norm"], cfg.eps)
    pos = np.arange(pos0, pos0 + T)
    q = apply_rope(q, pos, cfg.rotary_dim, cfg.rope_theta)
    k = apply_rope(k, pos, cfg.rotary_dim, cfg.rope_theta)
    q, k = maybe_bf16(q, bf16), maybe_bf16(k, bf16)
    assert cache.length == pos0, "cache length must equal the first new position"
    cache.append(k, v)
    o = attention_core(q, cache.k, cache.v, pos, bf16=bf16)
    return maybe_bf16(o.reshape(T, Hq * D) * sigmoid(g), bf16)


def full_attention(xn: np.ndarray, w: dict, cache: KVCache, pos0: int, cfg,
                   bf16: bool = False) -> np.ndarray:
    """Mixer output ``a`` [T, d] for one sequence whose new tokens sit at
    positions pos0 .. pos0+T-1; appends their K, V to ``cache``.  ``bf16``:
    the backbone precision policy of ``oracle.precision``."""
    proj = maybe_bf16(xn @ w["w_in"].T, bf16)
    return attention_mixer(proj, w, cache, pos0, cfg, bf16=bf16) @ w["w_o"].T
