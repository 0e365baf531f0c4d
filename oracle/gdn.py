"""Gated-DeltaNet (GDN) linear-attention layer.

[P1 section 3]: a linear-attention variant that keeps a constant-size
recurrent state and updates it with a gate plus the delta rule; the state size
does not depend on the sequence length.  The pages fix nothing more; the
reading taken is the standard gated delta rule (Yang, Kautz, Hatamizadeh,
"Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025):

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t

with S in R^{Dv x Dk}, S_0 = 0 for a fresh sequence, 16 heads of 128 key and
value dims at full size.  Readings for the block around it: one fused input
projection ``[W_q; W_k; W_v; W_z; W_a; W_b]`` of the normed input (no short
convolution, no activation on q/k/v); alpha_t = exp(-softplus(a_t)) and
beta_t = sigmoid(b_t) per head; q and k L2-normalised per head (eps 1e-6) and
q scaled by 1/sqrt(Dk); output = RMSNorm over Dv of o (one gain shared by the
heads) times SiLU(z), then ``W_o``.

``gdn_recurrent`` is the definition; ``gdn_chunked`` is the chunkwise form of
the same recurrence (a second routine that the tests hold equal to the first).
"""

from __future__ import annotations

import numpy as np

from .ops import rmsnorm, silu, sigmoid, softplus
from .precision import maybe_bf16


def gdn_recurrent(q, k, v, alpha, beta, S0):
    """Token-by-token recurrence.

    q, k: [T, H, Dk]; v: [T, H, Dv]; alpha, beta: [T, H]; S0: [H, Dv, Dk].
    Returns o [T, H, Dv] and the final state [H, Dv, Dk].  The product
    S (I - beta k k^T) is evaluated as S - beta (S k) k^T (associativity).
    """
    T, H, Dk = k.shape
    S = S0.copy()
    o = np.empty(v.shape, dtype=v.dtype)
    for t in range(T):
        a = alpha[t][:, None, None]
        b = beta[t][:, None, None]
        kt, vt = k[t], v[t]
        Sk = np.einsum("hvk,hk->hv", S, kt)
        S = a * (S - b * Sk[:, :, None] * kt[:, None, :]) + b * vt[:, :, None] * kt[:, None, :]
        o[t] = np.einsum("hvk,hk->hv", S, q[t])
    return o, S


def gdn_chunked(q, k, v, log_alpha, beta, S0, chunk: int = 64):
    """Chunkwise form of the same recurrence, one chunk of C tokens at a time.

    With G_r = sum_{j<=r} log alpha_j inside the chunk, gamma = exp(G) and
    A[r, i] = beta_r exp(G_r - G_i) (k_r . k_i) for i < r:
        T = (I + A)^-1,  W = T diag(beta*gamma) K,  U~ = T diag(beta) V,
        U = U~ - W S0^T,
        O = diag(gamma) Q S0^T + (tril(exp(G_r - G_i)) * Q K^T) U,
        S_C = gamma_C S0 + U^T diag(exp(G_C - G)) K.
    Arguments as in :func:`gdn_recurrent`, with ``log_alpha`` in place of alpha.
    """
    T, H, Dk = k.shape
    Dv = v.shape[2]
    S = S0.copy()
    o = np.empty((T, H, Dv), dtype=v.dtype)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        C = c1 - c0
        for h in range(H):
            Q, K, V = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h]
            b = beta[c0:c1, h]
            G = np.cumsum(log_alpha[c0:c1, h])
            gam = np.exp(G)
            dG = G[:, None] - G[None, :]
            low = np.tril(np.ones((C, C), dtype=bool), -1)
            A = np.where(low, b[:, None] * np.exp(np.where(low, dG, 0)) * (K @ K.T), 0).astype(K.dtype)
            Tm = np.linalg.inv(np.eye(C, dtype=K.dtype) + A)
            W = Tm @ ((b * gam)[:, None] * K)
            Ut = Tm @ (b[:, None] * V)
            S0h = S[h]
            U = Ut - W @ S0h.T
            incl = np.tril(np.ones((C, C), dtype=bool))
            Mqk = np.where(incl, np.exp(np.where(incl, dG, 0)) * (Q @ K.T), 0).astype(K.dtype)
            o[c0:c1, h] = gam[:, None] * (Q @ S0h.T) + Mqk @ U
            dec = np.exp(G[-1] - G)
            S[h] = gam[-1] * S0h + U.T @ (dec[:, None] * K)
    return o, S


def gdn_mixer(proj: np.ndarray, w: dict, S0: np.ndarray, cfg, chunked: bool = False,
              chunk: int = 64, bf16: bool = False):
    """The mixer between the two projections: from the input projection's
    output ``proj`` [T, 2 H Dk + 2 H Dv + 2 H] (columns q | k | v | z | a | b)
    of one sequence and its entering state ``S0`` [H, Dv, Dk], the gated
    output [T, H*Dv] that enters ``W_o`` and the new state.  ``bf16``: the
    backbone precision policy of ``oracle.precision`` (``proj`` is then
    already bf16-valued; the recurrence and its state stay fp32)."""
    T = proj.shape[0]
    H, Dk, Dv = cfg.gdn_heads, cfg.gdn_dk, cfg.gdn_dv
    o0 = 0
    q = proj[:, o0:o0 + H * Dk].reshape(T, H, Dk); o0 += H * Dk
    k = proj[:, o0:o0 + H * Dk].reshape(T, H, Dk); o0 += H * Dk
    v = proj[:, o0:o0 + H * Dv].reshape(T, H, Dv); o0 += H * Dv
    z = proj[:, o0:o0 + H * Dv].reshape(T, H, Dv); o0 += H * Dv
    a = proj[:, o0:o0 + H]; o0 += H
    b = proj[:, o0:o0 + H]
    eps = q.dtype.type(cfg.eps)
    qh = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps) / np.sqrt(q.dtype.type(Dk))
    kh = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    log_alpha = -softplus(a)
    beta = sigmoid(b)
    if chunked:
        o, S = gdn_chunked(qh, kh, v, log_alpha, beta, S0, chunk)
    else:
        o, S = gdn_recurrent(qh, kh, v, np.exp(log_alpha), beta, S0)
    o = maybe_bf16(rmsnorm(o, w["o_norm"], cfg.eps) * silu(z), bf16)
    return o.reshape(T, H * Dv), S


def gdn_layer(xn: np.ndarray, w: dict, S0: np.ndarray, cfg, chunked: bool = False,
              chunk: int = 64, bf16: bool = False):
    """Mixer output ``a`` [T, d] and the new state for one sequence.  ``bf16``:
    the backbone precision policy of ``oracle.precision`` (projection outputs
    and the gated output in bf16; the recurrence and its state in fp32)."""
    proj = maybe_bf16(xn @ w["w_in"].T, bf16)
    o, S = gdn_mixer(proj, w, S0, cfg, chunked=chunked, chunk=chunk, bf16=bf16)
    return o @ w["w_o"].T, S
