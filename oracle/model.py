"""Whole forward pass of the looped hybrid decoder: prefill and decode.

[P1 section 2] / [P2 section 2]: embed, run the execution schedule (head
layers, the shared block ``loop_passes`` times, tail layers), then the head.
[P1 section 6] (``LoopDecoder.forward``): copy h into the streams on entering
the loop, average the streams on leaving it.  [P1 section 4]: every
execution owns its cache slot.  [P2 section 4] (greedy decoding with the KV
cache): decode appends one token per step; the next token is the argmax of
the last position's logits (lowest index on ties).

Layer body (pre-norm residual), both in plain and in loop executions:
    a = Mixer(RMSNorm(x)),  hmid = x + a,  f = FFN(RMSNorm(hmid))
plain:  h <- hmid + f
loop:   streams <- mHC write of out = a + f   (see ``oracle.mhc``)
Readings: embedding unscaled, untied LM head, a final RMSNorm before the head,
logits in fp32.
"""

from __future__ import annotations

import numpy as np

from .config import Config, schedule, layer_kind
from .attention import KVCache, full_attention
from .gdn import gdn_layer
from .ops import rmsnorm, swiglu_ffn
from . import mhc
from .precision import maybe_bf16


class SeqState:
    """Per-sequence caches: one KV cache per full-attention execution and one
    Gated-DeltaNet state per GDN execution."""

    def __init__(self, cfg: Config, dtype=None):
        """``dtype``: working precision of the caches; None = that of the first
        forward pass that uses them."""
        rows = schedule(cfg)
        self.cfg = cfg
        self.n_full = sum(r.kind == "full" for r in rows)
        self.n_gdn = sum(r.kind == "gdn" for r in rows)
        self.kv = self.S = None
        self.length = 0
        if dtype is not None:
            self.allocate(dtype)

    def allocate(self, dtype):
        cfg = self.cfg
        self.kv = [KVCache(cfg.n_kv_heads, cfg.head_dim, dtype) for _ in range(self.n_full)]
        self.S = [np.zeros((cfg.gdn_heads, cfg.gdn_dv, cfg.gdn_dk), dtype)
                  for _ in range(self.n_gdn)]


def to_dtype(weights: dict, dtype=np.float32) -> dict:
    """bf16 bit patterns (uint16) or float arrays -> arrays of ``dtype``."""
    out = {}
    for k, v in weights.items():
        if v.dtype == np.uint16:
            v = (v.astype(np.uint32) << np.uint32(16)).view(np.float32)
        out[k] = np.asarray(v, dtype=dtype)
    return out


def layer_weights(W: dict, l: int) -> dict:
    """Weights of weight layer ``l`` (keys without the ``L{l}.`` prefix).  A
    ``W`` with a ``layer`` method supplies them itself (weights drawn per layer
    on demand, for stacks too large to hold at once)."""
    if hasattr(W, "layer"):
        return W.layer(l)
    p = f"L{l}."
    return {k[len(p):]: v for k, v in W.items() if k.startswith(p)}


def _layer_body(cfg, row, lw, x, st, pos0, chunked_gdn, bf16):
    xn = maybe_bf16(rmsnorm(x, lw["attn_norm"], cfg.eps), bf16)
    if row.kind == "full":
        a = full_attention(xn, lw, st.kv[row.slot], pos0, cfg, bf16=bf16)
    else:
        a, st.S[row.slot] = gdn_layer(xn, lw, st.S[row.slot], cfg, chunked=chunked_gdn, bf16=bf16)
    hmid = x + a
    hn = maybe_bf16(rmsnorm(hmid, lw["ffn_norm"], cfg.eps), bf16)
    f = swiglu_ffn(hn, lw["w_gateup"], lw["w_down"], bf16=bf16)
    return a, hmid, f


def forward_seq(cfg: Config, W: dict, st: SeqState, ids=None, hidden=None,
                chunked_gdn: bool = False, write_full: bool = False, taps=(),
                bf16: bool = False, taps_all: bool = False):
    """One sequence: T new tokens at positions st.length .. st.length+T-1.
    ``bf16``: the backbone precision policy of ``oracle.precision``.

    Returns (h [T, d] after the last execution, logits [V] of the last position
    or None, {tap exec: hidden [d] at the last position}).  A tap at a loop
    execution reports the mean of the streams after its write.  ``taps_all``:
    the taps hold every position ([T, d]) instead of the last.
    """
    if ids is not None:
        h = W["embed"][np.asarray(ids)]
    else:
        h = np.array(hidden, dtype=W["final_norm"].dtype, copy=True)
    if st.kv is None:
        st.allocate(h.dtype)
    pos0 = st.length
    streams = None
    tapped = {}
    for row in schedule(cfg):
        lw = layer_weights(W, row.layer)
        if not row.loop:
            a, hmid, f = _layer_body(cfg, row, lw, h, st, pos0, chunked_gdn, bf16)
            h = hmid + f
            if row.e in taps:
                tapped[row.e] = h.copy() if taps_all else h[-1].copy()
            continue
        if row.fork:
            streams = mhc.fork(h, cfg.n_streams)
        x, _ = mhc.read(streams, lw["mhc.read_w"], lw["mhc.read_b"])
        a, hmid, f = _layer_body(cfg, row, lw, x, st, pos0, chunked_gdn, bf16)
        out = (hmid + f) if write_full else (a + f)
        P = mhc.sinkhorn(lw["mhc.mix"], cfg.sinkhorn_iters)
        streams = mhc.write(streams, out, lw["mhc.write_w"], lw["mhc.write_b"], P)
        if row.merge:
            h = mhc.merge(streams)
        if row.e in taps:
            tapped[row.e] = mhc.merge(streams) if taps_all else mhc.merge(streams)[-1].copy()
    st.length += h.shape[0]
    logits = None
    if cfg.vocab:
        logits = maybe_bf16(rmsnorm(h[-1:], W["final_norm"], cfg.eps), bf16)[0] @ W["head"].T
    return h, logits, tapped


def prefill(cfg: Config, W: dict, states: list, ids=None, hidden=None, **kw):
    """Batch of sequences with the same number of new tokens.
    ``ids``: [B, T] or ``hidden``: [B, T, d].  Returns (h [B, T, d],
    logits [B, V] or None, taps {e: [B, d]})."""
    B = len(states)
    hs, ls, tps = [], [], []
    for b in range(B):
        h, lg, tp = forward_seq(cfg, W, states[b],
                                ids=None if ids is None else ids[b],
                                hidden=None if hidden is None else hidden[b], **kw)
        hs.append(h)
        ls.append(lg)
        tps.append(tp)
    logits = None if ls[0] is None else np.stack(ls)
    taps = {e: np.stack([tp[e] for tp in tps]) for e in tps[0]}
    return np.stack(hs), logits, taps


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Index of the maximum along the last axis, lowest index on ties."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def decode_step(cfg: Config, W: dict, states: list, tokens, **kw):
    """One new token per sequence at position = its current length.
    Returns (logits [B, V], next tokens [B], h [B, d])."""
    h, logits, _ = prefill(cfg, W, states, ids=np.asarray(tokens).reshape(-1, 1), **kw)
    return logits, argmax_lowest(logits), h[:, 0]


def unrolled(cfg: Config, W: dict):
    """The same model with the loop written out: n_layers = executions, one
    pass, each repeated weight layer (and its mHC parameters) copied."""
    rows = schedule(cfg)
    n = len(rows)
    n_loop = (cfg.loop_end - cfg.loop_start) * cfg.loop_passes
    ucfg = Config.from_dims(cfg.as_dict(), n_layers=n, loop_passes=1,
                            loop_end=cfg.loop_start + n_loop)
    UW = {k: v for k, v in W.items() if not k.startswith("L")}
    for row in rows:
        for k, v in layer_weights(W, row.layer).items():
            UW[f"L{row.e}.{k}"] = v.copy()
    assert all(layer_kind(ucfg, r.e) == r.kind for r in rows)
    return ucfg, UW
