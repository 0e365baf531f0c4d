"""Weight-only int8 encoding of the projection matrices for decode
(test infrastructure, like the rest of this package).

[P1 section 7] estimates the bf16 weights at about 18 GB, about 9 GB in INT8
and 4.5 GB in INT4, and expects the bandwidth saved to offset part of the
56-execution latency; the pages give no format.  The format taken here (the
plainest one): per output row n of a [N][K] matrix, a symmetric scale
s_n = max_k |w_nk| / 127 and codes q_nk = round_half_even(w_nk / s_n) in
[-127, 127] (a zero row has s_n = 0 and q = 0); the decode projections use
w'_nk = s_n * q_nk.  The scale and the division are taken in float32 (the
codes are integers decided by floating point, so both sides decide them in
the same precision).
"""

from __future__ import annotations

import numpy as np

PROJECTIONS = ("w_in", "w_o", "w_gateup", "w_down")


def quantize_rows_int8(w: np.ndarray):
    """(q int8 [N][K], s float32 [N]) of a float matrix (bf16 values)."""
    w32 = np.asarray(w, dtype=np.float32)
    s = (np.max(np.abs(w32), axis=1) / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(w32 / safe[:, None]).astype(np.float32)
    q = np.where(s[:, None] > 0, q, 0.0)
    return np.clip(q, -127, 127).astype(np.int8), s


def dequantize_rows(q: np.ndarray, s: np.ndarray, dtype=np.float32) -> np.ndarray:
    return (q.astype(dtype) * s.astype(dtype)[:, None]).astype(dtype)


def int8_decode_weights(W: dict, n_layers: int, dtype=np.float32) -> dict:
    """The weights the int8 decode path computes with: every layer's four
    projection matrices replaced by their dequantized codes, the rest
    (norm gains, mHC parameters, embedding, head) unchanged."""
    out = dict(W)
    for l in range(n_layers):
        for name in PROJECTIONS:
            key = f"L{l}.{name}"
            q, s = quantize_rows_int8(W[key])
            out[key] = dequantize_rows(q, s, dtype)
    return out
