"""Weight-only int8 and int4 encodings of the projection matrices for decode
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

int4 (the pages give no format for it either; this one is the usual
group-wise symmetric layout): per output row n and group g of 128
consecutive k, s_ng = max |w| over the group / 7 and codes
q = round_half_even(w / s_ng) in [-7, 7] (a zero group has s = 0, q = 0).
The decode projections use the bf16 value nearest to the float32 product
q * s_ng (the product rounded to float32 first).  Storage: codes offset by
8 (so 1 .. 15) in nibbles; each run of 8 consecutive k of a row takes 4
bytes, byte i holding k = i in its low nibble and k = i + 4 in its high
nibble; a row of K codes takes K / 2 bytes.  Scales float32 [N][K / 128].
"""

from __future__ import annotations

import numpy as np

from .precision import round_bf16

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


INT4_GROUP = 128


def quantize_groups_int4(w: np.ndarray, group: int = INT4_GROUP):
    """(q int8 [N][K] in [-7, 7], s float32 [N][K / group]) of a float
    matrix (bf16 values); K a multiple of ``group``."""
    w32 = np.asarray(w, dtype=np.float32)
    N, K = w32.shape
    assert K % group == 0
    wg = w32.reshape(N, K // group, group)
    s = (np.max(np.abs(wg), axis=2) / np.float32(7.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(wg / safe[:, :, None]).astype(np.float32)
    q = np.where(s[:, :, None] > 0, q, 0.0)
    return np.clip(q, -7, 7).astype(np.int8).reshape(N, K), s


def dequantize_groups_int4(q: np.ndarray, s: np.ndarray, group: int = INT4_GROUP) -> np.ndarray:
    """bf16 value (as float32) of the float32 product code * group scale."""
    N, K = q.shape
    prod = (q.reshape(N, K // group, group).astype(np.float32) * s.astype(np.float32)[:, :, None]).astype(np.float32)
    return round_bf16(prod.reshape(N, K))


def pack_int4(q: np.ndarray) -> np.ndarray:
    """uint8 [N][K / 2]: per 8 consecutive k, byte i = (q[i] + 8) | (q[i + 4] + 8) << 4."""
    N, K = q.shape
    assert K % 8 == 0
    n = (q.astype(np.int16) + 8).astype(np.uint8).reshape(N, K // 8, 2, 4)
    return (n[:, :, 0, :] | (n[:, :, 1, :] << 4)).astype(np.uint8).reshape(N, K // 2)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    N, H = p.shape
    b = p.reshape(N, H // 4, 4)
    lo = (b & 0x0F).astype(np.int16) - 8
    hi = (b >> 4).astype(np.int16) - 8
    return np.concatenate([lo, hi], axis=2).astype(np.int8).reshape(N, 2 * H)


def int4_decode_weights(W: dict, n_layers: int, dtype=np.float32) -> dict:
    """The weights the int4 decode path computes with: every layer's four
    projection matrices replaced by their dequantized group codes, the rest
    unchanged."""
    out = dict(W)
    for l in range(n_layers):
        for name in PROJECTIONS:
            key = f"L{l}.{name}"
            q, s = quantize_groups_int4(W[key])
            out[key] = dequantize_groups_int4(q, s).astype(dtype)
    return out
