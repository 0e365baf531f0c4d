"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no arithmetic of the model: only the counter-based random
number generator, the draw recipes (normal, uniform token ids) and the
dimension presets of the workloads.  Both the CPU oracle and the HIP path get
their weights, token ids, hidden inputs and pre-filled caches from here (or,
for the sizes that do not fit a host round trip, from the device generator in
the HIP library, which implements the same generator from the same published
definition, so the two sides draw identical values).

Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11).  One tensor is one stream: key
``(seed, fnv1a32(name))``; block ``j`` uses the counter ``(j mod 2^32,
j >> 32, 0, 0)`` and yields four 32-bit words, element ``4*j + m`` takes word
``m``.  Normal draws use the Box-Muller transform in float64 on the word pairs
(0, 1) and (2, 3) with ``u = (x + 0.5) * 2^-32``; the product with the
standard deviation is rounded to float32 (round to nearest even), then, for
bf16 tensors, to bf16 (round to nearest even).  Token ids are
``(x * vocab) >> 32``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .presets import PRESETS, preset  # noqa: F401

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)

SEED_W = 0  # weights
SEED_X = 1  # token ids / hidden inputs
SEED_C = 2  # pre-filled caches and states


def fnv1a32(name: str) -> int:
    """32-bit FNV-1a hash of the UTF-8 bytes of ``name`` (tensor stream id)."""
    h = 0x811C9DC5
    for b in name.encode("utf-8"):
        h ^= b
        h = (h * 0x01000193) & 0xFFFFFFFF
    return h


def philox4x32_10(ctr: np.ndarray, key: tuple[int, int]) -> np.ndarray:
    """Philox4x32 with 10 rounds.  ``ctr``: uint32 [n, 4]; returns uint32 [n, 4]."""
    c0 = ctr[:, 0].astype(np.uint64)
    c1 = ctr[:, 1].astype(np.uint64)
    c2 = ctr[:, 2].astype(np.uint64)
    c3 = ctr[:, 3].astype(np.uint64)
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = _M0 * c0
        p1 = _M1 * c2
        n0 = (p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0)
        n2 = (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1)
        c0, c1, c2, c3 = n0, p1 & _MASK, n2, p0 & _MASK
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def stream_u32(seed: int, name: str, n: int, start: int = 0) -> np.ndarray:
    """Words ``start .. start+n-1`` of the stream ``(seed, name)`` as uint32."""
    if n <= 0:
        return np.zeros(0, np.uint32)
    j0 = start // 4
    j1 = (start + n + 3) // 4
    j = np.arange(j0, j1, dtype=np.uint64)
    ctr = np.zeros((j.size, 4), np.uint32)
    ctr[:, 0] = (j & _MASK).astype(np.uint32)
    ctr[:, 1] = (j >> np.uint64(32)).astype(np.uint32)
    words = philox4x32_10(ctr, (seed, fnv1a32(name))).reshape(-1)
    off = start - 4 * j0
    return words[off:off + n]


def _box_muller(words: np.ndarray) -> np.ndarray:
    """float64 normals from a uint32 word array whose length is a multiple of 4
    and whose first word has index 0 mod 4 in its stream."""
    w = words.reshape(-1, 2).astype(np.float64)
    u1 = (w[:, 0] + 0.5) * 2.0 ** -32
    u2 = (w[:, 1] + 0.5) * 2.0 ** -32
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * np.pi * u2
    out = np.empty_like(w)
    out[:, 0] = r * np.cos(t)
    out[:, 1] = r * np.sin(t)
    return out.reshape(-1)


def normal_f64(seed: int, name: str, n: int, start: int = 0) -> np.ndarray:
    """Standard normal draws ``start .. start+n-1`` of a stream, float64."""
    a = (start // 4) * 4
    b = ((start + n + 3) // 4) * 4
    z = _box_muller(stream_u32(seed, name, b - a, a))
    return z[start - a:start - a + n]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_philox.so")
_lib = None


def build_host_generator() -> str:
    """Compile the C implementation of the generator (``_philox.so``)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
           "-o", _SO, os.path.join(_HERE, "_philox.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return _SO


def _c():
    """The compiled generator, or None when it has not been built."""
    global _lib
    if _lib is None and os.path.exists(_SO):
        lib = ctypes.CDLL(_SO)
        lib.synth_normal.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_int, ctypes.c_void_p]
        lib.synth_u32.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_void_p]
        lib.synth_token_ids.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                        ctypes.c_uint32, ctypes.c_void_p]
        _lib = lib
    return _lib


def normal(seed: int, name: str, shape, std: float, mean: float = 0.0,
           dtype: str = "f32", chunk: int = 1 << 24, use_c: bool = True,
           start: int = 0) -> np.ndarray:
    """N(mean, std) tensor of the given shape, from draws ``start ..`` of the
    stream (``start`` > 0 takes a slice of a longer tensor drawn from 0).

    ``dtype="f32"`` returns float32; ``dtype="bf16"`` returns the uint16 bf16
    bit patterns (use :func:`bf16_bits_to_f32` for the values).  ``mean`` is
    added in float64 before the float32 rounding.
    """
    shape = tuple(int(s) for s in np.atleast_1d(shape)) if not isinstance(shape, tuple) else shape
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)
    lib = _c() if use_c else None
    if lib is not None:
        lib.synth_normal(seed & 0xFFFFFFFF, fnv1a32(name), int(start), n, float(std), float(mean),
                         1 if dtype == "bf16" else 0, out.ctypes.data)
        return out.reshape(shape)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        v = (normal_f64(seed, name, m, start + s) * float(std) + float(mean)).astype(np.float32)
        out[s:s + m] = f32_to_bf16_bits(v) if dtype == "bf16" else v
    return out.reshape(shape)


def token_ids(seed: int, name: str, n: int, vocab: int, use_c: bool = True) -> np.ndarray:
    """Uniform token ids in [0, vocab): ``(x * vocab) >> 32``."""
    lib = _c() if use_c else None
    if lib is not None:
        out = np.empty(n, np.int32)
        lib.synth_token_ids(seed & 0xFFFFFFFF, fnv1a32(name), n, vocab, out.ctypes.data)
        return out
    x = stream_u32(seed, name, n).astype(np.uint64)
    return ((x * np.uint64(vocab)) >> np.uint64(32)).astype(np.int32)
