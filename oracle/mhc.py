"""Dual-stream mHC residual of the looped block, and its Sinkhorn normalisation.

[P1 section 5], [P2 section 2], [P4 section 02]: inside the looped block the
model keeps two residual streams; every layer reads its input from the streams
through a learned map, the streams are mixed by a 2x2 matrix pushed towards
doubly stochastic by 20 Sinkhorn iterations, and the layer's output is written
back through a learned map; the routing runs in fp32.  [P1 section 6]
(``sinkhorn``, ``MHC.forward``) gives the dataflow:

* Sinkhorn: in the log domain, subtract the row log-sum-exp, then the column
  log-sum-exp, ``iters`` times, then take a row softmax.
* read: ``r = softmax(W_r [s_0; ...; s_{n-1}] + b_r)`` per token over the
  streams, ``x = sum_s r_s s_s``.
* write: ``w = softmax(W_w out + b_w)``, ``P = Sinkhorn(L)``,
  ``s_s' = sum_t P[s, t] s_t + w_s out``.

Reading (R8 in the design notes): ``out`` is the layer's residual branch
``a + f`` (mixer output plus FFN output), not the whole block output
``x + a + f`` that the reproduction writes.  With one stream this makes the
mHC layer reduce to a plain residual layer, as hyper-connections widen the
single residual.  The reproduction's literal variant is kept behind
``write_full=True`` for comparison.
One parameter set per looped weight layer, used by every pass.
"""

from __future__ import annotations

import numpy as np

from .ops import logsumexp, softmax


def sinkhorn(logits: np.ndarray, iters: int) -> np.ndarray:
    m = np.array(logits, copy=True)
    for _ in range(iters):
        m = m - logsumexp(m, axis=1)
        m = m - logsumexp(m, axis=0)
    return softmax(m, axis=1)


def read(streams: list, w_r: np.ndarray, b_r: np.ndarray):
    """Layer input ``x`` [T, d] and the read weights ``r`` [T, n]."""
    cat = np.concatenate(streams, axis=-1)
    r = softmax(cat @ w_r.T + b_r, axis=-1)
    x = sum(r[:, s:s + 1] * streams[s] for s in range(len(streams)))
    return x, r


def write(streams: list, out: np.ndarray, w_w: np.ndarray, b_w: np.ndarray,
          P: np.ndarray) -> list:
    """New streams after mixing by ``P`` and writing ``out``."""
    wr = softmax(out @ w_w.T + b_w, axis=-1)
    n = len(streams)
    return [sum(P[s, t] * streams[t] for t in range(n)) + wr[:, s:s + 1] * out
            for s in range(n)]


def fork(h: np.ndarray, n: int) -> list:
    return [h.copy() for _ in range(n)]


def merge(streams: list) -> np.ndarray:
    return sum(streams) / streams[0].dtype.type(len(streams))
