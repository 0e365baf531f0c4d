"""CPU oracle of the looped hybrid decoder's forward pass (test infrastructure).

This package is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the HIP
library and its Python binding never do.  It shares no code with the HIP path:
the only thing both sides use is the ``synth`` package (seeded inputs, no model
arithmetic).

It is plain NumPy, float32 by default (every routine takes ``dtype`` so that
the pins can run it in float64), with no blocking, fusion or reordering beyond
what the definitions state.

Sources, cited by page address and section (the pages are the text of five web
pages about one looped decoder model):

* [P1] hncyxsy.com/news/268323 -- the technical article: section 2 (loop
  schedule and parameter / FLOP accounting), section 3 (hybrid attention,
  GQA, partial rotary, Gated-DeltaNet), section 4 (KV-cache accounting and its
  table), section 5 (dual-stream mHC residual, Sinkhorn), section 6 (a small
  PyTorch reproduction: ``CFG``, ``sinkhorn``, ``Block``, ``MHC``,
  ``LoopDecoder``), section 7 (deployment, quantisation estimates).
* [P2] yuliuswiki.com/sensenova-loop-9b -- section 2 (B(B(h)), mHC, 3+1 group
  order), section 3 (specification: hidden 4096, FFN 12288, vocab 248,320,
  16 Q / 4 KV heads, bf16 backbone with fp32 mHC routing).
* [P4] yeyulingfeng.com/a/1332585.html -- section 01 (config comparison),
  section 02 (fp32 routing, 20 Sinkhorn-Knopp iterations), section 03
  (draft-model taps at virtual execution indices 3, 27, 51, 53, 54).

Where the pages leave a step open, the reading taken is stated at the routine
(and collected in the design notes of the repository).

Parity status: every routine here is pinned by a ``-m "not gpu"`` test against
closed forms, invariants, brute force or the pages' printed numbers, except
the whole-model forward, whose output values the pages never print: the
whole-model composition is pinned only through its parts and the structural
invariants (looped vs unrolled identity, chunked vs whole prefill,
prefill-then-decode vs longer prefill, single-stream reduction).
"""

from .config import Config, ExecRow, schedule, layer_kind  # noqa: F401
from . import accounting, ops, attention, gdn, mhc, model, quant  # noqa: F401
