"""Writes ``full_stack_8192.json``: the oracle's values for the full looped
stack (32 weight layers run 4 + 24x2 + 4 = 56 executions at real width,
vocabulary 248,320) prefilling the 8192 uniform token ids of the full-prefill
workload, for the sampled comparison in ``tests/test_gpu_full_model.py``.

Calls only ``oracle`` and ``synth`` (the seeded inputs).  The weights are the
ones the GPU tests draw on the device (``synth.presets.weight_specs``, seed 0;
host and device generators follow the same published definition), drawn here
one layer at a time; the embedding rows of the 8192 ids are drawn directly
(counter offset id * d).  Two evaluations of the bf16 backbone policy
(Gated-DeltaNet chunked with 64-token chunks, and token by token) give the
noise floor of the comparison.  Stored per evaluation: the logits of the last
position at a fixed sample of vocabulary ids (every 61st id, plus the 16
largest of either evaluation), the final hidden state of the last position
before the final norm (every 2nd dimension), and the greedy token with its
top-1 / top-2 margin over the whole vocabulary.

Run from the repository root (about 30 minutes of host CPU):
    python tests/golden/make_full_stack_8192.py
(``--check N``: the same on the first N tokens, printed, nothing written.)
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import oracle  # noqa: E402
from oracle import model as om  # noqa: E402
from oracle.config import layer_kind  # noqa: E402
from synth.presets import weight_specs  # noqa: E402

T = 8192
IDS_NAME = "test.full.ids"
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "full_stack_8192.json")


class LayerWeights(dict):
    """The model's weights with the layers drawn on demand (one held at a
    time); holds ``final_norm`` and ``head`` itself."""

    def __init__(self, dims, cfg):
        super().__init__()
        kinds = [layer_kind(cfg, l) for l in range(dims["n_layers"])]
        self.specs = {n: (sh, dt, sd, mu) for n, sh, dt, sd, mu in weight_specs(dims, kinds)}
        self.cached = (None, None)
        for name in ("final_norm", "head"):
            self[name] = self.draw(name)

    def draw(self, name):
        shape, dt, std, mean = self.specs[name]
        if dt == "bf16":
            return synth.bf16_bits_to_f32(synth.normal(synth.SEED_W, name, shape, std, mean, dtype="bf16"))
        return synth.normal(synth.SEED_W, name, shape, std, mean)

    def layer(self, l):
        if self.cached[0] != l:
            p = f"L{l}."
            self.cached = (l, {k[len(p):]: self.draw(k) for k in self.specs if k.startswith(p)})
        return self.cached[1]


def embed_rows(dims, ids):
    V, d = dims["vocab"], dims["d_model"]
    assert (0 <= ids).all() and (ids < V).all()
    out = np.empty((len(ids), d), np.float32)
    for i, t in enumerate(ids):
        bits = synth.normal(synth.SEED_W, "embed", (d,), synth.presets.WEIGHT_STD, 0.0, dtype="bf16",
                            start=int(t) * d)
        out[i] = synth.bf16_bits_to_f32(bits)
    return out


def top2_margin(logits):
    x = np.sort(logits.astype(np.float64))
    return float((x[-1] - x[-2]) / np.max(np.abs(x)))


def main():
    n_tok = int(sys.argv[2]) if len(sys.argv) > 2 and sys.argv[1] == "--check" else T
    dims = synth.preset("full")
    cfg = oracle.Config.from_dims(dims)
    V = dims["vocab"]
    ids = synth.token_ids(synth.SEED_X, IDS_NAME, T, V)[:n_tok]
    W = LayerWeights(dims, cfg)
    h0 = embed_rows(dims, ids)
    evals = []
    for label, chunked in (("chunked", True), ("recurrent", False)):
        t0 = time.time()
        h, logits, _ = om.forward_seq(cfg, W, om.SeqState(cfg), hidden=h0, bf16=True, chunked_gdn=chunked)
        print(f"{label}: {time.time() - t0:.0f} s, argmax {int(np.argmax(logits))}", flush=True)
        evals.append((label, h[-1].astype(np.float32), logits.astype(np.float32)))
    if n_tok != T:
        return
    top = set()
    for _, _, lg in evals:
        top.update(int(i) for i in np.argsort(lg)[-16:])
    idx = sorted(set(range(0, V, 61)) | top)
    rec = {
        "source": "oracle.model.forward_seq, bf16 backbone policy, written by tests/golden/make_full_stack_8192.py",
        "workload": {"preset": "full", "tokens": T, "ids_seed": synth.SEED_X, "ids_name": IDS_NAME,
                     "weights_seed": synth.SEED_W},
        "logit_ids": idx,
        "hidden_dims": list(range(0, dims["d_model"], 2)),
        "evals": [
            {"gdn": label,
             "logits": [float(f"{v:.8g}") for v in lg[idx]],
             "hidden_last": [float(f"{v:.8g}") for v in hl[::2]],
             "argmax": int(np.argmax(lg)),
             "margin": top2_margin(lg),
             "max_abs_logit": float(np.max(np.abs(lg)))}
            for label, hl, lg in evals
        ],
    }
    with open(OUT, "w") as f:
        json.dump(rec, f)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
