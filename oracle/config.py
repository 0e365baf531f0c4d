"""Model configuration and the layer-execution schedule.

[P1 section 2], [P2 section 2]: the decoder stores ``n_layers`` weight layers;
layers ``[0, loop_start)`` run once, the block ``[loop_start, loop_end)`` runs
``loop_passes`` times in a row with the same weights (B(B(h)) for two passes),
then ``[loop_end, n_layers)`` run once and the head follows.  For the full
model 4 + 24*2 + 4 = 56 executions.

[P1 section 3], [P2 section 2]: every 4-layer group is three Gated-DeltaNet
layers followed by one full-attention layer, and the loop boundaries fall on
group boundaries, so both passes see the same order.  Reading: within a group
the full-attention layer is the last one, i.e. weight layer ``l`` is full
attention iff ``l % 4 == 3``.

[P1 section 4], [P4 section 01]: every execution keeps its own KV cache (full
attention) or recurrent state (Gated-DeltaNet); the two passes over the shared
block do not share caches.  Reading: slots are numbered by the rank of the
execution among the executions of its kind.

[P1 section 5], [P1 section 6] (``LoopDecoder.forward``): on entering the
loop the hidden state is copied into the streams; on leaving it the streams
are averaged.  Head and tail layers are plain residual layers.

[P4 section 03]: execution indices are 0-based (tap 3 = end of the head,
27 = end of pass 1, 51 = end of pass 2 for the full model).
"""

from __future__ import annotations

from dataclasses import dataclass, asdict


@dataclass(frozen=True)
class Config:
    n_layers: int
    loop_start: int
    loop_end: int
    loop_passes: int
    d_model: int
    d_ff: int
    vocab: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rotary_dim: int
    gdn_heads: int
    gdn_dk: int
    gdn_dv: int
    n_streams: int = 2
    sinkhorn_iters: int = 20
    rope_theta: float = 10000.0
    eps: float = 1e-6

    @classmethod
    def from_dims(cls, dims: dict, **overrides) -> "Config":
        d = {k: dims[k] for k in cls.__dataclass_fields__ if k in dims}
        d.update(overrides)
        return cls(**d)

    def as_dict(self) -> dict:
        return asdict(self)


def layer_kind(cfg: Config, layer: int) -> str:
    """'full' for the last layer of each 4-layer group, else 'gdn'."""
    return "full" if layer % 4 == 3 else "gdn"


@dataclass(frozen=True)
class ExecRow:
    e: int          # execution index, 0-based
    layer: int      # weight layer it runs
    kind: str       # 'full' or 'gdn'
    slot: int       # KV slot (full) or state slot (gdn): rank among its kind
    loop: bool      # inside the looped block (dual-stream residual)
    fork: bool      # first loop execution: copy h into the streams first
    merge: bool     # last loop execution: average the streams afterwards


def exec_layers(cfg: Config) -> list[int]:
    """Weight layer of each execution, in execution order."""
    out = list(range(cfg.loop_start))
    for _ in range(cfg.loop_passes):
        out += list(range(cfg.loop_start, cfg.loop_end))
    out += list(range(cfg.loop_end, cfg.n_layers))
    return out


def schedule(cfg: Config) -> list[ExecRow]:
    layers = exec_layers(cfg)
    n_loop = (cfg.loop_end - cfg.loop_start) * cfg.loop_passes
    first_loop, last_loop = cfg.loop_start, cfg.loop_start + n_loop - 1
    rows, n_full, n_gdn = [], 0, 0
    for e, l in enumerate(layers):
        kind = layer_kind(cfg, l)
        if kind == "full":
            slot, n_full = n_full, n_full + 1
        else:
            slot, n_gdn = n_gdn, n_gdn + 1
        loop = n_loop > 0 and first_loop <= e <= last_loop
        rows.append(ExecRow(e, l, kind, slot, loop, loop and e == first_loop,
                            loop and e == last_loop))
    return rows


def validate(cfg: Config) -> None:
    if not (0 <= cfg.loop_start <= cfg.loop_end <= cfg.n_layers):
        raise ValueError("loop bounds out of range")
    if cfg.loop_start % 4 or cfg.loop_end % 4 or cfg.n_layers % 4:
        raise ValueError("loop bounds and layer count must fall on 4-layer groups")
    if cfg.loop_passes < 1:
        raise ValueError("loop_passes must be >= 1")
    if cfg.n_q_heads % cfg.n_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    if cfg.rotary_dim % 2 or cfg.rotary_dim > cfg.head_dim:
        raise ValueError("rotary_dim must be even and <= head_dim")
