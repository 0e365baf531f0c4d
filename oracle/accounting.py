"""Execution counts, cache sizes, parameter and FLOP accounting.

[P1 section 2]: executions = head + block * passes + tail; per-layer
parameters estimated from hidden 4096 / FFN 12288 as the three SwiGLU
matrices plus the attention projections (about 230 M); executed-parameter
and per-token FLOP estimates (about 2 FLOP per parameter per execution,
attention ignored).
[P1 section 4] and its table: full-attention KV per token per execution =
KV heads * head dim * 2 (K and V) * 2 bytes (bf16); only full-attention
executions hold KV; Gated-DeltaNet executions hold a state whose size does
not depend on the context length.
"""

from __future__ import annotations

from .config import Config, schedule


def exec_counts(cfg: Config) -> dict:
    rows = schedule(cfg)
    return dict(n_exec=len(rows),
                n_full=sum(r.kind == "full" for r in rows),
                n_gdn=sum(r.kind == "gdn" for r in rows),
                n_loop=sum(r.loop for r in rows))


def kv_bytes_per_token_per_exec(cfg: Config, bytes_per_elem: int = 2) -> int:
    return cfg.n_kv_heads * cfg.head_dim * 2 * bytes_per_elem


def kv_bytes(cfg: Config, batch: int, seq_len: int) -> int:
    """Bytes of bf16 K and V over all full-attention executions."""
    return exec_counts(cfg)["n_full"] * kv_bytes_per_token_per_exec(cfg) * batch * seq_len


def state_bytes(cfg: Config, batch: int) -> int:
    """Bytes of the fp32 Gated-DeltaNet states over all GDN executions."""
    return exec_counts(cfg)["n_gdn"] * cfg.gdn_heads * cfg.gdn_dk * cfg.gdn_dv * 4 * batch


def layer_params_exact(cfg: Config, kind: str) -> int:
    """Parameters of one weight layer under the readings taken here
    (fused input projections, no biases, RMSNorm gains)."""
    d, F = cfg.d_model, cfg.d_ff
    ffn = 3 * d * F
    norms = 2 * d
    if kind == "full":
        qgkv = (2 * cfg.n_q_heads * cfg.head_dim + 2 * cfg.n_kv_heads * cfg.head_dim) * d
        o = d * cfg.n_q_heads * cfg.head_dim
        return ffn + qgkv + o + norms + 2 * cfg.head_dim
    H, Dk, Dv = cfg.gdn_heads, cfg.gdn_dk, cfg.gdn_dv
    inp = (2 * H * Dk + 2 * H * Dv + 2 * H) * d
    o = d * H * Dv
    return ffn + inp + o + norms + Dv


def layer_params_recipe(cfg: Config) -> int:
    """[P1 section 2]'s estimate: three SwiGLU matrices plus attention
    projections taken as five d x d matrices (q, k, v, o and the output
    gate).  3*d*F + 5*d^2 = 234.9 M at d=4096, F=12288."""
    d, F = cfg.d_model, cfg.d_ff
    return 3 * d * F + 5 * d * d


def executed_params(cfg: Config, per_layer: int) -> dict:
    c = exec_counts(cfg)
    head_tail = cfg.loop_start + (cfg.n_layers - cfg.loop_end)
    block = (cfg.loop_end - cfg.loop_start) * cfg.loop_passes
    return dict(stored=cfg.n_layers * per_layer, head_tail=head_tail * per_layer,
                loop=block * per_layer, executed=c["n_exec"] * per_layer,
                embedding=cfg.vocab * cfg.d_model)


def flops_per_token_estimate(n_exec: int, per_layer: float) -> float:
    """About 2 FLOP per parameter per layer execution, attention ignored."""
    return 2.0 * per_layer * n_exec


def gemm_flops_per_token_exact(cfg: Config) -> int:
    """2 * (executed layer matrix parameters) per token, norms excluded."""
    total = 0
    for r in schedule(cfg):
        total += 2 * (layer_params_exact(cfg, r.kind) - 2 * cfg.d_model
                      - (2 * cfg.head_dim if r.kind == "full" else cfg.gdn_dv))
    return total
