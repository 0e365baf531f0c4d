"""Dimension presets and the weight-draw recipe of the synthetic workloads.

Plain data: the model dimensions of the three model sizes, the five
workloads that run on them, and, for every weight tensor, its name, shape,
storage type and the normal distribution it is drawn from.  Which weight
layers are full-attention and which are Gated-DeltaNet is passed in by the
caller (each side derives it from its own schedule code).
"""

from __future__ import annotations

import numpy as np

# Model dimensions.  Names follow the pages: d = hidden size, F = FFN size,
# V = vocabulary, Hq/Hkv/D = query heads / KV heads / head dim of the full
# attention, R = rotary dims, H/Dk/Dv = Gated-DeltaNet heads and key/value dims.
PRESETS = {
    # 12 weight layers run 4 + 4x2 + 4 = 16 executions.
    "tiny": dict(n_layers=12, loop_start=4, loop_end=8, loop_passes=2,
                 d_model=256, d_ff=768, vocab=1024,
                 n_q_heads=4, n_kv_heads=1, head_dim=64, rotary_dim=16,
                 gdn_heads=4, gdn_dk=64, gdn_dv=64,
                 n_streams=2, sinkhorn_iters=20, rope_theta=10000.0, eps=1e-6),
    # One shared 4-layer group at real width, run once as a loop block with
    # fork at entry and merge at exit; no embedding or head.
    "group": dict(n_layers=4, loop_start=0, loop_end=4, loop_passes=1,
                  d_model=4096, d_ff=12288, vocab=0,
                  n_q_heads=16, n_kv_heads=4, head_dim=256, rotary_dim=64,
                  gdn_heads=16, gdn_dk=128, gdn_dv=128,
                  n_streams=2, sinkhorn_iters=20, rope_theta=10000.0, eps=1e-6),
    # The full model: 32 weight layers run 4 + 24x2 + 4 = 56 executions.
    "full": dict(n_layers=32, loop_start=4, loop_end=28, loop_passes=2,
                 d_model=4096, d_ff=12288, vocab=248320,
                 n_q_heads=16, n_kv_heads=4, head_dim=256, rotary_dim=64,
                 gdn_heads=16, gdn_dk=128, gdn_dv=128,
                 n_streams=2, sinkhorn_iters=20, rope_theta=10000.0, eps=1e-6),
}

# The five workloads.  "tokens": uniform ids; "hidden": N(0, 1) hidden states.
WORKLOADS = {
    "tiny_prefill_decode": dict(model="tiny", batch=1, seq_len=256, input="tokens",
                                decode_steps=8),
    "group_prefill_4096": dict(model="group", batch=1, seq_len=4096, input="hidden"),
    "full_prefill_8192": dict(model="full", batch=1, seq_len=8192, input="tokens"),
    "full_decode_b64_ctx32768": dict(model="full", batch=64, context=32768, steps=128,
                                     input="tokens", kv_std=1.0, state_std=0.1),
    "full_prefill_131072_chunked": dict(model="full", batch=1, seq_len=131072, chunk=8192,
                                        input="tokens"),
}

WEIGHT_STD = 0.02
MIX_STD = 0.5


def preset(name: str, **overrides) -> dict:
    d = dict(PRESETS[name])
    d.update(overrides)
    return d


def weight_specs(dims: dict, kinds, gain_std: float = 0.0, bias_std: float = 0.0):
    """List of (name, shape, dtype, std, mean) for every weight tensor.

    ``kinds[l]`` is "full" or "gdn" for weight layer ``l``.  Gains are drawn
    N(1, gain_std) and biases N(0, bias_std) (both 0-spread by default:
    gains 1, biases 0).  Matrices are N(0, 0.02) in bf16; the stream-mixing
    parameters are float32, mix logits N(0, 0.5).
    """
    d, F, V = dims["d_model"], dims["d_ff"], dims["vocab"]
    Hq, Hkv, D = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
    H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
    ns = dims["n_streams"]
    specs = []
    if V:
        specs.append(("embed", (V, d), "bf16", WEIGHT_STD, 0.0))
        specs.append(("head", (V, d), "bf16", WEIGHT_STD, 0.0))
    specs.append(("final_norm", (d,), "bf16", gain_std, 1.0))
    for l in range(dims["n_layers"]):
        p = f"L{l}."
        specs.append((p + "attn_norm", (d,), "bf16", gain_std, 1.0))
        specs.append((p + "ffn_norm", (d,), "bf16", gain_std, 1.0))
        if kinds[l] == "full":
            specs.append((p + "w_in", (2 * Hq * D + 2 * Hkv * D, d), "bf16", WEIGHT_STD, 0.0))
            specs.append((p + "w_o", (d, Hq * D), "bf16", WEIGHT_STD, 0.0))
            specs.append((p + "q_norm", (D,), "bf16", gain_std, 1.0))
            specs.append((p + "k_norm", (D,), "bf16", gain_std, 1.0))
        else:
            specs.append((p + "w_in", (2 * H * Dk + 2 * H * Dv + 2 * H, d), "bf16", WEIGHT_STD, 0.0))
            specs.append((p + "w_o", (d, H * Dv), "bf16", WEIGHT_STD, 0.0))
            specs.append((p + "o_norm", (Dv,), "bf16", gain_std, 1.0))
        specs.append((p + "w_gateup", (2 * F, d), "bf16", WEIGHT_STD, 0.0))
        specs.append((p + "w_down", (d, F), "bf16", WEIGHT_STD, 0.0))
        if dims["loop_start"] <= l < dims["loop_end"]:
            specs.append((p + "mhc.read_w", (ns, ns * d), "f32", WEIGHT_STD, 0.0))
            specs.append((p + "mhc.read_b", (ns,), "f32", bias_std, 0.0))
            specs.append((p + "mhc.write_w", (ns, d), "f32", WEIGHT_STD, 0.0))
            specs.append((p + "mhc.write_b", (ns,), "f32", bias_std, 0.0))
            specs.append((p + "mhc.mix", (ns, ns), "f32", MIX_STD, 0.0))
    return specs


def make_weights(dims: dict, kinds, seed: int = 0, gain_std: float = 0.0,
                 bias_std: float = 0.0, only=None) -> dict:
    """Draw the weight tensors on the host.  bf16 tensors are returned as
    uint16 bit patterns.  ``only``: optional predicate on the name."""
    from . import normal
    out = {}
    for name, shape, dt, std, mean in weight_specs(dims, kinds, gain_std, bias_std):
        if only is not None and not only(name):
            continue
        out[name] = normal(seed, name, shape, std, mean=mean, dtype=dt)
    return out


def as_f32(x: np.ndarray) -> np.ndarray:
    """Values of a tensor from :func:`make_weights` as float32."""
    from . import bf16_bits_to_f32
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)
