"""Shared set-up of the model-level GPU tests: device weights from the
seeded host draw, arena / workspace buffers, a model handle, and the GPU's
caches read back into the oracle's cache structures.  Marshalling only."""
import numpy as np

import synth
from synth.presets import make_weights
from gpu_util import dev


def kinds_from_schedule(L, cfg, n_layers):
    sched = L.loop_schedule(cfg)
    kinds = {}
    for layer, full, *_ in sched:
        kinds[layer] = "full" if full else "gdn"
    return [kinds[l] for l in range(n_layers)]


class GpuModel:
    def __init__(self, torch, dims, max_batch, max_seq, max_tokens, host_weights=None,
                 gain_std=0.1, bias_std=0.1):
        import looped_hybrid_attention_amd as L
        self.L, self.torch = L, torch
        self.dims = dims
        self.cfg = L.make_config(dims, max_batch=max_batch, max_seq=max_seq, max_tokens=max_tokens)
        self.kinds = kinds_from_schedule(L, self.cfg, dims["n_layers"])
        if host_weights is None:
            host_weights = make_weights(dims, self.kinds, gain_std=gain_std, bias_std=bias_std)
        self.host_weights = host_weights
        self.dev = {k: dev(v, torch) for k, v in host_weights.items()}
        ptrs = {k: t.data_ptr() for k, t in self.dev.items()}
        self.wstruct = L.make_weights_struct(dims["n_layers"], ptrs)
        ab = L.loop_arena_bytes(self.cfg)
        wb = L.loop_workspace_bytes(self.cfg, max_tokens)
        assert ab > 0 and wb > 0
        self.arena = torch.zeros(ab, dtype=torch.uint8, device="cuda")
        self.ws = torch.zeros(wb, dtype=torch.uint8, device="cuda")
        self.handle = L.loop_model_create(self.cfg, self.wstruct, self.arena.data_ptr(), ab,
                                          self.ws.data_ptr(), wb)

    def close(self):
        if self.handle:
            self.L.loop_model_destroy(self.handle)
            self.handle = 0

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream


def device_full_weights(torch, L, dims, kinds, stream):
    """The full model's weights drawn on the device by the seeded generator
    (same stream names and recipe as the host draw): (tensors, weights struct)."""
    from synth.presets import weight_specs
    tensors, ptrs = {}, {}
    for name, shape, dt, std, mean in weight_specs(dims, kinds):
        t = torch.empty(shape, dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda")
        L.loop_synth_normal(t.data_ptr(), t.numel(), 1 if dt == "bf16" else 0, synth.SEED_W,
                            synth.fnv1a32(name), 0, std, mean, stream)
        tensors[name] = t
        ptrs[name] = t.data_ptr()
    return tensors, L.make_weights_struct(dims["n_layers"], ptrs)


def state_from_gpu(g, ocfg, seq_slot, length, dtype, slot_map=None):
    """An oracle SeqState (``oracle.model``) holding the GPU arena's caches of
    sequence slot ``seq_slot``: K, V of every full-attention execution at
    positions 0 .. length-1 (V un-blocked from its 32-position transposed
    blocks) and every Gated-DeltaNet state.  ``slot_map``: {("full" | "gdn",
    oracle slot): arena slot} when the call's schedule is a part of the
    configured one (fewer block passes); default the identity."""
    import torch
    from oracle import model as om
    from gpu_util import host
    L, cfg, dims = g.L, g.cfg, g.dims
    Hkv, D, S = dims["n_kv_heads"], dims["head_dim"], cfg.max_seq
    H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
    st = om.SeqState(ocfg, dtype)
    slot_map = slot_map or {}

    def view(off, n, bf):
        t = g.arena[off:off + n * (2 if bf else 4)]
        return host(t.view(torch.bfloat16 if bf else torch.float32))

    for f in range(st.n_full):
        a = slot_map.get(("full", f), f)
        K = view(L.loop_cache_offset(cfg, 0, a, seq_slot), Hkv * S * D, True).reshape(Hkv, S, D)
        Vb = view(L.loop_cache_offset(cfg, 1, a, seq_slot), Hkv * S * D, True).reshape(Hkv, S // 32, D, 32)
        st.kv[f].k = np.ascontiguousarray(K[:, :length], dtype)
        st.kv[f].v = np.ascontiguousarray(Vb.transpose(0, 1, 3, 2).reshape(Hkv, S, D)[:, :length], dtype)
    for j in range(st.n_gdn):
        a = slot_map.get(("gdn", j), j)
        st.S[j] = view(L.loop_cache_offset(cfg, 2, a, seq_slot), H * Dv * Dk, False).reshape(H, Dv, Dk).astype(dtype)
    st.length = length
    return st


def pass_slot_map(L, cfg, passes):
    """{(kind, slot in the p-pass schedule): slot in the configured schedule}:
    a call with fewer block passes keeps every execution on its slot of the
    full schedule."""
    rows = L.loop_schedule(cfg)
    ls, le = cfg.loop_start, cfg.loop_end
    blk = le - ls
    kept = [r for e, r in enumerate(rows)
            if not (ls <= e < ls + blk * cfg.loop_passes) or (e - ls) // blk < passes]
    out, rank = {}, {"full": 0, "gdn": 0}
    for layer, full, slot, *_ in kept:
        kind = "full" if full else "gdn"
        out[(kind, rank[kind])] = slot
        rank[kind] += 1
    return out
