"""Shared set-up of the model-level GPU tests: device weights from the
seeded host draw, arena / workspace buffers, a model handle.  Marshalling
only."""
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
