"""Weight sharing on the GPU: the looped tiny model (12 weight layers run
4 + 4x2 + 4 = 16 executions) against the same model written out -- 16 weight
layers run once, the block's layers and their mHC parameters copied into the
second pass's positions -- bit for bit.

[P1] hncyxsy.com/news/268323 section 2 and section 6 (the reproduction keeps
one module list and runs the block twice): the two passes use the same
weights, so replaying shared weights must give exactly what separate copies
give.  Prefill of 256 token ids (logits, hidden states at every position,
taps after every execution) and 3 greedy decode steps."""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from gpu_util import torch_cuda, dev, host, say
from model_util import GpuModel

pytestmark = pytest.mark.gpu


def test_looped_equals_unrolled_bitwise():
    torch = torch_cuda()
    dims = synth.preset("tiny")
    T, V, d = 256, dims["vocab"], dims["d_model"]
    looped = GpuModel(torch, dims, max_batch=1, max_seq=512, max_tokens=T)
    ocfg = oracle.Config.from_dims(dims)
    ucfg, UW = om.unrolled(ocfg, looped.host_weights)   # copies of the bf16 / fp32 tensors
    udims = dict(dims, **{k: getattr(ucfg, k) for k in ("n_layers", "loop_start", "loop_end", "loop_passes")})
    assert udims["n_layers"] == 16 and udims["loop_passes"] == 1
    unrolled = GpuModel(torch, udims, max_batch=1, max_seq=512, max_tokens=T, host_weights=UW)
    try:
        ids = synth.token_ids(synth.SEED_X, "tiny.unrolled", T, V)
        d_ids = dev(ids, torch)
        taps = list(range(16))
        res = []
        for name, g in (("looped", looped), ("unrolled", unrolled)):
            say("tiny", name)
            lg = torch.zeros((1, V), dtype=torch.float32, device="cuda")
            hid = torch.zeros((T, d), dtype=torch.float32, device="cuda")
            tp = torch.zeros((len(taps), T, d), dtype=torch.float32, device="cuda")
            g.L.loop_prefill(g.handle, 1, T, [0], [0], d_tokens=d_ids.data_ptr(), d_logits=lg.data_ptr(),
                             d_hidden_out=hid.data_ptr(), tap_exec=taps, d_taps=tp.data_ptr(),
                             taps_all_positions=True, stream=g.stream())
            out = [host(lg), host(hid), host(tp)]
            tok = torch.tensor([int(ids[-1])], dtype=torch.int32, device="cuda")
            nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
            for step in range(3):
                g.L.loop_decode_step(g.handle, 1, [0], [T + step], tok.data_ptr(), d_logits=lg.data_ptr(),
                                     d_next=nxt.data_ptr(), stream=g.stream())
                torch.cuda.synchronize()
                out.append(host(lg))
                tok = nxt.clone()
            res.append(out)
        for i, (a, b) in enumerate(zip(*res)):
            assert np.isfinite(a).all()
            assert np.array_equal(a, b), i
    finally:
        looped.close()
        unrolled.close()
