"""The decode step captured in a HIP graph (loop_decode_graph_*) against the
eager loop_decode_step: the graph's launches must reproduce the eager steps
bit for bit (same kernels, same launch shapes), with the graph feeding each
step's greedy token to the next on the device and advancing its own
positions.

Two identical batches are prefilled into different cache slots; one is
decoded eagerly, the other by graph launches interleaved with the eager steps
(so the shared workspace and the program's own work sit between replays, and
every replay is checked, not only the first).  Tiny model (12 layers, 16
executions) at batch 2 with ragged prompt lengths, then one real-width group
(d 4096, GDN 16 x 128, 16 Q / 4 KV heads x 256) at batch 1, the batch-1
decode configuration.  The eager path itself is compared with the oracle by
the model and decode tests."""
import numpy as np
import pytest

import synth
from gpu_util import torch_cuda, say
from model_util import GpuModel

pytestmark = pytest.mark.gpu


def _run(torch, g, prompts, steps, vocab):
    L = g.L
    B = len(prompts)
    s = g.stream()
    eager_slots = list(range(B))
    graph_slots = list(range(B, 2 * B))
    lens = [len(p) for p in prompts]
    for slots in (eager_slots, graph_slots):
        for b, p in enumerate(prompts):  # ragged prompts: one prefill per sequence
            ids = torch.tensor(p, dtype=torch.int32, device="cuda")
            L.loop_prefill(g.handle, 1, len(p), [slots[b]], [0], d_tokens=ids.data_ptr(), stream=s)
    first = torch.tensor([p[-1] for p in prompts], dtype=torch.int32, device="cuda")
    tok_e = first.clone()
    next_e = torch.zeros(B, dtype=torch.int32, device="cuda")
    log_e = torch.zeros(B, vocab, dtype=torch.float32, device="cuda")
    tok_g = first.clone()  # the graph's input and greedy output
    log_g = torch.zeros(B, vocab, dtype=torch.float32, device="cuda")
    hid_g = torch.zeros(B, g.dims["d_model"], dtype=torch.float32, device="cuda")
    hid_e = torch.zeros_like(hid_g)
    graph = L.loop_decode_graph_create(g.handle, B, graph_slots, lens, tok_g.data_ptr(), steps,
                                       d_logits=log_g.data_ptr(), d_next=tok_g.data_ptr(),
                                       d_hidden_out=hid_g.data_ptr())
    try:
        for t in range(steps):
            pos = [n + t for n in lens]
            L.loop_decode_step(g.handle, B, eager_slots, pos, tok_e.data_ptr(), d_logits=log_e.data_ptr(),
                               d_next=next_e.data_ptr(), d_hidden_out=hid_e.data_ptr(), stream=s)
            torch.cuda.synchronize()
            ref_logits, ref_next, ref_hid = log_e.clone(), next_e.clone(), hid_e.clone()
            tok_e.copy_(next_e)
            _ = (log_e * 2).sum().item()  # eager torch work between the replays
            L.loop_decode_graph_launch(graph, s)
            torch.cuda.synchronize()
            same_logits = torch.equal(log_g, ref_logits)
            same_hidden = torch.equal(hid_g, ref_hid)
            same_next = torch.equal(tok_g, ref_next)
            say(f"decode graph step {t}: logits identical {same_logits}, hidden identical {same_hidden}, "
                f"tokens {tok_g.tolist()} vs {ref_next.tolist()}")
            assert same_logits and same_hidden and same_next, f"graph step {t} differs from the eager step"
            assert L.loop_decode_graph_positions(graph, B) == [n + t + 1 for n in lens]
        with pytest.raises(L.LoopError) as e:
            L.loop_decode_graph_launch(graph, s)
        assert e.value.code == -3  # LOOP_ECAPACITY: all of its steps were launched
    finally:
        L.loop_decode_graph_destroy(graph)


def test_decode_graph_tiny_matches_eager():
    torch = torch_cuda()
    dims = synth.preset("tiny")
    g = GpuModel(torch, dims, max_batch=4, max_seq=256, max_tokens=256)
    rng = np.random.default_rng(11)
    prompts = [list(rng.integers(0, dims["vocab"], 37)), list(rng.integers(0, dims["vocab"], 100))]
    say("[gpu-case] decode graph tiny, batch 2, prompts 37 / 100, 6 steps")
    try:
        _run(torch, g, prompts, 6, dims["vocab"])
    finally:
        g.close()


def test_decode_graph_rejects_positions_past_max_seq():
    torch = torch_cuda()
    dims = synth.preset("tiny")
    g = GpuModel(torch, dims, max_batch=2, max_seq=128, max_tokens=128)
    L = g.L
    try:
        tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        with pytest.raises(L.LoopError) as e:
            L.loop_decode_graph_create(g.handle, 1, [0], [120], tok.data_ptr(), 9)
        assert e.value.code == -3  # 120 + 9 > 128
        with pytest.raises(L.LoopError) as e:
            L.loop_decode_graph_create(g.handle, 1, [0], [5], tok.data_ptr(), 0)
        assert e.value.code == -1
    finally:
        g.close()


def test_decode_graph_group_batch1_matches_eager():
    torch = torch_cuda()
    dims = dict(synth.preset("group"), vocab=1024)
    g = GpuModel(torch, dims, max_batch=2, max_seq=512, max_tokens=512)
    rng = np.random.default_rng(12)
    prompts = [list(rng.integers(0, dims["vocab"], 300))]
    say("[gpu-case] decode graph real-width group, batch 1, prompt 300, 4 steps")
    try:
        _run(torch, g, prompts, 4, dims["vocab"])
    finally:
        g.close()
