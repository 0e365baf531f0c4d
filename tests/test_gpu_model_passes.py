"""Block pass count per call on the tiny looped model: a model configured for
3 passes of the shared block (4 + 4x3 + 4 = 20 executions) serves sequences
run with 3, 2 and 1 passes (20, 16 and 12 executions), each against the CPU
oracle configured with that pass count, on the same weights: prefill of 256
token ids, then 3 greedy decode steps (teacher-forced with the oracle's
tokens; the oracle decodes from the GPU's own caches).  Bars as in the tiny-model test (``parity.bar`` over the oracle's own
evaluations).  A call that changes a sequence's pass count is rejected."""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from gpu_util import torch_cuda, dev, host, say, rel_err
from model_util import GpuModel, state_from_gpu, pass_slot_map
from parity import bar, argmax_ok

pytestmark = pytest.mark.gpu
T = 256


@pytest.fixture(scope="module")
def tiny3():
    torch = torch_cuda()
    dims = dict(synth.preset("tiny"), loop_passes=3)
    g = GpuModel(torch, dims, max_batch=3, max_seq=512, max_tokens=512)
    W = om.to_dtype(g.host_weights, np.float32)
    W64 = om.to_dtype(g.host_weights, np.float64)
    yield torch, dims, g, W, W64
    g.close()


@pytest.mark.parametrize("passes,slot", [(3, 0), (2, 1), (1, 2)])
def test_pass_count_per_call(tiny3, passes, slot):
    torch, dims, g, W, W64 = tiny3
    V, d = dims["vocab"], dims["d_model"]
    ocfg = oracle.Config.from_dims(dict(dims, loop_passes=passes))
    assert len(oracle.schedule(ocfg)) == 4 + 4 * passes + 4
    ids = synth.token_ids(synth.SEED_X, f"tiny.passes.{passes}", T, V)
    say("tiny prefill with", passes, "passes")
    d_ids = dev(ids, torch)
    logits = torch.zeros((1, V), dtype=torch.float32, device="cuda")
    hid = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    # the configuration's count is asked for as 0
    g.L.loop_prefill(g.handle, 1, T, [slot], [0], d_tokens=d_ids.data_ptr(), d_logits=logits.data_ptr(),
                     d_hidden_out=hid.data_ptr(), stream=g.stream(), loop_passes=0 if passes == 3 else passes)
    torch.cuda.synchronize()
    runs = []
    for w in (W, W64):
        for ch in (False, True):
            st = [om.SeqState(ocfg)]
            h, lg, _ = om.prefill(ocfg, w, st, ids=ids.reshape(1, -1), bf16=True, chunked_gdn=ch)
            runs.append((w, st, h, lg))
    h_ref, lg_ref = runs[0][2], runs[0][3]
    tol_h, tol_l = bar([r[2] for r in runs]), bar([r[3] for r in runs])
    eh, el = rel_err(host(hid), h_ref[0]), rel_err(host(logits), lg_ref)
    print("passes %d prefill: hidden %.4f (bar %.4f), logits %.4f (bar %.4f)" % (passes, eh, tol_h, el, tol_l))
    assert eh <= tol_h and el <= tol_l
    assert argmax_ok(int(np.argmax(host(logits)[0])), [r[3][0] for r in runs], tol_l)
    tok = int(om.argmax_lowest(lg_ref)[0])
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    smap = pass_slot_map(g.L, g.cfg, passes)
    for step in range(3):
        # the GPU against the oracle decoding from the GPU's own caches (each
        # execution on its slot of the configured schedule); the bar is the
        # spread of this step's evaluations (from the GPU's caches in fp32 /
        # fp64 and from the oracle's own prefill caches)
        sts = [state_from_gpu(g, ocfg, slot, T + step, dt, smap) for dt in (np.float32, np.float64)]
        d_tok = torch.tensor([tok], dtype=torch.int32, device="cuda")
        g.L.loop_decode_step(g.handle, 1, [slot], [T + step], d_tok.data_ptr(), d_logits=logits.data_ptr(),
                             d_next=nxt.data_ptr(), stream=g.stream(), loop_passes=passes)
        torch.cuda.synchronize()
        outs = [om.decode_step(ocfg, w, [st], [tok], bf16=True) for w, st in zip((W, W64), sts)]
        outs += [om.decode_step(ocfg, r[0], r[1], [tok], bf16=True) for r in (runs[0], runs[3])]
        el, bl = rel_err(host(logits), outs[0][0]), bar([o[0] for o in outs])
        print("passes %d decode %d: logits %.4f (bar %.4f)" % (passes, step, el, bl))
        assert el <= bl, step
        assert argmax_ok(int(host(nxt)[0]), [o[0][0] for o in outs], bl), step
        tok = int(outs[0][1][0])
    # a different pass count on this sequence is refused (nothing enqueued)
    other = 1 if passes != 1 else 2
    with pytest.raises(Exception):
        g.L.loop_decode_step(g.handle, 1, [slot], [T + 3], d_tok.data_ptr(), stream=g.stream(), loop_passes=other)
    with pytest.raises(Exception):
        g.L.loop_prefill(g.handle, 1, 4, [slot], [T + 3], d_tokens=d_ids.data_ptr(), stream=g.stream(),
                         loop_passes=other)
    with pytest.raises(Exception):
        g.L.loop_decode_step(g.handle, 1, [slot], [T + 3], d_tok.data_ptr(), stream=g.stream(), loop_passes=4)
