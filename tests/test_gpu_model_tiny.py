"""Whole-model parity on the tiny looped model (12 weight layers run as
4 + 4x2 + 4 = 16 executions, hidden 256): prefill of 256 uniform token ids
then 8 greedy decode steps, GPU against the CPU oracle on the same
bf16-rounded weights.

The oracle runs the pages' precision policy (bf16 backbone tensors, fp32
residual / mHC / state: ``oracle.precision``).  Metric: max |gpu - oracle| /
max |oracle| per tensor.  Bar: 2e-2 for the final hidden states (all
positions) and the logits, unless the oracle itself is less stable than that:
this random-weight model amplifies a relative input perturbation of 1e-7 about
100x at 256 tokens, so two evaluations that are identical in exact arithmetic
(the oracle with its token-by-token and with its chunked Gated-DeltaNet) land
~4e-2 apart once bf16 rounding decisions flip.  The bar is therefore
max(2e-2, 1.5 * that self-spread + 5e-3), computed here from the oracle alone.
Exact next-token argmax; Sinkhorn matrices within 1e-4.  Against the plain
fp32 definition the GPU may drift as much as the bf16 policy itself does:
bounded by 1.5x the policy oracle's drift + 5e-3.  Decode is teacher-forced
with the oracle's greedy tokens so that every step compares the same inputs.
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from gpu_util import torch_cuda, dev, host, say, rel_err
from model_util import GpuModel

pytestmark = pytest.mark.gpu
TOL = 2e-2


def spread_tol(a, b):
    """Bar for a whole-model comparison: 2e-2, or 1.5x the oracle's own spread
    between two evaluations that are equal in exact arithmetic, + 5e-3."""
    return max(TOL, 1.5 * rel_err(a, b) + 5e-3)


@pytest.fixture(scope="module")
def tiny():
    torch = torch_cuda()
    dims = synth.preset("tiny")
    g = GpuModel(torch, dims, max_batch=3, max_seq=512, max_tokens=512)
    ocfg = oracle.Config.from_dims(dims)
    W = om.to_dtype(g.host_weights, np.float32)
    yield torch, dims, g, ocfg, W
    g.close()


def test_schedule_matches_oracle(tiny):
    torch, dims, g, ocfg, W = tiny
    sched = g.L.loop_schedule(g.cfg)
    orows = oracle.schedule(ocfg)
    assert [(r.layer, int(r.kind == "full"), r.slot, int(r.loop), int(r.fork), int(r.merge))
            for r in orows] == [tuple(x) for x in sched]


def test_mhc_sinkhorn_matrices(tiny):
    torch, dims, g, ocfg, W = tiny
    say("tiny mhc matrices")
    n = dims["loop_end"] - dims["loop_start"]
    out = torch.zeros(n * 4, dtype=torch.float32, device="cuda")
    g.L.loop_debug_mhc(g.handle, out.data_ptr(), g.stream())
    torch.cuda.synchronize()
    got = host(out).reshape(n, 2, 2)
    for i in range(n):
        ref = oracle.mhc.sinkhorn(W[f"L{dims['loop_start'] + i}.mhc.mix"], dims["sinkhorn_iters"])
        assert np.abs(got[i] - ref).max() <= 1e-4
        assert np.abs(got[i].sum(0) - 1).max() <= 1e-5 and np.abs(got[i].sum(1) - 1).max() <= 1e-5


def test_prefill_and_greedy_decode(tiny):
    torch, dims, g, ocfg, W = tiny
    T, V, d = 256, dims["vocab"], dims["d_model"]
    ids = synth.token_ids(synth.SEED_X, "tiny.ids", T, V)
    say("tiny prefill", T)
    d_ids = dev(ids, torch)
    logits = torch.zeros((1, V), dtype=torch.float32, device="cuda")
    hid = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    g.L.loop_prefill(g.handle, 1, T, [0], [0], d_tokens=d_ids.data_ptr(), d_logits=logits.data_ptr(),
                     d_hidden_out=hid.data_ptr(), stream=g.stream())
    torch.cuda.synchronize()
    st = [om.SeqState(ocfg)]
    h_ref, lg_ref, _ = om.prefill(ocfg, W, st, ids=ids.reshape(1, -1), bf16=True)
    h_c, lg_c, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], ids=ids.reshape(1, -1), bf16=True,
                              chunked_gdn=True)
    tol_h, tol_l = spread_tol(h_c, h_ref), spread_tol(lg_c, lg_ref)
    print("tiny prefill: gpu-vs-oracle hidden %.4f (bar %.4f), logits %.4f (bar %.4f)"
          % (rel_err(host(hid), h_ref[0]), tol_h, rel_err(host(logits), lg_ref), tol_l))
    assert rel_err(host(hid), h_ref[0]) <= tol_h
    assert rel_err(host(logits), lg_ref) <= tol_l
    assert int(np.argmax(host(logits)[0])) == int(om.argmax_lowest(lg_ref)[0])
    # against the fp32 definition: no worse than the bf16 policy's own drift
    h32, lg32, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], ids=ids.reshape(1, -1))
    bound = 1.5 * rel_err(h_ref[0], h32[0]) + 5e-3
    assert rel_err(host(hid), h32[0]) <= bound
    tok = int(om.argmax_lowest(lg_ref)[0])
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    for step in range(8):
        say("tiny decode step", step)
        d_tok = torch.tensor([tok], dtype=torch.int32, device="cuda")
        g.L.loop_decode_step(g.handle, 1, [0], [T + step], d_tok.data_ptr(), d_logits=logits.data_ptr(),
                             d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), stream=g.stream())
        torch.cuda.synchronize()
        lg_o, nx_o, h_o = om.decode_step(ocfg, W, st, [tok], bf16=True)
        print("tiny decode %d: logits %.4f hidden %.4f" % (step, rel_err(host(logits), lg_o),
                                                          rel_err(host(hid)[0], h_o[0])))
        assert rel_err(host(logits), lg_o) <= tol_l, step
        assert rel_err(host(hid)[0], h_o[0]) <= tol_h, step
        assert int(host(nxt)[0]) == int(nx_o[0]), step
        tok = int(nx_o[0])


def test_batched_ragged_chunked_prefill(tiny):
    """Two sequences in other slots, prefilled in two chunks of 100 and 37
    tokens (several GDN chunks, a ragged tail, start_pos > 0), equal to the
    oracle's whole prefill of each sequence."""
    torch, dims, g, ocfg, W = tiny
    V, d = dims["vocab"], dims["d_model"]
    ids = synth.token_ids(synth.SEED_X, "tiny.ids2", 2 * 137, V).reshape(2, 137)
    hid = torch.zeros((2 * 100, d), dtype=torch.float32, device="cuda")
    logits = torch.zeros((2, V), dtype=torch.float32, device="cuda")
    say("tiny chunked prefill A")
    a = dev(np.ascontiguousarray(ids[:, :100]).reshape(-1), torch)
    g.L.loop_prefill(g.handle, 2, 100, [2, 1], [0, 0], d_tokens=a.data_ptr(), stream=g.stream())
    say("tiny chunked prefill B")
    b = dev(np.ascontiguousarray(ids[:, 100:]).reshape(-1), torch)
    g.L.loop_prefill(g.handle, 2, 37, [2, 1], [100, 100], d_tokens=b.data_ptr(),
                     d_logits=logits.data_ptr(), d_hidden_out=hid.data_ptr(), stream=g.stream())
    torch.cuda.synchronize()
    for s in range(2):
        h_ref, lg_ref, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], ids=ids[s:s + 1], bf16=True)
        h_c, lg_c, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], ids=ids[s:s + 1], bf16=True,
                                  chunked_gdn=True)
        assert rel_err(host(hid)[s * 37:(s + 1) * 37], h_ref[0, 100:]) <= spread_tol(h_c[0, 100:], h_ref[0, 100:])
        assert rel_err(host(logits)[s], lg_ref[0]) <= spread_tol(lg_c[0], lg_ref[0])
        assert int(np.argmax(host(logits)[s])) == int(np.argmax(lg_ref[0]))


def test_taps(tiny):
    torch, dims, g, ocfg, W = tiny
    T, V, d = 40, dims["vocab"], dims["d_model"]
    ids = synth.token_ids(synth.SEED_X, "tiny.ids3", T, V)
    taps = [3, 7, 11, 13, 15]
    d_taps = torch.zeros((len(taps), 1, d), dtype=torch.float32, device="cuda")
    d_ids = dev(ids, torch)
    say("tiny taps")
    g.L.loop_prefill(g.handle, 1, T, [0], [0], d_tokens=d_ids.data_ptr(), tap_exec=taps,
                     d_taps=d_taps.data_ptr(), stream=g.stream())
    torch.cuda.synchronize()
    _, _, tref = om.prefill(ocfg, W, [om.SeqState(ocfg)], ids=ids.reshape(1, -1), taps=tuple(taps),
                            bf16=True)
    for i, e in enumerate(taps):
        assert rel_err(host(d_taps)[i, 0], tref[e][0]) <= TOL, e


def test_deterministic_rerun(tiny):
    torch, dims, g, ocfg, W = tiny
    T, V, d = 96, dims["vocab"], dims["d_model"]
    ids = dev(synth.token_ids(synth.SEED_X, "tiny.ids4", T, V), torch)
    outs = []
    for rep in range(2):
        say("tiny rerun", rep)
        hid = torch.zeros((T, d), dtype=torch.float32, device="cuda")
        g.L.loop_prefill(g.handle, 1, T, [0], [0], d_tokens=ids.data_ptr(), d_hidden_out=hid.data_ptr(),
                         stream=g.stream())
        torch.cuda.synchronize()
        outs.append(host(hid))
    assert np.array_equal(outs[0], outs[1])
