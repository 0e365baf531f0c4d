"""Whole-model parity on the tiny looped model (12 weight layers run as
4 + 4x2 + 4 = 16 executions, hidden 256): prefill of 256 uniform token ids
then 8 greedy decode steps, GPU against the CPU oracle on the same
bf16-rounded weights.

The oracle runs the pages' precision policy (bf16 backbone tensors, fp32
residual / mHC / state: ``oracle.precision``).  Metric: max |gpu - oracle| /
max |oracle| per tensor.  Bar: 2e-2 for the final hidden states (all
positions) and the logits, unless the oracle itself is less stable than that:
this random-weight model amplifies a relative input perturbation of 1e-7 about
100x at 256 tokens, so evaluations that are identical in exact arithmetic (the
oracle with token-by-token or chunked Gated-DeltaNet, in fp32 or fp64) land
~4e-2 apart once bf16 rounding decisions flip.  The bar is therefore
max(2e-2, 2 x the largest spread among those evaluations) (``parity.bar``),
computed here from the oracle alone.
Next-token argmax (``parity.argmax_ok``): exact wherever the oracle's
evaluations pick the same token; where they disagree (a near-tie that the
order of rounding decides) the GPU's token must be within the bar of the
oracle's best.  Every decode step is compared
with the oracle started from the GPU's own caches (as the prefill and the
earlier steps left them), so the step is judged on its own arithmetic; its bar
is the spread of this step's own evaluations (from the GPU's caches in fp32
and fp64, and from the oracle's own prefill caches), not the prefill's.
Sinkhorn matrices within 1e-4.  Against the plain
fp32 definition the GPU may drift as much as the bf16 policy itself does:
bounded by 2x the policy oracle's own drift.  Decode is teacher-forced
with the oracle's greedy tokens so that every step compares the same inputs.
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from gpu_util import torch_cuda, dev, host, say, rel_err
from model_util import GpuModel, state_from_gpu
from parity import bar, argmax_ok, exact_required, oracle_tokens, margin

pytestmark = pytest.mark.gpu
TOL = 2e-2


def oracle_evals(ocfg, W, W64, ids):
    """The policy oracle evaluated four ways that agree in exact arithmetic."""
    out = []
    for w in (W, W64):
        for ch in (False, True):
            out.append(om.prefill(ocfg, w, [om.SeqState(ocfg)], ids=ids, bf16=True, chunked_gdn=ch))
    return out


@pytest.fixture(scope="module")
def tiny():
    torch = torch_cuda()
    dims = synth.preset("tiny")
    g = GpuModel(torch, dims, max_batch=3, max_seq=512, max_tokens=512)
    ocfg = oracle.Config.from_dims(dims)
    W = om.to_dtype(g.host_weights, np.float32)
    W64 = om.to_dtype(g.host_weights, np.float64)
    yield torch, dims, g, ocfg, W, W64
    g.close()


def test_schedule_matches_oracle(tiny):
    torch, dims, g, ocfg, W, W64 = tiny
    sched = g.L.loop_schedule(g.cfg)
    orows = oracle.schedule(ocfg)
    assert [(r.layer, int(r.kind == "full"), r.slot, int(r.loop), int(r.fork), int(r.merge))
            for r in orows] == [tuple(x) for x in sched]


def test_mhc_sinkhorn_matrices(tiny):
    torch, dims, g, ocfg, W, W64 = tiny
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
    torch, dims, g, ocfg, W, W64 = tiny
    T, V, d = 256, dims["vocab"], dims["d_model"]
    ids = synth.token_ids(synth.SEED_X, "tiny.ids", T, V)
    say("tiny prefill", T)
    d_ids = dev(ids, torch)
    logits = torch.zeros((1, V), dtype=torch.float32, device="cuda")
    hid = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    fin = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    g.L.loop_prefill(g.handle, 1, T, [0], [0], d_tokens=d_ids.data_ptr(), d_logits=logits.data_ptr(),
                     d_hidden_out=hid.data_ptr(), d_final_out=fin.data_ptr(), stream=g.stream())
    torch.cuda.synchronize()
    # four oracle evaluations of the prefill
    runs = []
    for w in (W, W64):
        for ch in (False, True):
            st = [om.SeqState(ocfg)]
            h, lg, _ = om.prefill(ocfg, w, st, ids=ids.reshape(1, -1), bf16=True, chunked_gdn=ch)
            runs.append((w, st, h, lg))
    h_ref, lg_ref = runs[0][2], runs[0][3]
    tol_h, tol_l = bar([r[2] for r in runs]), bar([r[3] for r in runs])
    print("tiny prefill: gpu-vs-oracle hidden %.4f (bar %.4f), logits %.4f (bar %.4f)"
          % (rel_err(host(hid), h_ref[0]), tol_h, rel_err(host(logits), lg_ref), tol_l))
    assert rel_err(host(hid), h_ref[0]) <= tol_h
    assert rel_err(host(logits), lg_ref) <= tol_l
    # the final RMSNorm at every position (d_final_out): the bf16 values the
    # head multiplies, against each evaluation's final norm (bar from their
    # spread), and against the GPU's own h normalised on the host in fp64
    # (one bf16 rounding apart)
    from oracle.ops import rmsnorm
    from oracle.precision import round_bf16
    fins = [round_bf16(rmsnorm(r[2][0].astype(np.float64), W["final_norm"].astype(np.float64), ocfg.eps))
            for r in runs]
    tol_f = bar(fins)
    own = rmsnorm(host(hid).astype(np.float64), W["final_norm"].astype(np.float64), ocfg.eps)
    print("tiny final norm: gpu-vs-oracle %.4f (bar %.4f), vs its own h %.2e"
          % (rel_err(host(fin), fins[0]), tol_f, rel_err(host(fin), own)))
    assert rel_err(host(fin), fins[0]) <= tol_f
    assert rel_err(host(fin), own) <= 2.0 ** -7
    exact = 0
    ev_l = [r[3][0] for r in runs]
    print("tiny prefill greedy: gpu %d, oracle %s, margin %.4f"
          % (int(np.argmax(host(logits)[0])), oracle_tokens(ev_l), margin(ev_l[0])))
    assert argmax_ok(int(np.argmax(host(logits)[0])), ev_l, tol_l, exact_if_unanimous=True)
    exact += exact_required(ev_l, tol_l, exact_if_unanimous=True)
    # against the fp32 definition: no worse than the bf16 policy's own drift
    h32, lg32, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], ids=ids.reshape(1, -1))
    assert rel_err(host(hid), h32[0]) <= 2 * max(rel_err(r[2][0], h32[0]) for r in runs)
    tok = int(om.argmax_lowest(lg_ref)[0])
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    own = [runs[0], runs[3]]     # fp32 recurrent and fp64 chunked, each continuing its own prefill
    for step in range(8):
        # the oracle decodes from the GPU's own caches (K / V and the
        # Gated-DeltaNet states as the prefill and the earlier steps left
        # them): the GPU is compared with that evaluation, so the step is
        # judged on its own arithmetic.  The bar is the spread of this step's
        # evaluations: from the GPU's caches in fp32 and fp64, and from the
        # oracle's own prefill caches (a correct start that differs by the
        # prefill's rounding)
        sts = [state_from_gpu(g, ocfg, 0, T + step, dt) for dt in (np.float32, np.float64)]
        say("tiny decode step", step)
        d_tok = torch.tensor([tok], dtype=torch.int32, device="cuda")
        g.L.loop_decode_step(g.handle, 1, [0], [T + step], d_tok.data_ptr(), d_logits=logits.data_ptr(),
                             d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), stream=g.stream())
        torch.cuda.synchronize()
        outs = [om.decode_step(ocfg, w, [st], [tok], bf16=True) for w, st in zip((W, W64), sts)]
        outs += [om.decode_step(ocfg, r[0], r[1], [tok], bf16=True) for r in own]
        lg_o, nx_o, h_o = outs[0]
        sl, sh = bar([o[0] for o in outs]), bar([o[2] for o in outs])
        print("tiny decode %d: logits %.4f (bar %.4f, same-cache fp32/fp64 %.4f) hidden %.4f (bar %.4f)"
              % (step, rel_err(host(logits), lg_o), sl, rel_err(outs[1][0], lg_o), rel_err(host(hid)[0], h_o[0]), sh))
        assert rel_err(host(logits), lg_o) <= sl, step
        assert rel_err(host(hid)[0], h_o[0]) <= sh, step
        ev_l = [o[0][0] for o in outs]
        print("tiny decode %d greedy: gpu %d, oracle %s, margin %.4f"
              % (step, int(host(nxt)[0]), oracle_tokens(ev_l), margin(ev_l[0])))
        assert argmax_ok(int(host(nxt)[0]), ev_l, sl, exact_if_unanimous=True), step
        exact += exact_required(ev_l, sl, exact_if_unanimous=True)
        tok = int(nx_o[0])
    print("tiny greedy decisions required to be exact: %d of 9" % exact)


def test_batched_ragged_chunked_prefill(tiny):
    """Two sequences in other slots, prefilled in two chunks of 100 and 37
    tokens (several GDN chunks, a ragged tail, start_pos > 0), equal to the
    oracle's whole prefill of each sequence."""
    torch, dims, g, ocfg, W, W64 = tiny
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
        ev = oracle_evals(ocfg, W, W64, ids[s:s + 1])
        h_ref, lg_ref = ev[0][0], ev[0][1]
        assert rel_err(host(hid)[s * 37:(s + 1) * 37], h_ref[0, 100:]) <= bar([e[0][0, 100:] for e in ev])
        assert rel_err(host(logits)[s], lg_ref[0]) <= bar([e[1][0] for e in ev])
        assert argmax_ok(int(np.argmax(host(logits)[s])), [e[1][0] for e in ev], bar([e[1][0] for e in ev]))


def test_taps(tiny):
    torch, dims, g, ocfg, W, W64 = tiny
    T, V, d = 40, dims["vocab"], dims["d_model"]
    ids = synth.token_ids(synth.SEED_X, "tiny.ids3", T, V)
    taps = [3, 7, 11, 13, 15]
    d_taps = torch.zeros((len(taps), 1, d), dtype=torch.float32, device="cuda")
    d_ids = dev(ids, torch)
    say("tiny taps")
    g.L.loop_prefill(g.handle, 1, T, [0], [0], d_tokens=d_ids.data_ptr(), tap_exec=taps,
                     d_taps=d_taps.data_ptr(), stream=g.stream())
    torch.cuda.synchronize()
    trefs = [om.prefill(ocfg, w, [om.SeqState(ocfg)], ids=ids.reshape(1, -1), taps=tuple(taps), bf16=True,
                        chunked_gdn=ch)[2] for w in (W, W64) for ch in (False, True)]
    for i, e in enumerate(taps):
        assert rel_err(host(d_taps)[i, 0], trefs[0][e][0]) <= bar([t[e][0] for t in trefs]), e


def test_deterministic_rerun(tiny):
    torch, dims, g, ocfg, W, W64 = tiny
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
