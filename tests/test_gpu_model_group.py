"""Whole-group parity at real width: one 4-layer group (GDN, GDN, GDN, full
attention; d 4096, FFN 12288, 16 Q / 4 KV heads x 256, GDN 16 x 128) run as a
loop block of one pass with fork at entry and merge at exit, no embedding or
head, on 4096 tokens of N(0, 1) hidden states -- the one-group workload at its
full size.

GPU against the CPU oracle with the pages' bf16 backbone policy, metric
max |gpu - oracle| / max |oracle| over all positions; bar ``parity.bar`` over
the oracle evaluated with chunked (64, 32) and token-by-token Gated-DeltaNet
(and, for the 64-token prefix, also in fp64).
The plain fp32 definition is reported beside it and bounded by twice the bf16
policy's own drift.
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from gpu_util import torch_cuda, dev, host, say, rel_err
from model_util import GpuModel
from parity import bar as parity_bar, FLAT

pytestmark = pytest.mark.gpu


def test_group_prefill_4096():
    torch = torch_cuda()
    dims = synth.preset("group")
    T, d = 4096, dims["d_model"]
    g = GpuModel(torch, dims, max_batch=1, max_seq=T, max_tokens=T)
    try:
        x = synth.normal(synth.SEED_X, "group.hidden", (T, d), 1.0)
        d_x = dev(x, torch)
        hid = torch.zeros((T, d), dtype=torch.float32, device="cuda")
        say("group prefill", T)
        g.L.loop_prefill(g.handle, 1, T, [0], [0], d_hidden_in=d_x.data_ptr(), d_hidden_out=hid.data_ptr(),
                         stream=g.stream())
        torch.cuda.synchronize()
        got = host(hid)
        assert np.isfinite(got).all()
        ocfg = oracle.Config.from_dims(dims)
        W = om.to_dtype(g.host_weights, np.float32)
        say("group oracle")
        hc, _, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], hidden=x[None], bf16=True, chunked_gdn=True)
        hr, _, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], hidden=x[None], bf16=True)
        h32, _, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], hidden=x[None], chunked_gdn=True)
        from oracle import gdn as og
        orig = og.gdn_chunked
        og.gdn_chunked = lambda *a, **k: orig(*a[:6], chunk=32)
        try:
            hc32, _, _ = om.prefill(ocfg, W, [om.SeqState(ocfg)], hidden=x[None], bf16=True, chunked_gdn=True)
        finally:
            og.gdn_chunked = orig
        bar = parity_bar([hc[0], hr[0], hc32[0]])
        e16 = rel_err(got, hc[0])
        e32 = rel_err(got, h32[0])
        print("group: gpu-vs-policy %.4f (bar %.4f, oracle spread %.4f), gpu-vs-fp32 %.4f, policy-vs-fp32 %.4f"
              % (e16, bar, rel_err(hc[0], hr[0]), e32, rel_err(hc[0], h32[0])))
        assert e16 <= bar
        assert e32 <= 2 * rel_err(hc[0], h32[0])
        # causal: the first rows depend only on the first tokens (sampled prefix)
        W64 = om.to_dtype(g.host_weights, np.float64)
        hps = [om.prefill(ocfg, w, [om.SeqState(ocfg)], hidden=x[None, :64], bf16=True, chunked_gdn=ch)[0][0]
               for w in (W, W64) for ch in (True, False)]
        assert rel_err(got[:64], hps[0]) <= parity_bar(hps + [hc[0, :64], hr[0, :64], hc32[0, :64]])
    finally:
        g.close()


def test_group_prefill_two_calls_taps():
    """The group on 1024 tokens in two calls (500, then 524 at start position
    500: the cached prefix of the full-attention layer and the carried
    Gated-DeltaNet states), with the hidden state after every execution at
    every position.  Execution 0 is held to the flat 2e-2 (the oracle's own
    evaluations agree there to ~0.3 %); executions 1-3 amplify the rounding
    of the bf16 backbone (the oracle's fp32 and fp64 evaluations already
    differ by 1.6-2.8 % there), so they take the noise-floor bar."""
    torch = torch_cuda()
    dims = synth.preset("group")
    d = dims["d_model"]
    split = (500, 524)
    T = sum(split)
    g = GpuModel(torch, dims, max_batch=1, max_seq=T, max_tokens=max(split))
    try:
        x = synth.normal(synth.SEED_X, "group.hidden2", (T, d), 1.0)
        taps = (0, 1, 2, 3)
        got_t, got_h = [], []
        p0 = 0
        for i, n in enumerate(split):
            d_x = dev(x[p0:p0 + n], torch)
            hid = torch.zeros((n, d), dtype=torch.float32, device="cuda")
            tp = torch.zeros((len(taps), n, d), dtype=torch.float32, device="cuda")
            say("group call", i, "tokens", n, "start", p0)
            g.L.loop_prefill(g.handle, 1, n, [0], [p0], d_hidden_in=d_x.data_ptr(), d_hidden_out=hid.data_ptr(),
                             tap_exec=taps, d_taps=tp.data_ptr(), taps_all_positions=True, stream=g.stream())
            torch.cuda.synchronize()
            got_t.append(host(tp))
            got_h.append(host(hid))
            p0 += n
        got_t = np.concatenate(got_t, axis=1)
        got_h = np.concatenate(got_h)
        ocfg = oracle.Config.from_dims(dims)
        evals = []
        for dt, ch in ((np.float32, True), (np.float32, False), (np.float64, True)):
            say("group oracle", np.dtype(dt).name, "chunked" if ch else "recurrent")
            W = om.to_dtype(g.host_weights, dt)
            st = [om.SeqState(ocfg)]
            outs = [om.prefill(ocfg, W, st, hidden=x[None, a:b].astype(dt), bf16=True, chunked_gdn=ch,
                               taps=taps, taps_all=True) for a, b in ((0, split[0]), (split[0], T))]
            evals.append(({e: np.concatenate([o[2][e][0] for o in outs]) for e in taps},
                          np.concatenate([o[0][0] for o in outs])))
        for i, e in enumerate(taps):
            err = rel_err(got_t[i], evals[0][0][e])
            b = parity_bar([v[0][e] for v in evals])
            print("group exec %d: gpu-vs-oracle %.4f (noise bar %.4f)" % (e, err, b))
            assert err <= (FLAT if e == 0 else b), e
        err = rel_err(got_h, evals[0][1])
        b = parity_bar([v[1] for v in evals])
        print("group output: gpu-vs-oracle %.4f (noise bar %.4f)" % (err, b))
        assert err <= b
        assert np.array_equal(got_h, got_t[3])
    finally:
        g.close()
