"""Multi-token verify step on the tiny looped model: two sequences prefilled
(200 and 150 tokens), then k = 5 drafted tokens each checked in one call.
Logits, greedy next tokens, final hidden states and the drafter taps at every
one of the 5 positions are compared with the CPU oracle run token by token
over the same tokens (teacher-forced), bars as in the tiny-model test
(``parity.bar`` over the oracle's own evaluations).  Then the documented
rollback: the saved GDN states are restored, the first 3 tokens verified
again from position 200 / 150, and the next decode step continues from there;
both against the oracle."""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from gpu_util import torch_cuda, dev, host, say, rel_err
from model_util import GpuModel
from parity import bar, argmax_ok

pytestmark = pytest.mark.gpu
K = 5
TAPS = (3, 7, 11, 13, 14)


@pytest.fixture(scope="module")
def tiny():
    torch = torch_cuda()
    dims = synth.preset("tiny")
    g = GpuModel(torch, dims, max_batch=2, max_seq=512, max_tokens=512)
    ocfg = oracle.Config.from_dims(dims)
    W = om.to_dtype(g.host_weights, np.float32)
    W64 = om.to_dtype(g.host_weights, np.float64)
    yield torch, dims, g, ocfg, W, W64
    g.close()


def oracle_steps(ocfg, Ws, prefix, toks):
    """Per evaluation (weights, chunked GDN or not): logits [K, V], hidden
    [K, d], taps {e: [K, d]} of the tokens `toks` after prefilling `prefix`."""
    out = []
    for w in Ws:
        for ch in (False, True):
            st = om.SeqState(ocfg)
            om.prefill(ocfg, w, [st], ids=prefix.reshape(1, -1), bf16=True, chunked_gdn=ch)
            lg, hs, tp = [], [], {e: [] for e in TAPS}
            for t in toks:
                h, l, taps = om.prefill(ocfg, w, [st], ids=np.array([[t]]), taps=TAPS, bf16=True, chunked_gdn=ch)
                lg.append(l[0])
                hs.append(h[0, 0])
                for e in TAPS:
                    tp[e].append(taps[e][0])
            out.append((np.stack(lg), np.stack(hs), {e: np.stack(v) for e, v in tp.items()}, st))
    return out


def test_verify_k5_then_rollback(tiny):
    torch, dims, g, ocfg, W, W64 = tiny
    V, d = dims["vocab"], dims["d_model"]
    T0 = [200, 150]
    ids = [synth.token_ids(synth.SEED_X, f"tiny.verify.{s}", T0[s] + K + 1, V) for s in range(2)]
    s = g.stream()
    say("tiny verify: prefill")
    for b in range(2):
        g.L.loop_prefill(g.handle, 1, T0[b], [b], [0], d_tokens=dev(ids[b][:T0[b]], torch).data_ptr(), stream=s)
    # save the GDN states of both sequences (the rollback contract)
    n_gdn = sum(1 for r in g.L.loop_schedule(g.cfg) if not r[1])
    st_bytes = dims["gdn_heads"] * dims["gdn_dv"] * dims["gdn_dk"] * 4
    offs = [g.L.loop_cache_offset(g.cfg, 2, j, b) for j in range(n_gdn) for b in range(2)]
    saved = [g.arena[o:o + st_bytes].clone() for o in offs]

    toks = np.stack([ids[b][T0[b]:T0[b] + K] for b in range(2)]).astype(np.int32)
    d_tok = dev(toks.reshape(-1), torch)
    logits = torch.zeros((2 * K, V), dtype=torch.float32, device="cuda")
    nxt = torch.zeros(2 * K, dtype=torch.int32, device="cuda")
    hid = torch.zeros((2 * K, d), dtype=torch.float32, device="cuda")
    taps = torch.zeros((len(TAPS), 2 * K, d), dtype=torch.float32, device="cuda")
    say("tiny verify k =", K)
    g.L.loop_verify_step(g.handle, 2, K, [0, 1], T0, d_tok.data_ptr(), d_logits=logits.data_ptr(),
                         d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), tap_exec=TAPS,
                         d_taps=taps.data_ptr(), stream=s)
    torch.cuda.synchronize()
    lg_g, nx_g, h_g, tp_g = host(logits), host(nxt), host(hid), host(taps)
    for b in range(2):
        ev = oracle_steps(ocfg, (W, W64), ids[b][:T0[b]], toks[b])
        tol_l = bar([e[0] for e in ev])
        tol_h = bar([e[1] for e in ev])
        el, eh = rel_err(lg_g[b * K:(b + 1) * K], ev[0][0]), rel_err(h_g[b * K:(b + 1) * K], ev[0][1])
        print("verify seq %d: logits %.4f (bar %.4f), hidden %.4f (bar %.4f)" % (b, el, tol_l, eh, tol_h))
        assert el <= tol_l and eh <= tol_h
        for j in range(K):
            assert int(nx_g[b * K + j]) == int(np.argmax(lg_g[b * K + j]))
            assert argmax_ok(int(nx_g[b * K + j]), [e[0][j] for e in ev], tol_l), (b, j)
        for i, e in enumerate(TAPS):
            assert rel_err(tp_g[i, b * K:(b + 1) * K], ev[0][2][e]) <= bar([x[2][e] for x in ev]), (b, e)

    # rollback: restore the states, verify the first 3 tokens again, then decode the 4th
    for o, t in zip(offs, saved):
        g.arena[o:o + st_bytes].copy_(t)
    say("tiny verify after rollback, k = 3")
    d_tok3 = dev(np.ascontiguousarray(toks[:, :3]).reshape(-1), torch)
    g.L.loop_verify_step(g.handle, 2, 3, [0, 1], T0, d_tok3.data_ptr(), d_logits=logits.data_ptr(), stream=s)
    d_one = dev(np.ascontiguousarray(toks[:, 3]), torch)
    dl = torch.zeros((2, V), dtype=torch.float32, device="cuda")
    g.L.loop_decode_step(g.handle, 2, [0, 1], [T0[0] + 3, T0[1] + 3], d_one.data_ptr(), d_logits=dl.data_ptr(),
                         stream=s)
    torch.cuda.synchronize()
    lg3, dl_g = host(logits)[:6], host(dl)
    for b in range(2):
        ev = oracle_steps(ocfg, (W, W64), ids[b][:T0[b]], toks[b][:4])
        tol_l = bar([e[0] for e in ev])
        assert rel_err(lg3[b * 3:(b + 1) * 3], ev[0][0][:3]) <= tol_l, b
        assert rel_err(dl_g[b], ev[0][0][3]) <= tol_l, b


def test_verify_rejects_bad_arguments(tiny):
    torch, dims, g, ocfg, W, W64 = tiny
    t = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(Exception):
        g.L.loop_verify_step(g.handle, 1, 17, [0], [0], t.data_ptr(), stream=g.stream())  # k > 16
    with pytest.raises(Exception):
        g.L.loop_verify_step(g.handle, 1, 4, [0], [510], t.data_ptr(), stream=g.stream())  # past max_seq
    with pytest.raises(Exception):
        g.L.loop_verify_step(g.handle, 1, 4, [0], [0], t.data_ptr(), d_next=t.data_ptr(), stream=g.stream())
