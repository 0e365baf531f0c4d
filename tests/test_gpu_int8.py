"""Weight-only int8 decode.

- The device quantizer against the oracle's definition: codes and scales bit
  for bit (integers decided by floating point: both sides divide in fp32,
  correctly rounded), on ragged shapes with a zero row.
- The tiny looped model: bf16 prefill of 256 tokens, then the int8 codes of
  every layer's four projections registered and 4 greedy decode steps
  (teacher-forced) against the oracle decoding with the dequantized codes
  (``oracle.quant.int8_decode_weights``).  Bars ``parity.bar`` per step over
  four oracle evaluations that agree in exact arithmetic (fp32 / fp64, the
  prefill's Gated-DeltaNet token by token / chunked): this random-weight
  model amplifies small differences from step to step, more so with the
  int8 weights.  The int8 oracle is closer to the int8 run than the bf16
  oracle is; with int8 turned off the next step matches the bf16 oracle.
The real-width, split-K variants of the int8 projections are checked in the
batch-64 decode test at 32K context.
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from oracle.quant import quantize_rows_int8, int8_decode_weights, PROJECTIONS
from gpu_util import torch_cuda, dev, host, say, rel_err
from model_util import GpuModel
from parity import bar, argmax_ok

pytestmark = pytest.mark.gpu


def device_int8(torch, L, g, n_layers, stream):
    """Codes and scales of every layer's projections, quantized on the device
    from the model's bf16 matrices: (list of pointer dicts, keep-alive list)."""
    keep, layers = [], []
    for l in range(n_layers):
        d = {}
        for name in PROJECTIONS:
            w = g.dev[f"L{l}.{name}"]
            N, K = w.shape
            q = torch.empty((N, K), dtype=torch.int8, device="cuda")
            sc = torch.empty(N, dtype=torch.float32, device="cuda")
            L.loop_quantize_int8(w.data_ptr(), N, K, K, q.data_ptr(), sc.data_ptr(), stream)
            keep += [q, sc]
            short = {"w_in": "in", "w_o": "o", "w_gateup": "gateup", "w_down": "down"}[name]
            d["w_" + short], d["s_" + short] = q.data_ptr(), sc.data_ptr()
        layers.append(d)
    return layers, keep


@pytest.mark.parametrize("N,K,ld", [(300, 512, 512), (17, 1280, 1300), (5, 128, 128)])
def test_quantize_matches_oracle_bitwise(N, K, ld):
    torch = torch_cuda()
    import looped_hybrid_attention_amd as L
    w = synth.normal(synth.SEED_W, f"q8.{N}.{K}", (N, ld), 0.02, dtype="bf16")
    w[2 % N] = 0  # a zero row
    d_w = dev(w, torch)
    q = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    sc = torch.zeros(N, dtype=torch.float32, device="cuda")
    L.loop_quantize_int8(d_w.data_ptr(), N, K, ld, q.data_ptr(), sc.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    q_ref, s_ref = quantize_rows_int8(synth.bf16_bits_to_f32(w)[:, :K])
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_int8_decode_tiny():
    torch = torch_cuda()
    dims = synth.preset("tiny")
    g = GpuModel(torch, dims, max_batch=1, max_seq=512, max_tokens=512)
    try:
        L, s = g.L, g.stream()
        T, V, d = 256, dims["vocab"], dims["d_model"]
        ocfg = oracle.Config.from_dims(dims)
        W32 = om.to_dtype(g.host_weights, np.float32)
        W64 = om.to_dtype(g.host_weights, np.float64)
        Q32 = int8_decode_weights(W32, dims["n_layers"], np.float32)
        Q64 = int8_decode_weights(W32, dims["n_layers"], np.float64)
        ids = synth.token_ids(synth.SEED_X, "tiny.int8.ids", T, V)
        say("tiny int8: bf16 prefill")
        logits = torch.zeros((1, V), dtype=torch.float32, device="cuda")
        L.loop_prefill(g.handle, 1, T, [0], [0], d_tokens=dev(ids, torch).data_ptr(), d_logits=logits.data_ptr(),
                       stream=s)
        layers, keep = device_int8(torch, L, g, dims["n_layers"], s)
        L.loop_model_set_int8(g.handle, layers)
        # oracle tracks: (prefill weights, decode weights, dtype, chunked GDN)
        tracks = [(W32, Q32, np.float32, False), (W32, Q32, np.float32, True),
                  (W64, Q64, np.float64, False), (W64, Q64, np.float64, True)]
        sts = []
        for Wp, _, dt, ch in tracks:
            st = om.SeqState(ocfg, dt)
            om.prefill(ocfg, Wp, [st], ids=ids.reshape(1, -1), bf16=True, chunked_gdn=ch)
            sts.append(st)
        st_b = om.SeqState(ocfg)
        om.prefill(ocfg, W32, [st_b], ids=ids.reshape(1, -1), bf16=True)
        _, lg_ref, _ = om.prefill(ocfg, W32, [om.SeqState(ocfg)], ids=ids.reshape(1, -1), bf16=True)
        tok = int(om.argmax_lowest(lg_ref)[0])
        nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
        hid = torch.zeros((1, d), dtype=torch.float32, device="cuda")
        for step in range(4):
            say("tiny int8 decode step", step)
            d_tok = torch.tensor([tok], dtype=torch.int32, device="cuda")
            L.loop_decode_step(g.handle, 1, [0], [T + step], d_tok.data_ptr(), d_logits=logits.data_ptr(),
                               d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), stream=s)
            torch.cuda.synchronize()
            outs = [om.decode_step(ocfg, Wd, [st], [tok], bf16=True) for (_, Wd, _, _), st in zip(tracks, sts)]
            o32 = outs[0]
            ob = om.decode_step(ocfg, W32, [st_b], [tok], bf16=True)
            tol_l, tol_h = bar([o[0] for o in outs]), bar([o[2] for o in outs])
            el, eh = rel_err(host(logits), o32[0]), rel_err(host(hid), o32[2])
            eb = rel_err(host(logits), ob[0])
            print("int8 decode %d: logits %.4f (bar %.4f), hidden %.4f (bar %.4f); vs the bf16 oracle %.4f"
                  % (step, el, tol_l, eh, tol_h, eb))
            assert el <= tol_l and eh <= tol_h, step
            assert argmax_ok(int(host(nxt)[0]), [o[0][0] for o in outs], tol_l), step
            assert el < eb, step
            tok = int(o32[1][0])
        # int8 off: the bf16 matrices again (the caches hold the int8 steps, as the oracle's do)
        L.loop_model_set_int8(g.handle, None)
        d_tok = torch.tensor([tok], dtype=torch.int32, device="cuda")
        L.loop_decode_step(g.handle, 1, [0], [T + 4], d_tok.data_ptr(), d_logits=logits.data_ptr(), stream=s)
        torch.cuda.synchronize()
        outs = [om.decode_step(ocfg, W32 if dt == np.float32 else W64, [st], [tok], bf16=True)
                for (_, _, dt, _), st in zip(tracks, sts)]
        assert rel_err(host(logits), outs[0][0]) <= bar([o[0] for o in outs])
        del keep
    finally:
        g.close()
