"""Decode at real width and full context, in the launch configuration of the
decode benchmark: two 4-layer groups (GDN, GDN, GDN, full attention; d 4096,
FFN 12288, 16 Q / 4 KV heads x 256, GDN 16 x 128), the first run as plain
residual layers and the second as a one-pass loop block (fork, mHC, merge),
with a 1024-token vocabulary, batch 64, every sequence at position 32,768
over pre-filled caches (K and V N(0, 1) bf16 at positions 0..32767 of both
full-attention slots, GDN states N(0, 0.1) fp32), as the decode workload
fills its 14 KV and 42 GDN slots.  This runs the kernels the benchmark
times: the split decode attention over 32,769 keys with its combine, the
Gated-DeltaNet single-token recurrence, the batch-64 projections (plain and
loop epilogues, the split sum fused with the FFN pre-norm).

Sampled: the oracle decodes 3 of the 64 sequences (every step of the path is
independent across sequences: the projections are row-wise, attention and
the recurrence are per sequence).  The cache contents are drawn on the device
by the seeded generator in the documented arena layout (V transposed in
blocks of 32 positions) and
regenerated on the host for the sampled sequences from the same counter
streams.  Metric max |gpu - oracle| / max |oracle| per tensor (logits and
final hidden state of each sampled sequence); bar ``parity.bar`` over the
oracle in fp32 and fp64; greedy token by ``parity.argmax_ok``.  The decode
also appends the new token's K and V at position 32,768: the appended K row
is checked against the oracle's rotated, normalised key.

Then the same step again (GDN states regenerated, the appended position
rewritten) with the weight-only int8 codes of every projection registered:
the batch-64 int8 projections with split K (the in / gate-up / down
widths, and the O-projection's split sum fused with the FFN pre-norm),
against the oracle decoding with the dequantized codes, 2 sampled sequences;
then once more with the int4 group codes (2 other sampled sequences).
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from gpu_util import torch_cuda, dev, host, say, rel_err
from model_util import GpuModel
from parity import bar as parity_bar, argmax_ok
from oracle.quant import int8_decode_weights, int4_decode_weights

pytestmark = pytest.mark.gpu

B, CTX, V = 64, 32768, 1024
SAMPLE = (0, 37, 63)


def test_decode_b64_ctx32768_group():
    torch = torch_cuda()
    dims = synth.preset("group", vocab=V, n_layers=8, loop_start=4, loop_end=8)
    d = dims["d_model"]
    Hkv, D = dims["n_kv_heads"], dims["head_dim"]
    H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
    max_seq = CTX + 64
    g = GpuModel(torch, dims, max_batch=B, max_seq=max_seq, max_tokens=B)
    try:
        L, cfg, s = g.L, g.cfg, g.stream()
        rows = L.loop_schedule(cfg)
        n_full = sum(r[1] for r in rows)
        n_gdn = len(rows) - n_full
        assert n_full == 2 and n_gdn == 6
        kv_n = B * Hkv * max_seq * D
        for f in range(n_full):
            for which, name in ((0, f"test.decode.k.{f}"), (1, f"test.decode.v.{f}")):
                L.loop_synth_normal(g.arena.data_ptr() + L.loop_cache_offset(cfg, which, f, 0), kv_n, 1,
                                    synth.SEED_C, synth.fnv1a32(name), 0, 1.0, 0.0, s)
        st_n = B * H * Dv * Dk
        for j in range(n_gdn):
            L.loop_synth_normal(g.arena.data_ptr() + L.loop_cache_offset(cfg, 2, j, 0), st_n, 0,
                                synth.SEED_C, synth.fnv1a32(f"test.decode.state.{j}"), 0, 0.1, 0.0, s)
        ids = synth.token_ids(synth.SEED_X, "test.decode.ids", B, V)
        d_ids = dev(ids, torch)
        logits = torch.zeros((B, V), dtype=torch.float32, device="cuda")
        hid = torch.zeros((B, d), dtype=torch.float32, device="cuda")
        nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
        say("decode b64 ctx32768 group")
        L.loop_decode_step(g.handle, B, list(range(B)), [CTX] * B, d_ids.data_ptr(), d_logits=logits.data_ptr(),
                           d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), stream=s)
        torch.cuda.synchronize()
        got_l, got_h, got_n = host(logits), host(hid), host(nxt)
        assert np.isfinite(got_l).all() and np.isfinite(got_h).all()
        k0 = L.loop_cache_offset(cfg, 0, n_full - 1, 0)
        k_new = host(g.arena[k0:k0 + kv_n * 2].view(torch.bfloat16).view(B, Hkv, max_seq, D)[:, :, CTX]
                     .contiguous())

        ocfg = oracle.Config.from_dims(dims)
        W32 = om.to_dtype(g.host_weights, np.float32)
        W64 = om.to_dtype(g.host_weights, np.float64)

        def state_of(b, dtype):
            st = om.SeqState(ocfg, dtype)
            per = Hkv * max_seq * D
            for f in range(n_full):
                kb = synth.normal(synth.SEED_C, f"test.decode.k.{f}", (per,), 1.0, dtype="bf16", start=b * per)
                vb = synth.normal(synth.SEED_C, f"test.decode.v.{f}", (per,), 1.0, dtype="bf16", start=b * per)
                K = synth.bf16_bits_to_f32(kb).reshape(Hkv, max_seq, D)[:, :CTX]
                # V cache: [Hkv][max_seq / 32][D][32] (blocks of 32 positions, transposed)
                Vb = synth.bf16_bits_to_f32(vb).reshape(Hkv, max_seq // 32, D, 32)
                Vp = Vb.transpose(0, 1, 3, 2).reshape(Hkv, max_seq, D)[:, :CTX]
                st.kv[f].k = np.ascontiguousarray(K, dtype)
                st.kv[f].v = np.ascontiguousarray(Vp, dtype)
            for j in range(n_gdn):
                per_s = H * Dv * Dk
                S = synth.normal(synth.SEED_C, f"test.decode.state.{j}", (per_s,), 0.1, start=b * per_s)
                st.S[j] = S.reshape(H, Dv, Dk).astype(dtype)
            st.length = CTX
            return st

        for b in SAMPLE:
            say("decode oracle seq", b)
            evals = []
            for W, dt in ((W32, np.float32), (W64, np.float64)):
                st = state_of(b, dt)
                lg, nx, h = om.decode_step(ocfg, W, [st], [int(ids[b])], bf16=True)
                evals.append((lg[0], h[0], st.kv[n_full - 1].k[:, CTX]))
            tol_l = parity_bar([e[0] for e in evals])
            tol_h = parity_bar([e[1] for e in evals])
            el = rel_err(got_l[b], evals[0][0])
            eh = rel_err(got_h[b], evals[0][1])
            ek = rel_err(k_new[b], evals[0][2])
            print("decode seq %d: logits %.4f (bar %.4f), hidden %.4f (bar %.4f), appended K %.4f"
                  % (b, el, tol_l, eh, tol_h, ek))
            assert el <= tol_l, b
            assert eh <= tol_h, b
            assert ek <= 2e-2, b
            assert argmax_ok(int(got_n[b]), [e[0] for e in evals], tol_l), b

        # --- the same step with int8 projections
        from test_gpu_int8 import device_int8
        for j in range(n_gdn):
            L.loop_synth_normal(g.arena.data_ptr() + L.loop_cache_offset(cfg, 2, j, 0), st_n, 0,
                                synth.SEED_C, synth.fnv1a32(f"test.decode.state.{j}"), 0, 0.1, 0.0, s)
        layers, keep = device_int8(torch, L, g, dims["n_layers"], s)
        L.loop_model_set_int8(g.handle, layers)
        say("decode b64 ctx32768 group, int8 projections")
        L.loop_decode_step(g.handle, B, list(range(B)), [CTX] * B, d_ids.data_ptr(), d_logits=logits.data_ptr(),
                           d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), stream=s)
        torch.cuda.synchronize()
        got_l, got_h, got_n = host(logits), host(hid), host(nxt)
        L.loop_model_set_int8(g.handle, None)
        del keep
        Q32 = int8_decode_weights(W32, dims["n_layers"], np.float32)
        Q64 = int8_decode_weights(W32, dims["n_layers"], np.float64)
        for b in SAMPLE[:2]:
            say("int8 decode oracle seq", b)
            evals = []
            for W, dt in ((Q32, np.float32), (Q64, np.float64)):
                st = state_of(b, dt)
                lg, nx, h = om.decode_step(ocfg, W, [st], [int(ids[b])], bf16=True)
                evals.append((lg[0], h[0]))
            tol_l = parity_bar([e[0] for e in evals])
            tol_h = parity_bar([e[1] for e in evals])
            el, eh = rel_err(got_l[b], evals[0][0]), rel_err(got_h[b], evals[0][1])
            print("int8 decode seq %d: logits %.4f (bar %.4f), hidden %.4f (bar %.4f)" % (b, el, tol_l, eh, tol_h))
            assert el <= tol_l and eh <= tol_h, b
            assert argmax_ok(int(got_n[b]), [e[0] for e in evals], tol_l), b
        del Q32, Q64

        # --- the same step with int4 projections
        from test_gpu_int4 import device_int4
        for j in range(n_gdn):
            L.loop_synth_normal(g.arena.data_ptr() + L.loop_cache_offset(cfg, 2, j, 0), st_n, 0,
                                synth.SEED_C, synth.fnv1a32(f"test.decode.state.{j}"), 0, 0.1, 0.0, s)
        layers, keep = device_int4(torch, L, g, dims["n_layers"], s)
        L.loop_model_set_int4(g.handle, layers)
        say("decode b64 ctx32768 group, int4 projections")
        L.loop_decode_step(g.handle, B, list(range(B)), [CTX] * B, d_ids.data_ptr(), d_logits=logits.data_ptr(),
                           d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), stream=s)
        torch.cuda.synchronize()
        got_l, got_h, got_n = host(logits), host(hid), host(nxt)
        L.loop_model_set_int4(g.handle, None)
        del keep
        Q32 = int4_decode_weights(W32, dims["n_layers"], np.float32)
        Q64 = int4_decode_weights(W32, dims["n_layers"], np.float64)
        for b in SAMPLE[1:]:
            say("int4 decode oracle seq", b)
            evals = []
            for W, dt in ((Q32, np.float32), (Q64, np.float64)):
                st = state_of(b, dt)
                lg, nx, h = om.decode_step(ocfg, W, [st], [int(ids[b])], bf16=True)
                evals.append((lg[0], h[0]))
            tol_l = parity_bar([e[0] for e in evals])
            tol_h = parity_bar([e[1] for e in evals])
            el, eh = rel_err(got_l[b], evals[0][0]), rel_err(got_h[b], evals[0][1])
            print("int4 decode seq %d: logits %.4f (bar %.4f), hidden %.4f (bar %.4f)" % (b, el, tol_l, eh, tol_h))
            assert el <= tol_l and eh <= tol_h, b
            assert argmax_ok(int(got_n[b]), [e[0] for e in evals], tol_l), b
    finally:
        g.close()
