"""Weight-only int4 decode (group-wise symmetric codes, groups of 128 k).

- The device quantizer against the oracle's definition: packed codes and
  group scales bit for bit (integers decided by floating point: both sides
  divide in fp32, correctly rounded), on ragged row counts with a zero
  group and a padded source stride.
- The tiny looped model from seeded caches (KV at context 256 and GDN
  states drawn on the device by the counter-based generator, regenerated
  on the host for the oracle), the int4 codes of every layer's four
  projections registered: 3 greedy decode steps (teacher-forced) against
  the oracle decoding with the dequantized codes
  (``oracle.quant.int4_decode_weights``: bf16 values of code x scale).
  Bars ``parity.bar`` per step over the oracle in fp32 and fp64.  The int4
  oracle is closer to the int4 run than the bf16 oracle is.  Registering
  int8 codes afterwards replaces the int4 ones (the next step matches the
  int8 oracle); turning int8 off returns to bf16.
- A ragged batch (29 sequences, so the tiles' clamped activation rows and
  guarded stores run) from seeded caches: one int4 step, one int8 step,
  sampled sequences against the oracle.
The real-width, split-K variants of the int4 projections are checked in the
batch-64 decode test at 32K context.
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from oracle.quant import (quantize_groups_int4, pack_int4, int4_decode_weights, int8_decode_weights,
                          PROJECTIONS)
from gpu_util import torch_cuda, dev, host, say, rel_err
from test_gpu_int8 import device_int8
from model_util import GpuModel
from parity import bar, argmax_ok

pytestmark = pytest.mark.gpu


def device_int4(torch, L, g, n_layers, stream):
    """Packed codes and group scales of every layer's projections, quantized
    on the device from the model's bf16 matrices: (pointer dicts, keep-alive)."""
    keep, layers = [], []
    for l in range(n_layers):
        d = {}
        for name in PROJECTIONS:
            w = g.dev[f"L{l}.{name}"]
            N, K = w.shape
            q = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
            sc = torch.empty((N, K // 128), dtype=torch.float32, device="cuda")
            L.loop_quantize_int4(w.data_ptr(), N, K, K, q.data_ptr(), sc.data_ptr(), stream)
            keep += [q, sc]
            short = {"w_in": "in", "w_o": "o", "w_gateup": "gateup", "w_down": "down"}[name]
            d["w_" + short], d["s_" + short] = q.data_ptr(), sc.data_ptr()
        layers.append(d)
    return layers, keep


@pytest.mark.parametrize("N,K,ld", [(300, 512, 512), (17, 1280, 1300), (5, 128, 128), (1, 4096, 4096)])
def test_quantize_int4_matches_oracle_bitwise(N, K, ld):
    torch = torch_cuda()
    import looped_hybrid_attention_amd as L
    w = synth.normal(synth.SEED_W, f"q4.{N}.{K}", (N, ld), 0.02, dtype="bf16")
    g0 = 128 if K > 128 else 0
    w[2 % N, g0:g0 + 128] = 0  # a zero group
    d_w = dev(w, torch)
    q = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((N, K // 128), dtype=torch.float32, device="cuda")
    L.loop_quantize_int4(d_w.data_ptr(), N, K, ld, q.data_ptr(), sc.data_ptr(),
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    q_ref, s_ref = quantize_groups_int4(synth.bf16_bits_to_f32(w)[:, :K])
    assert np.array_equal(q.cpu().numpy(), pack_int4(q_ref))
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_quantize_int4_rejects_bad_shapes():
    torch = torch_cuda()
    import looped_hybrid_attention_amd as L
    buf = torch.zeros(4096, dtype=torch.float32, device="cuda")
    p = buf.data_ptr()
    for N, K, ld in ((4, 100, 100), (0, 128, 128), (4, 256, 128)):
        with pytest.raises(L.LoopError):
            L.loop_quantize_int4(p, N, K, ld, p, p, 0)


def _synth_state(ocfg, dims, n_full, n_gdn, max_seq, ctx, dtype):
    """The oracle's state of sequence 0 from the counter streams the device
    caches were drawn from (K, V ~ N(0, 1) bf16, V stored in blocks of 32
    positions transposed; GDN states ~ N(0, 0.1) fp32)."""
    Hkv, D = dims["n_kv_heads"], dims["head_dim"]
    H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
    st = om.SeqState(ocfg, dtype)
    per = Hkv * max_seq * D
    for f in range(n_full):
        kb = synth.normal(synth.SEED_C, f"tiny.q4.k.{f}", (per,), 1.0, dtype="bf16")
        vb = synth.normal(synth.SEED_C, f"tiny.q4.v.{f}", (per,), 1.0, dtype="bf16")
        K = synth.bf16_bits_to_f32(kb).reshape(Hkv, max_seq, D)[:, :ctx]
        Vb = synth.bf16_bits_to_f32(vb).reshape(Hkv, max_seq // 32, D, 32)
        Vp = Vb.transpose(0, 1, 3, 2).reshape(Hkv, max_seq, D)[:, :ctx]
        st.kv[f].k = np.ascontiguousarray(K, dtype)
        st.kv[f].v = np.ascontiguousarray(Vp, dtype)
    for j in range(n_gdn):
        S = synth.normal(synth.SEED_C, f"tiny.q4.state.{j}", (H * Dv * Dk,), 0.1)
        st.S[j] = S.reshape(H, Dv, Dk).astype(dtype)
    st.length = ctx
    return st


def test_int4_decode_tiny():
    """Three decode steps of the tiny model from seeded caches (context 256)
    with the int4 codes registered, then one with int8 codes registered in
    their place, then one in bf16; each against the oracle from the same
    seeded state (fp32 and fp64)."""
    torch = torch_cuda()
    dims = synth.preset("tiny")
    max_seq, T = 512, 256
    g = GpuModel(torch, dims, max_batch=1, max_seq=max_seq, max_tokens=512)
    try:
        L, cfg, s = g.L, g.cfg, g.stream()
        V, d = dims["vocab"], dims["d_model"]
        rows = L.loop_schedule(cfg)
        n_full = sum(r[1] for r in rows)
        n_gdn = len(rows) - n_full
        Hkv, D = dims["n_kv_heads"], dims["head_dim"]
        H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
        for f in range(n_full):
            for which, name in ((0, f"tiny.q4.k.{f}"), (1, f"tiny.q4.v.{f}")):
                L.loop_synth_normal(g.arena.data_ptr() + L.loop_cache_offset(cfg, which, f, 0), Hkv * max_seq * D, 1,
                                    synth.SEED_C, synth.fnv1a32(name), 0, 1.0, 0.0, s)
        for j in range(n_gdn):
            L.loop_synth_normal(g.arena.data_ptr() + L.loop_cache_offset(cfg, 2, j, 0), H * Dv * Dk, 0,
                                synth.SEED_C, synth.fnv1a32(f"tiny.q4.state.{j}"), 0, 0.1, 0.0, s)
        ocfg = oracle.Config.from_dims(dims)
        W32 = om.to_dtype(g.host_weights, np.float32)
        W64 = om.to_dtype(g.host_weights, np.float64)
        nl = dims["n_layers"]
        Q = {np.float32: int4_decode_weights(W32, nl, np.float32), np.float64: int4_decode_weights(W32, nl, np.float64)}
        R = {np.float32: int8_decode_weights(W32, nl, np.float32), np.float64: int8_decode_weights(W32, nl, np.float64)}
        Wb = {np.float32: W32, np.float64: W64}
        sts = {dt: _synth_state(ocfg, dims, n_full, n_gdn, max_seq, T, dt) for dt in (np.float32, np.float64)}
        st_b = _synth_state(ocfg, dims, n_full, n_gdn, max_seq, T, np.float32)  # bf16 weights, for contrast
        layers, keep = device_int4(torch, L, g, nl, s)
        L.loop_model_set_int4(g.handle, layers)
        logits = torch.zeros((1, V), dtype=torch.float32, device="cuda")
        nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
        hid = torch.zeros((1, d), dtype=torch.float32, device="cuda")
        tok = int(synth.token_ids(synth.SEED_X, "tiny.q4.first", 1, V)[0])
        keep8 = None
        for step in range(5):
            mode = "int4" if step < 3 else ("int8" if step == 3 else "bf16")
            if step == 3:  # int8 codes replace the int4 ones
                layers8, keep8 = device_int8(torch, L, g, nl, s)
                L.loop_model_set_int8(g.handle, layers8)
            if step == 4:
                L.loop_model_set_int8(g.handle, None)
            say("tiny decode step", step, mode)
            d_tok = torch.tensor([tok], dtype=torch.int32, device="cuda")
            L.loop_decode_step(g.handle, 1, [0], [T + step], d_tok.data_ptr(), d_logits=logits.data_ptr(),
                               d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), stream=s)
            torch.cuda.synchronize()
            Wd = Q if mode == "int4" else (R if mode == "int8" else Wb)
            outs = [om.decode_step(ocfg, Wd[dt], [sts[dt]], [tok], bf16=True) for dt in (np.float32, np.float64)]
            o32 = outs[0]
            tol_l, tol_h = bar([o[0] for o in outs]), bar([o[2] for o in outs])
            el, eh = rel_err(host(logits), o32[0]), rel_err(host(hid), o32[2])
            msg = "%s decode %d: logits %.4f (bar %.4f), hidden %.4f (bar %.4f)" % (mode, step, el, tol_l, eh, tol_h)
            if mode == "int4":
                ob = om.decode_step(ocfg, W32, [st_b], [tok], bf16=True)
                eb = rel_err(host(logits), ob[0])
                msg += "; vs the bf16 oracle %.4f" % eb
            print(msg)
            assert el <= tol_l and eh <= tol_h, step
            assert argmax_ok(int(host(nxt)[0]), [o[0][0] for o in outs], tol_l), step
            if mode == "int4":
                assert el < eb, step
            tok = int(o32[1][0])
        del keep, keep8
    finally:
        g.close()


@pytest.mark.parametrize("B", [9, 29, 37])
def test_quantized_decode_ragged_batch(B):
    """B sequences (a ragged M for the weight-streaming tiles: 9, 29 and 37
    rows reach the one-, two- and four-tile activation variants, the last
    tile part-filled) of the tiny model from seeded caches, one decode step
    with int4 codes, then (GDN states regenerated, the appended position
    rewritten) one with int8 codes; sampled sequences (first, middle, last)
    against the oracle in fp32 and fp64."""
    torch = torch_cuda()
    dims = synth.preset("tiny")
    max_seq, T = 512, 200
    g = GpuModel(torch, dims, max_batch=B, max_seq=max_seq, max_tokens=512)
    try:
        L, cfg, s = g.L, g.cfg, g.stream()
        V, d = dims["vocab"], dims["d_model"]
        rows = L.loop_schedule(cfg)
        n_full = sum(r[1] for r in rows)
        n_gdn = len(rows) - n_full
        Hkv, D = dims["n_kv_heads"], dims["head_dim"]
        H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
        per, per_s = Hkv * max_seq * D, H * Dv * Dk
        for f in range(n_full):
            for which, name in ((0, f"rag.q.k.{f}"), (1, f"rag.q.v.{f}")):
                L.loop_synth_normal(g.arena.data_ptr() + L.loop_cache_offset(cfg, which, f, 0), B * per, 1,
                                    synth.SEED_C, synth.fnv1a32(name), 0, 1.0, 0.0, s)

        def fill_states():
            for j in range(n_gdn):
                L.loop_synth_normal(g.arena.data_ptr() + L.loop_cache_offset(cfg, 2, j, 0), B * per_s, 0,
                                    synth.SEED_C, synth.fnv1a32(f"rag.q.state.{j}"), 0, 0.1, 0.0, s)

        def state_of(b, dtype):
            st = om.SeqState(om_cfg, dtype)
            for f in range(n_full):
                kb = synth.normal(synth.SEED_C, f"rag.q.k.{f}", (per,), 1.0, dtype="bf16", start=b * per)
                vb = synth.normal(synth.SEED_C, f"rag.q.v.{f}", (per,), 1.0, dtype="bf16", start=b * per)
                K = synth.bf16_bits_to_f32(kb).reshape(Hkv, max_seq, D)[:, :T]
                Vb = synth.bf16_bits_to_f32(vb).reshape(Hkv, max_seq // 32, D, 32)
                st.kv[f].k = np.ascontiguousarray(K, dtype)
                st.kv[f].v = np.ascontiguousarray(Vb.transpose(0, 1, 3, 2).reshape(Hkv, max_seq, D)[:, :T], dtype)
            for j in range(n_gdn):
                S = synth.normal(synth.SEED_C, f"rag.q.state.{j}", (per_s,), 0.1, start=b * per_s)
                st.S[j] = S.reshape(H, Dv, Dk).astype(dtype)
            st.length = T
            return st

        om_cfg = oracle.Config.from_dims(dims)
        W32 = om.to_dtype(g.host_weights, np.float32)
        nl = dims["n_layers"]
        ids = synth.token_ids(synth.SEED_X, "rag.q.ids", B, V)
        d_ids = dev(ids, torch)
        logits = torch.zeros((B, V), dtype=torch.float32, device="cuda")
        hid = torch.zeros((B, d), dtype=torch.float32, device="cuda")
        nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
        for bits in (4, 8):
            fill_states()
            if bits == 4:
                layers, keep = device_int4(torch, L, g, nl, s)
                L.loop_model_set_int4(g.handle, layers)
                Wq = {dt: int4_decode_weights(W32, nl, dt) for dt in (np.float32, np.float64)}
            else:
                layers, keep = device_int8(torch, L, g, nl, s)
                L.loop_model_set_int8(g.handle, layers)
                Wq = {dt: int8_decode_weights(W32, nl, dt) for dt in (np.float32, np.float64)}
            say("ragged batch decode, int%d" % bits)
            L.loop_decode_step(g.handle, B, list(range(B)), [T] * B, d_ids.data_ptr(), d_logits=logits.data_ptr(),
                               d_next=nxt.data_ptr(), d_hidden_out=hid.data_ptr(), stream=s)
            torch.cuda.synchronize()
            got_l, got_h, got_n = host(logits), host(hid), host(nxt)
            L.loop_model_set_int4(g.handle, None)
            L.loop_model_set_int8(g.handle, None)
            del keep
            for b in (0, B // 2, B - 1):
                outs = []
                for dt in (np.float32, np.float64):
                    st = state_of(b, dt)
                    outs.append(om.decode_step(om_cfg, Wq[dt], [st], [int(ids[b])], bf16=True))
                tol_l, tol_h = bar([o[0][0] for o in outs]), bar([o[2][0] for o in outs])
                el, eh = rel_err(got_l[b], outs[0][0][0]), rel_err(got_h[b], outs[0][2][0])
                print("int%d ragged seq %d: logits %.4f (bar %.4f), hidden %.4f (bar %.4f)"
                      % (bits, b, el, tol_l, eh, tol_h))
                assert el <= tol_l and eh <= tol_h, (bits, b)
                assert argmax_ok(int(got_n[b]), [o[0][0] for o in outs], tol_l), (bits, b)
    finally:
        g.close()
