"""The two sequence mixers at real width on identical inputs, GPU against the
oracle at a flat 2e-2.

Inside a stack the mixers' inputs already differ between the GPU and the
oracle (every earlier rounding decision of the bf16 backbone), so a
whole-stack comparison can only be judged against the oracle's own noise.
Here the in-projection output is given -- the same bf16 values to both sides
-- and ``loop_exec_mixer`` runs one execution's mixer with its cache slot
exactly as the prefill runs it, so the comparison is well conditioned and the
bar is the flat one (metric max |gpu - oracle| / max |oracle| per tensor).

* Full attention ([P1] hncyxsy.com/news/268323 section 3: 16 Q / 4 KV heads x
  256, QK-norm, sigmoid output gate, rotary on 64 of 256 dims; section 4: the
  cache holds K and V): the gated output, and the K rows appended to the cache
  (post-norm, post-rotary) and V rows.
* Gated-DeltaNet ([P1] section 3: gate + delta rule with a constant-size state;
  16 heads x 128): the normed, gated output and the state left in the slot.

Each runs two sequences in two calls of 500 and 524 tokens (ragged chunks,
the second call at start position 500 on the cached prefix / the carried
state).  A third test runs full attention for 64 tokens at positions
262,080 .. 262,143 over a cache seeded with N(0, 1) bf16 K / V at positions
0 .. 262,079 in a sequence slot whose V block lies beyond 2^31 bytes of the
arena (rotary angles at the pages' trained length, 64-bit cache offsets).

Inputs: the projection is seeded N(0, 1.28) bf16 -- the spread of xn W_in^T
for a unit-RMS xn and N(0, 0.02) weights of depth 4096; norm gains N(1, 0.1).
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import attention as oa, gdn as og
from oracle import model as om
from gpu_util import torch_cuda, dev, host, say, rel_err
from model_util import GpuModel
from parity import FLAT

pytestmark = pytest.mark.gpu

PROJ_STD = 0.02 * 64.0


def _arena_view(g, off, n, dtype):
    t = g.arena[off:off + n * (2 if dtype == "bf16" else 4)]
    import torch
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float32)


def _k_rows(g, cfg, slot, seq, p0, p1, dims):
    """K of (kv slot, sequence slot) at positions p0 .. p1-1: [Hkv, p1-p0, D]."""
    Hkv, D, S = dims["n_kv_heads"], dims["head_dim"], cfg.max_seq
    off = g.L.loop_cache_offset(cfg, 0, slot, seq)
    K = host(_arena_view(g, off, Hkv * S * D, "bf16")).reshape(Hkv, S, D)
    return K[:, p0:p1]


def _v_rows(g, cfg, slot, seq, p0, p1, dims):
    """V of (kv slot, sequence slot) at positions p0 .. p1-1: [Hkv, p1-p0, D]
    (the cache holds blocks of 32 positions transposed)."""
    Hkv, D, S = dims["n_kv_heads"], dims["head_dim"], cfg.max_seq
    off = g.L.loop_cache_offset(cfg, 1, slot, seq)
    Vb = host(_arena_view(g, off, Hkv * S * D, "bf16")).reshape(Hkv, S // 32, D, 32)
    return Vb.transpose(0, 1, 3, 2).reshape(Hkv, S, D)[:, p0:p1]


@pytest.fixture(scope="module")
def group():
    torch = torch_cuda()
    dims = synth.preset("group")
    g = GpuModel(torch, dims, max_batch=2, max_seq=1024, max_tokens=2 * 524)
    yield torch, dims, g
    g.close()


SPLIT = (500, 524)


def _proj(name, T, n_in):
    return synth.normal(synth.SEED_X, name, (T, n_in), PROJ_STD, dtype="bf16")


def _run_gpu(torch, g, exec_index, width, projs, slots):
    """Both calls on the GPU; returns the outputs per call [B*T, width] (float32)."""
    outs, p0 = [], 0
    for i, T in enumerate(SPLIT):
        x = np.concatenate([p[p0:p0 + T] for p in projs])
        d_x = dev(x, torch)
        d_o = torch.zeros((len(projs) * T, width), dtype=torch.bfloat16, device="cuda")
        say("mixer exec", exec_index, "call", i, "tokens", T, "start", p0)
        g.L.loop_exec_mixer(g.handle, exec_index, len(projs), T, slots, [p0] * len(projs), d_x.data_ptr(),
                            x.shape[1], d_o.data_ptr(), width, stream=g.stream())
        torch.cuda.synchronize()
        outs.append(host(d_o))
        p0 += T
    return outs


def test_full_attention_mixer_real_width(group):
    torch, dims, g = group
    ocfg = oracle.Config.from_dims(dims)
    Hq, Hkv, D = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
    n_in, width = 2 * Hq * D + 2 * Hkv * D, Hq * D
    exec_index = 3                                   # the group's full-attention execution
    W32 = om.layer_weights(om.to_dtype(g.host_weights, np.float32), 3)
    W64 = om.layer_weights(om.to_dtype(g.host_weights, np.float64), 3)
    slots = [1, 0]
    projs = [synth.bf16_bits_to_f32(_proj(f"mixer.attn.proj.{b}", sum(SPLIT), n_in)) for b in range(2)]
    outs = _run_gpu(torch, g, exec_index, width, [synth.f32_to_bf16_bits(p) for p in projs], slots)
    for b in range(2):
        evals = []
        for w, dt in ((W32, np.float32), (W64, np.float64)):
            cache = oa.KVCache(Hkv, D, dt)
            o1 = oa.attention_mixer(projs[b][:SPLIT[0]].astype(dt), w, cache, 0, ocfg, bf16=True)
            o2 = oa.attention_mixer(projs[b][SPLIT[0]:].astype(dt), w, cache, SPLIT[0], ocfg, bf16=True)
            evals.append((o1, o2, cache))
        for i, T in enumerate(SPLIT):
            got = outs[i][b * T:(b + 1) * T]
            e, spread = rel_err(got, evals[0][i]), rel_err(evals[1][i], evals[0][i])
            print("attention mixer seq %d call %d: %.4f (oracle fp32/fp64 spread %.4f)" % (b, i, e, spread))
            assert e <= FLAT, (b, i)
        ek = rel_err(_k_rows(g, g.cfg, 0, slots[b], 0, sum(SPLIT), dims), evals[0][2].k)
        ev = rel_err(_v_rows(g, g.cfg, 0, slots[b], 0, sum(SPLIT), dims), evals[0][2].v)
        print("attention mixer seq %d: cached K %.5f, V %.5f" % (b, ek, ev))
        assert ek <= FLAT and ev == 0.0, b


def test_gdn_mixer_real_width(group):
    torch, dims, g = group
    ocfg = oracle.Config.from_dims(dims)
    H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
    n_in, width = 2 * H * Dk + 2 * H * Dv + 2 * H, H * Dv
    exec_index = 1                                   # a GDN execution (gdn slot 1)
    W32 = om.layer_weights(om.to_dtype(g.host_weights, np.float32), 1)
    W64 = om.layer_weights(om.to_dtype(g.host_weights, np.float64), 1)
    slots = [0, 1]
    projs = [synth.bf16_bits_to_f32(_proj(f"mixer.gdn.proj.{b}", sum(SPLIT), n_in)) for b in range(2)]
    outs = _run_gpu(torch, g, exec_index, width, [synth.f32_to_bf16_bits(p) for p in projs], slots)
    for b in range(2):
        evals = []
        for w, dt, ch in ((W32, np.float32, True), (W32, np.float32, False), (W64, np.float64, True)):
            S0 = np.zeros((H, Dv, Dk), dt)
            o1, S1 = og.gdn_mixer(projs[b][:SPLIT[0]].astype(dt), w, S0, ocfg, chunked=ch, bf16=True)
            o2, S2 = og.gdn_mixer(projs[b][SPLIT[0]:].astype(dt), w, S1, ocfg, chunked=ch, bf16=True)
            evals.append((o1, o2, S2))
        for i, T in enumerate(SPLIT):
            got = outs[i][b * T:(b + 1) * T]
            e = rel_err(got, evals[0][i])
            spread = max(rel_err(x[i], evals[0][i]) for x in evals[1:])
            print("GDN mixer seq %d call %d: %.4f (oracle spread %.4f)" % (b, i, e, spread))
            assert e <= FLAT, (b, i)
        off = g.L.loop_cache_offset(g.cfg, 2, 1, slots[b])
        S = host(_arena_view(g, off, H * Dv * Dk, "f32")).reshape(H, Dv, Dk)
        es = rel_err(S, evals[0][2])
        print("GDN mixer seq %d: final state %.2e" % (b, es))
        assert es <= 1e-3, b


def test_full_attention_mixer_at_262k():
    torch = torch_cuda()
    dims = synth.preset("group")
    ocfg = oracle.Config.from_dims(dims)
    Hq, Hkv, D = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
    n_in, width = 2 * Hq * D + 2 * Hkv * D, Hq * D
    CTX, T, SEQ = 262080, 64, 2
    g = GpuModel(torch, dims, max_batch=3, max_seq=CTX + T, max_tokens=T)
    try:
        cfg, s = g.cfg, g.stream()
        k_off = g.L.loop_cache_offset(cfg, 0, 0, SEQ)
        v_off = g.L.loop_cache_offset(cfg, 1, 0, SEQ)
        assert v_off > 2 ** 31            # 64-bit offsets into the arena
        per = Hkv * cfg.max_seq * D
        say("seed 262K caches")
        g.L.loop_synth_normal(g.arena.data_ptr() + k_off, per, 1, synth.SEED_C, synth.fnv1a32("mixer.long.k"),
                              0, 1.0, 0.0, s)
        g.L.loop_synth_normal(g.arena.data_ptr() + v_off, per, 1, synth.SEED_C, synth.fnv1a32("mixer.long.v"),
                              0, 1.0, 0.0, s)
        proj = _proj("mixer.long.proj", T, n_in)
        d_x = dev(proj, torch)
        d_o = torch.zeros((T, width), dtype=torch.bfloat16, device="cuda")
        say("mixer at positions", CTX, "..", CTX + T - 1)
        g.L.loop_exec_mixer(g.handle, 3, 1, T, [SEQ], [CTX], d_x.data_ptr(), n_in, d_o.data_ptr(), width, stream=s)
        torch.cuda.synchronize()
        got = host(d_o)
        got_k = _k_rows(g, cfg, 0, SEQ, CTX, CTX + T, dims)
        # the seeded prefix as the device wrote it, regenerated on the host
        K = synth.bf16_bits_to_f32(synth.normal(synth.SEED_C, "mixer.long.k", (per,), 1.0, dtype="bf16"))
        K = K.reshape(Hkv, cfg.max_seq, D)[:, :CTX]
        Vb = synth.bf16_bits_to_f32(synth.normal(synth.SEED_C, "mixer.long.v", (per,), 1.0, dtype="bf16"))
        V = Vb.reshape(Hkv, cfg.max_seq // 32, D, 32).transpose(0, 1, 3, 2).reshape(Hkv, cfg.max_seq, D)[:, :CTX]
        del Vb
        w = om.layer_weights(om.to_dtype(g.host_weights, np.float32), 3)
        cache = oa.KVCache(Hkv, D, np.float32)
        cache.k, cache.v = np.ascontiguousarray(K), np.ascontiguousarray(V)
        del K, V
        say("oracle at 262K")
        ref = oa.attention_mixer(synth.bf16_bits_to_f32(proj), w, cache, CTX, ocfg, bf16=True)
        e = rel_err(got, ref)
        ek = rel_err(got_k, cache.k[:, CTX:])
        print("attention mixer at 262,080: output %.4f, appended K %.5f" % (e, ek))
        assert e <= FLAT and ek <= FLAT
    finally:
        g.close()


@pytest.mark.parametrize("preset,T", [("tiny", 100), ("group", 300)])
def test_mixers_prefill_then_decode_path(preset, T):
    """Each mixer's prefill path on T tokens, then three steps of its decode
    path (split-key decode attention, the token-by-token Gated-DeltaNet
    recurrence) continuing the same cache slot, two sequences at a time,
    against the oracle at the flat bar."""
    torch = torch_cuda()
    dims = synth.preset(preset)
    ocfg = oracle.Config.from_dims(dims)
    g = GpuModel(torch, dims, max_batch=2, max_seq=512, max_tokens=2 * T)
    try:
        Hq, Hkv, D = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
        H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
        kinds = {3: ("full", 2 * Hq * D + 2 * Hkv * D, Hq * D), 0: ("gdn", 2 * H * Dk + 2 * H * Dv + 2 * H, H * Dv)}
        for ex, (kind, n_in, width) in kinds.items():
            layer = ex  # the group's and the tiny model's executions 0 and 3 run weight layers 0 and 3
            W32 = om.layer_weights(om.to_dtype(g.host_weights, np.float32), layer)
            projs = [synth.bf16_bits_to_f32(_proj(f"mixer.{preset}.{kind}.{b}", T + 3, n_in)) for b in range(2)]
            # GPU: prefill of T tokens, then three decode steps
            outs = []
            for i, (p0, n, dec) in enumerate(((0, T, False), (T, 1, True), (T + 1, 1, True), (T + 2, 1, True))):
                x = np.concatenate([p[p0:p0 + n] for p in projs])
                d_x = dev(synth.f32_to_bf16_bits(x), torch)
                d_o = torch.zeros((2 * n, width), dtype=torch.bfloat16, device="cuda")
                say(preset, kind, "mixer call", i, "decode" if dec else "prefill")
                g.L.loop_exec_mixer(g.handle, ex, 2, n, [0, 1], [p0, p0], d_x.data_ptr(), n_in, d_o.data_ptr(),
                                    width, decode=dec, stream=g.stream())
                torch.cuda.synchronize()
                outs.append(host(d_o).reshape(2, n, width))
            for b in range(2):
                if kind == "full":
                    cache = oa.KVCache(Hkv, D, np.float32)
                    refs = [oa.attention_mixer(projs[b][:T], W32, cache, 0, ocfg, bf16=True)]
                    refs += [oa.attention_mixer(projs[b][T + j:T + j + 1], W32, cache, T + j, ocfg, bf16=True)
                             for j in range(3)]
                else:
                    S = np.zeros((H, Dv, Dk), np.float32)
                    o, S = og.gdn_mixer(projs[b][:T], W32, S, ocfg, chunked=True, bf16=True)
                    refs = [o]
                    for j in range(3):
                        o, S = og.gdn_mixer(projs[b][T + j:T + j + 1], W32, S, ocfg, bf16=True)
                        refs.append(o)
                errs = [rel_err(outs[i][b], refs[i]) for i in range(4)]
                print("%s %s mixer seq %d: prefill %.4f, decode %s" % (preset, kind, b, errs[0],
                                                                       " ".join("%.4f" % e for e in errs[1:])))
                assert max(errs) <= FLAT, (kind, b)
    finally:
        g.close()


def test_gdn_mixer_long_call_equals_split_calls():
    """A long Gated-DeltaNet prefill call (4,100 tokens: 65 chunks, the last
    one ragged, the state carried through all of them inside one scan) must
    equal, bit for bit, the same tokens in calls of 1,024 + 1,024 + 1,024 +
    1,028 (the same chunk boundaries, the state handed from call to call
    through the cache slot), and the oracle at the flat bar ([P1]
    hncyxsy.com/news/268323 section 3: 16 heads x 128 at real width)."""
    torch = torch_cuda()
    dims = synth.preset("group")
    ocfg = oracle.Config.from_dims(dims)
    H, Dk, Dv = dims["gdn_heads"], dims["gdn_dk"], dims["gdn_dv"]
    n_in, width = 2 * H * Dk + 2 * H * Dv + 2 * H, H * Dv
    T, parts = 4100, (1024, 1024, 1024, 1028)
    g = GpuModel(torch, dims, max_batch=2, max_seq=4160, max_tokens=T)
    try:
        proj = _proj("mixer.gdn.long", T, n_in)
        d_x = dev(proj, torch)
        outs = []
        for slot, split in ((0, (T,)), (1, parts)):
            d_o = torch.zeros((T, width), dtype=torch.bfloat16, device="cuda")
            p0 = 0
            for n in split:
                say("gdn mixer slot", slot, "tokens", n, "start", p0)
                g.L.loop_exec_mixer(g.handle, 0, 1, n, [slot], [p0], d_x.data_ptr() + p0 * n_in * 2, n_in,
                                    d_o.data_ptr() + p0 * width * 2, width, stream=g.stream())
                p0 += n
            torch.cuda.synchronize()
            outs.append(host(d_o))
        assert np.array_equal(outs[0], outs[1]), "one long call differs from the split calls"
        S = [host(_arena_view(g, g.L.loop_cache_offset(g.cfg, 2, 0, s), H * Dv * Dk, "f32")) for s in (0, 1)]
        assert np.array_equal(S[0], S[1]), "final state differs"
        W32 = om.layer_weights(om.to_dtype(g.host_weights, np.float32), 0)
        say("oracle, 4100 tokens")
        ref, Sref = og.gdn_mixer(synth.bf16_bits_to_f32(proj), W32, np.zeros((H, Dv, Dk), np.float32), ocfg,
                                 chunked=True, bf16=True)
        e, es = rel_err(outs[0], ref), rel_err(S[0].reshape(H, Dv, Dk), Sref)
        print("GDN mixer, 4100 tokens in one call: output %.4f, final state %.2e" % (e, es))
        assert e <= FLAT and es <= 1e-3
    finally:
        g.close()


def test_full_attention_mixer_mixed_starts():
    """One prefill call of two sequences at different start positions (a
    fresh sequence at 0, and one continuing a 700-token cached prefix at
    700): every query tile of the call sees its own sequence's key range,
    causal mask and cache tail, at real width ([P1] hncyxsy.com/news/268323
    section 3), against the oracle at the flat bar."""
    torch = torch_cuda()
    dims = synth.preset("group")
    ocfg = oracle.Config.from_dims(dims)
    Hq, Hkv, D = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
    n_in, width = 2 * Hq * D + 2 * Hkv * D, Hq * D
    PRE, T = 700, 300
    g = GpuModel(torch, dims, max_batch=2, max_seq=1024, max_tokens=2 * PRE)
    try:
        W32 = om.layer_weights(om.to_dtype(g.host_weights, np.float32), 3)
        pre = _proj("mixer.attn.mixed.pre", PRE, n_in)
        new = [_proj(f"mixer.attn.mixed.{b}", T, n_in) for b in range(2)]
        d_pre = dev(pre, torch)
        d_po = torch.zeros((PRE, width), dtype=torch.bfloat16, device="cuda")
        say("mixer prefix", PRE, "tokens in slot 1")
        g.L.loop_exec_mixer(g.handle, 3, 1, PRE, [1], [0], d_pre.data_ptr(), n_in, d_po.data_ptr(), width,
                            stream=g.stream())
        d_x = dev(np.concatenate(new), torch)
        d_o = torch.zeros((2 * T, width), dtype=torch.bfloat16, device="cuda")
        say("mixer, two sequences at starts 0 and", PRE)
        g.L.loop_exec_mixer(g.handle, 3, 2, T, [0, 1], [0, PRE], d_x.data_ptr(), n_in, d_o.data_ptr(), width,
                            stream=g.stream())
        torch.cuda.synchronize()
        got = host(d_o).reshape(2, T, width)
        c0 = oa.KVCache(Hkv, D, np.float32)
        ref0 = oa.attention_mixer(synth.bf16_bits_to_f32(new[0]), W32, c0, 0, ocfg, bf16=True)
        c1 = oa.KVCache(Hkv, D, np.float32)
        oa.attention_mixer(synth.bf16_bits_to_f32(pre), W32, c1, 0, ocfg, bf16=True)
        ref1 = oa.attention_mixer(synth.bf16_bits_to_f32(new[1]), W32, c1, PRE, ocfg, bf16=True)
        e0, e1 = rel_err(got[0], ref0), rel_err(got[1], ref1)
        print("attention mixer, mixed starts: seq at 0 %.4f, seq at %d %.4f" % (e0, PRE, e1))
        assert e0 <= FLAT and e1 <= FLAT
    finally:
        g.close()
