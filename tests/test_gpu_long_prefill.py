"""Long-context prefill on the full stack at its real size: one sequence of
131,072 uniform token ids prefilled in 16 calls of 8192 (call c starts at
position 8192 c and attends to the cached keys of every earlier call; the
Gated-DeltaNet executions carry their states across calls).  Full-attention
KV grows to 57,344 bytes per token (7,516,192,768 bytes), the GDN state stays
42 MiB.

The oracle cannot run this length within a test, so these are properties that
hold at any size (the values themselves are pinned by the one-group, decode and
tiny-model tests, which share every kernel):
- the KV bytes the library sizes for the sequence equal the article's figure;
- every full-attention cache holds keys and values up to position 131,071 and
  nothing past it;
- logits and final hidden states are finite;
- tokens 8192 .. 16383 prefilled as part of this 16-call run and, in another
  sequence slot, as the last two of four calls of 4096 give bit-identical
  hidden states (per-row arithmetic does not depend on the call's length).
Then the pages' trained length, 262,144 tokens (32 calls of 8192, KV
15,032,385,536 bytes), with the same cache and finiteness checks, and a batch
of two sequences prefilled together in calls of 2 x 8192 up to 32,768 tokens,
each bit-identical to the same sequence prefilled alone.
"""
import numpy as np
import pytest

import synth
from gpu_util import torch_cuda, host, say
from model_util import device_full_weights

pytestmark = pytest.mark.gpu

T = 131072
T2 = 262144
CHUNK = 8192


@pytest.fixture(scope="module")
def long_model():
    torch = torch_cuda()
    import looped_hybrid_attention_amd as L
    dims = synth.preset("full")
    cfg = L.make_config(dims, max_batch=2, max_seq=T2 + 64, max_tokens=2 * CHUNK)
    sched = L.loop_schedule(cfg)
    kinds_layer = {layer: ("full" if full else "gdn") for layer, full, *_ in sched}
    kinds = [kinds_layer[l] for l in range(dims["n_layers"])]
    s = torch.cuda.current_stream().cuda_stream
    say("long prefill weights")
    tensors, wstruct = device_full_weights(torch, L, dims, kinds, s)
    ab, wb = L.loop_arena_bytes(cfg), L.loop_workspace_bytes(cfg, 2 * CHUNK)
    arena = torch.zeros(ab, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(wb, dtype=torch.uint8, device="cuda")
    handle = L.loop_model_create(cfg, wstruct, arena.data_ptr(), ab, ws.data_ptr(), wb)
    torch.cuda.synchronize()
    yield torch, L, dims, cfg, sched, handle, arena, s
    L.loop_model_destroy(handle)


def test_long_prefill_131072_in_8192_chunks(long_model):
    torch, L, dims, cfg, sched, handle, arena, s = long_model
    V, d, Hkv, D = dims["vocab"], dims["d_model"], dims["n_kv_heads"], dims["head_dim"]
    assert L.loop_kv_bytes(cfg, 1, T) == 7_516_192_768 == 57_344 * T
    assert L.loop_state_bytes(cfg, 1) == 42 * 1024 * 1024
    ids = torch.empty(T, dtype=torch.int32, device="cuda")
    L.loop_synth_token_ids(ids.data_ptr(), T, V, synth.SEED_X, synth.fnv1a32("test.long.ids"), s)
    logits = torch.zeros((1, V), dtype=torch.float32, device="cuda")
    h1 = torch.zeros((CHUNK, d), dtype=torch.float32, device="cuda")
    hl = torch.zeros((CHUNK, d), dtype=torch.float32, device="cuda")
    for c in range(T // CHUNK):
        say("long prefill call", c, "start", c * CHUNK)
        last = c == T // CHUNK - 1
        L.loop_prefill(handle, 1, CHUNK, [0], [c * CHUNK], d_tokens=ids[c * CHUNK:].data_ptr(),
                       d_logits=logits.data_ptr() if last else 0,
                       d_hidden_out=h1.data_ptr() if c == 1 else (hl.data_ptr() if last else 0), stream=s)
        torch.cuda.synchronize()
    assert np.isfinite(host(logits)).all() and np.isfinite(host(hl)).all() and np.isfinite(host(h1)).all()

    # caches: positions 0 .. T-1 written, nothing past them (the arena
    # started zeroed)
    n_full = sum(r[1] for r in sched)
    ms = cfg.max_seq
    for f in range(n_full):
        ko = L.loop_cache_offset(cfg, 0, f, 0)
        vo = L.loop_cache_offset(cfg, 1, f, 0)
        nb = Hkv * ms * D * 2
        k = arena[ko:ko + nb].view(torch.int16).view(Hkv, ms, D)
        v = arena[vo:vo + nb].view(torch.int16).view(Hkv, ms // 32, D, 32)
        for p in (0, T // 2, T - 1):
            assert bool((k[:, p] != 0).any()), (f, p)
            assert bool((v[:, p // 32, :, p % 32] != 0).any()), (f, p)
        assert not bool((k[:, T:] != 0).any()), f
        assert not bool((v[:, T // 32:] != 0).any()), f

    # tokens 8192 .. 16383 again, in slot 1, as the last two of four calls of 4096
    say("long prefill: slot 1, 4 x 4096")
    h2 = torch.zeros((CHUNK, d), dtype=torch.float32, device="cuda")
    for c in range(4):
        q = CHUNK // 2
        out = h2[(c - 2) * q:].data_ptr() if c >= 2 else 0
        L.loop_prefill(handle, 1, q, [1], [c * q], d_tokens=ids[c * q:].data_ptr(), d_hidden_out=out, stream=s)
    torch.cuda.synchronize()
    print("long prefill: 4096-call vs 8192-call hidden max |diff| %.3e" % float((h2 - h1).abs().max()))
    assert torch.equal(h2, h1)


def _check_caches(torch, L, cfg, sched, arena, dims, slot, n):
    """Full-attention caches of `slot` hold positions 0 .. n-1 and nothing past them."""
    Hkv, D, ms = dims["n_kv_heads"], dims["head_dim"], cfg.max_seq
    for f in range(sum(r[1] for r in sched)):
        ko = L.loop_cache_offset(cfg, 0, f, slot)
        vo = L.loop_cache_offset(cfg, 1, f, slot)
        nb = Hkv * ms * D * 2
        k = arena[ko:ko + nb].view(torch.int16).view(Hkv, ms, D)
        v = arena[vo:vo + nb].view(torch.int16).view(Hkv, ms // 32, D, 32)
        for p in (0, n // 2, n - 1):
            assert bool((k[:, p] != 0).any()), (f, p)
            assert bool((v[:, p // 32, :, p % 32] != 0).any()), (f, p)
        assert not bool((k[:, n:] != 0).any()), f
        assert not bool((v[:, n // 32:] != 0).any()), f


def test_long_prefill_262144(long_model):
    torch, L, dims, cfg, sched, handle, arena, s = long_model
    V = dims["vocab"]
    assert L.loop_kv_bytes(cfg, 1, T2) == 15_032_385_536 == 57_344 * T2
    arena.zero_()
    ids = torch.empty(T2, dtype=torch.int32, device="cuda")
    L.loop_synth_token_ids(ids.data_ptr(), T2, V, synth.SEED_X, synth.fnv1a32("test.long262k.ids"), s)
    logits = torch.zeros((1, V), dtype=torch.float32, device="cuda")
    for c in range(T2 // CHUNK):
        if c % 8 == 0:
            say("262K prefill call", c)
        last = c == T2 // CHUNK - 1
        L.loop_prefill(handle, 1, CHUNK, [0], [c * CHUNK], d_tokens=ids[c * CHUNK:].data_ptr(),
                       d_logits=logits.data_ptr() if last else 0, stream=s)
        torch.cuda.synchronize()
    assert np.isfinite(host(logits)).all()
    _check_caches(torch, L, cfg, sched, arena, dims, 0, T2)


def test_batched_long_prefill_equals_single(long_model):
    torch, L, dims, cfg, sched, handle, arena, s = long_model
    V, d = dims["vocab"], dims["d_model"]
    n = 32768
    arena.zero_()
    ids = torch.empty((2, n), dtype=torch.int32, device="cuda")
    for b in range(2):
        L.loop_synth_token_ids(ids[b].data_ptr(), n, V, synth.SEED_X, synth.fnv1a32(f"test.longbatch.{b}"), s)
    hb = torch.zeros((2 * CHUNK, d), dtype=torch.float32, device="cuda")
    lb = torch.zeros((2, V), dtype=torch.float32, device="cuda")
    say("batched long prefill: 2 x", n)
    for c in range(n // CHUNK):
        last = c == n // CHUNK - 1
        tok = torch.stack([ids[0, c * CHUNK:(c + 1) * CHUNK], ids[1, c * CHUNK:(c + 1) * CHUNK]]).contiguous()
        L.loop_prefill(handle, 2, CHUNK, [0, 1], [c * CHUNK, c * CHUNK], d_tokens=tok.data_ptr(),
                       d_logits=lb.data_ptr() if last else 0, d_hidden_out=hb.data_ptr() if last else 0, stream=s)
    torch.cuda.synchronize()
    # sequence 1 alone, into slot 0 (overwriting), calls of 8192
    h1 = torch.zeros((CHUNK, d), dtype=torch.float32, device="cuda")
    l1 = torch.zeros((1, V), dtype=torch.float32, device="cuda")
    for c in range(n // CHUNK):
        last = c == n // CHUNK - 1
        L.loop_prefill(handle, 1, CHUNK, [0], [c * CHUNK], d_tokens=ids[1, c * CHUNK:].data_ptr(),
                       d_logits=l1.data_ptr() if last else 0, d_hidden_out=h1.data_ptr() if last else 0, stream=s)
    torch.cuda.synchronize()
    print("batched vs single long prefill: hidden max |diff| %.3e" % float((hb[CHUNK:] - h1).abs().max()))
    assert torch.equal(hb[CHUNK:], h1) and torch.equal(lb[1:2], l1)
