"""The C-ABI boundary without a GPU: the library loads, exports every function
that include/loop.h declares, and its host-side size and schedule functions
give the figures the article fixes for the full model (KV bytes per token,
constant GDN state, 56 executions of which 14 full attention) and report
invalid configurations as errors.  No call here touches a device."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "loop.h")) as f:
        text = f.read()
    body = text[text.index('extern "C" {'):]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return sorted(set(re.findall(r"\b(loop_\w+)\s*\(", body)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for must in ("loop_model_create", "loop_model_destroy", "loop_prefill", "loop_decode_step", "loop_kv_bytes",
                 "loop_state_bytes", "loop_arena_bytes", "loop_workspace_bytes", "loop_schedule", "loop_last_error"):
        assert must in names
    assert len(names) >= 15


def test_library_exports_every_declared_function():
    import looped_hybrid_attention_amd as L
    lib = ctypes.CDLL(L.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared in include/loop.h but not exported: {missing}"


@pytest.fixture(scope="module")
def full_cfg():
    import looped_hybrid_attention_amd as L
    return L, L.make_config(synth.preset("full"), max_batch=1, max_seq=131072 + 64, max_tokens=8192)


def test_kv_bytes_per_token_and_long_context(full_cfg):
    # article section 4: 14 full-attention executions x K and V x 4 KV heads
    # x 256 dims x bf16 = 57,344 bytes per token; 7.5 GB (about 7.2 GiB) at
    # 131,072 tokens
    L, cfg = full_cfg
    assert L.loop_kv_bytes(cfg, 1, 1) == 57344
    assert L.loop_kv_bytes(cfg, 1, 131072) == 7_516_192_768
    assert L.loop_kv_bytes(cfg, 3, 1000) == 3 * 1000 * 57344


def test_gdn_state_is_constant(full_cfg):
    # 42 GDN executions x 16 heads x 128 x 128 fp32 = 42 MiB per sequence,
    # whatever the context length
    L, cfg = full_cfg
    assert L.loop_state_bytes(cfg, 1) == 42 * 1024 * 1024
    assert L.loop_arena_bytes(cfg) == L.loop_kv_bytes(cfg, 1, cfg.max_seq) + 42 * 1024 * 1024


def test_schedule_counts_host(full_cfg):
    L, cfg = full_cfg
    rows = L.loop_schedule(cfg)
    assert len(rows) == 56
    assert sum(r[1] for r in rows) == 14
    # the loop block's 24 weight layers run twice, the 4 + 4 outer ones once
    layers = [r[0] for r in rows]
    assert layers[:4] == [0, 1, 2, 3] and layers[-4:] == [28, 29, 30, 31]
    assert layers[4:28] == layers[28:52] == list(range(4, 28))


def test_cache_offsets_disjoint(full_cfg):
    L, cfg = full_cfg
    kv_one = 4 * cfg.max_seq * 256 * 2
    assert L.loop_cache_offset(cfg, 0, 0, 0) == 0
    assert L.loop_cache_offset(cfg, 1, 0, 0) == kv_one
    assert L.loop_cache_offset(cfg, 0, 1, 0) == 2 * kv_one
    assert L.loop_cache_offset(cfg, 2, 0, 0) == L.loop_kv_bytes(cfg, 1, cfg.max_seq)
    assert L.loop_cache_offset(cfg, 2, 41, 0) + 16 * 128 * 128 * 4 == L.loop_arena_bytes(cfg)


def test_invalid_configuration_is_an_error(full_cfg):
    L, cfg = full_cfg
    bad = L.make_config(synth.preset("full"), max_batch=1, max_seq=64, max_tokens=64)
    bad.head_dim = 0
    assert L.loop_kv_bytes(bad, 1, 10) == -1
    assert L.loop_state_bytes(bad, 1) == -1
    assert L.loop_arena_bytes(bad) == -1
    assert L.loop_kv_bytes(cfg, -1, 10) == -1
    assert L.loop_cache_offset(cfg, 3, 0, 0) == -1
    assert L.loop_cache_offset(cfg, 0, 0, 1) == -1  # sequence slot past max_batch
    with pytest.raises(Exception):
        L.loop_schedule(bad)
    assert L.loop_last_error()


# ------------------------------------------- loop_model_create's host checks
# loop_model_create validates its arguments on the host before it queries the
# device, so every rejection below is reached without a GPU.  The pointers
# are fake addresses: nothing is dereferenced on the host, and an invalid
# call enqueues nothing.

LOOP_EINVAL, LOOP_ESHAPE, LOOP_ECAPACITY, LOOP_EHIP, LOOP_EDEVICE = -1, -2, -3, -4, -5
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def _tiny_create_args(L):
    dims = synth.preset("tiny")
    cfg = L.make_config(dims, max_batch=2, max_seq=128, max_tokens=64)
    kinds = ["full" if l % 4 == 3 else "gdn" for l in range(dims["n_layers"])]
    from synth.presets import weight_specs
    ptrs = {name: FAKE + 4096 * i for i, (name, *_r) in enumerate(weight_specs(dims, kinds))}
    return cfg, ptrs


def _create(L, cfg, w, arena, ab, ws, wb, out=True):
    h = ctypes.c_void_p()
    code = L._lib.loop_model_create(ctypes.byref(cfg), ctypes.byref(w) if w is not None else None, arena, ab, ws,
                                    wb, ctypes.byref(h) if out else None)
    return code, L.loop_last_error()


def test_model_create_rejects_bad_arguments_on_host():
    import looped_hybrid_attention_amd as L
    cfg, ptrs = _tiny_create_args(L)
    ab, wb = L.loop_arena_bytes(cfg), L.loop_workspace_bytes(cfg, cfg.max_tokens)
    assert ab > 0 and wb > 0
    w = L.make_weights_struct(cfg.n_layers, ptrs)
    # no output handle
    assert _create(L, cfg, w, FAKE, ab, FAKE + (1 << 36), wb, out=False)[0] == LOOP_EINVAL
    # weights missing, a layer's matrix missing, mHC parameters missing
    code, msg = _create(L, cfg, None, FAKE, ab, FAKE + (1 << 36), wb)
    assert code == LOOP_EINVAL and "weights" in msg
    for drop, needle in (("L5.w_in", "layer 5"), ("L3.q_norm", "q_norm"), ("L0.o_norm", "o_norm"),
                         ("L6.mhc.mix", "mHC"), ("embed", "embed"), ("final_norm", "final_norm")):
        p = dict(ptrs)
        del p[drop]
        code, msg = _create(L, cfg, L.make_weights_struct(cfg.n_layers, p), FAKE, ab, FAKE + (1 << 36), wb)
        assert code == LOOP_EINVAL and needle in msg, (drop, msg)
    # n_layers mismatch
    w_short = L.make_weights_struct(cfg.n_layers - 4, ptrs)
    assert _create(L, cfg, w_short, FAKE, ab, FAKE + (1 << 36), wb)[0] == LOOP_EINVAL
    # arena / workspace too small or missing
    code, msg = _create(L, cfg, w, FAKE, ab - 1, FAKE + (1 << 36), wb)
    assert code == LOOP_ECAPACITY and "arena" in msg
    assert _create(L, cfg, w, 0, ab, FAKE + (1 << 36), wb)[0] == LOOP_ECAPACITY
    code, msg = _create(L, cfg, w, FAKE, ab, FAKE + (1 << 36), wb - 1)
    assert code == LOOP_ECAPACITY and "workspace" in msg
    assert _create(L, cfg, w, FAKE, ab, 0, wb)[0] == LOOP_ECAPACITY
    # misaligned buffers
    code, msg = _create(L, cfg, w, FAKE + 16, ab, FAKE + (1 << 36), wb)
    assert code == LOOP_EINVAL and "aligned" in msg
    assert _create(L, cfg, w, FAKE, ab, FAKE + (1 << 36) + 128, wb)[0] == LOOP_EINVAL
    # unsupported dimensions are a configuration error
    bad = L.make_config(dict(synth.preset("tiny"), head_dim=96), max_batch=2, max_seq=128, max_tokens=64)
    assert _create(L, bad, w, FAKE, ab, FAKE + (1 << 36), wb)[0] in (LOOP_EINVAL, LOOP_ESHAPE)


def test_model_create_valid_arguments_reach_the_device_query():
    """With every argument valid the only remaining check is the device: on a
    host without a gfx950 GPU the call fails with a HIP or device error (and
    creates nothing), never a crash."""
    import looped_hybrid_attention_amd as L
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: creation would succeed")
    cfg, ptrs = _tiny_create_args(L)
    ab, wb = L.loop_arena_bytes(cfg), L.loop_workspace_bytes(cfg, cfg.max_tokens)
    w = L.make_weights_struct(cfg.n_layers, ptrs)
    code, msg = _create(L, cfg, w, FAKE, ab, FAKE + (1 << 36), wb)
    assert code in (LOOP_EHIP, LOOP_EDEVICE), (code, msg)


def test_decode_graph_rejects_null_arguments_on_host():
    # the graph entry points check their handles before any HIP call
    import looped_hybrid_attention_amd as L
    lib = L._lib
    g = ctypes.c_void_p()
    assert lib.loop_decode_graph_create(None, None, 1, None) == -1  # LOOP_EINVAL
    assert lib.loop_decode_graph_create(None, None, 1, ctypes.byref(g)) == -1  # LOOP_EINVAL
    assert g.value is None
    assert lib.loop_decode_graph_launch(None, None) == -1  # LOOP_EINVAL
    out = (ctypes.c_int32 * 1)()
    assert lib.loop_decode_graph_positions(None, out) == -1  # LOOP_EINVAL
    lib.loop_decode_graph_destroy(None)  # a no-op
