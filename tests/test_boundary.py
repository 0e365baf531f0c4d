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
