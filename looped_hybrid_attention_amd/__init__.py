"""Python binding of the looped hybrid decoder's HIP library (gfx950).

Argument marshalling only: every function here has the name of the C entry
point it calls (see ``include/loop.h``) and passes plain pointers and sizes.
Device buffers are typically ``torch`` tensors on the GPU (their
``data_ptr()``), streams are ``torch.cuda.Stream``/``hipStream_t`` handles.
Importing the package loads ``_lib/libloop.so``; there is no fallback: if the
library is missing or fails to load, the import raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libloop.so")

LOOP_EPI_BF16, LOOP_EPI_F32, LOOP_EPI_F32_RES, LOOP_EPI_SWIGLU = 0, 1, 2, 3

_i32, _i64, _u32, _f32, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float, ctypes.c_double
_vp, _sz = ctypes.c_void_p, ctypes.c_size_t


class LoopError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class loop_config(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "n_layers", "loop_start", "loop_end", "loop_passes", "d_model", "d_ff", "vocab",
        "n_q_heads", "n_kv_heads", "head_dim", "rotary_dim", "gdn_heads", "gdn_dk", "gdn_dv",
        "n_streams", "sinkhorn_iters")] + [("rope_theta", _f32), ("eps", _f32)] + [
        (n, _i32) for n in ("max_batch", "max_seq", "max_tokens", "gdn_chunk")]


class loop_layer_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "attn_norm", "ffn_norm", "w_in", "w_o", "q_norm", "k_norm", "o_norm", "w_gateup",
        "w_down", "mhc_read_w", "mhc_read_b", "mhc_write_w", "mhc_write_b", "mhc_mix")]


class loop_weights(ctypes.Structure):
    _fields_ = [("embed", _vp), ("final_norm", _vp), ("head", _vp), ("n_layers", _i32),
                ("layers", ctypes.POINTER(loop_layer_weights))]


class loop_prefill_args(ctypes.Structure):
    _fields_ = [("batch", _i32), ("seq_len", _i32), ("slots", ctypes.POINTER(_i32)),
                ("start_pos", ctypes.POINTER(_i32)), ("d_tokens", _vp), ("d_hidden_in", _vp),
                ("d_logits", _vp), ("d_hidden_out", _vp), ("n_taps", _i32),
                ("tap_exec", ctypes.POINTER(_i32)), ("d_taps", _vp), ("loop_passes", _i32),
                ("taps_all_positions", _i32), ("d_final_out", _vp)]


class loop_decode_args(ctypes.Structure):
    _fields_ = [("batch", _i32), ("slots", ctypes.POINTER(_i32)), ("pos", ctypes.POINTER(_i32)),
                ("d_tokens", _vp), ("d_logits", _vp), ("d_next", _vp), ("d_hidden_out", _vp),
                ("loop_passes", _i32)]


class loop_verify_args(ctypes.Structure):
    _fields_ = [("batch", _i32), ("k", _i32), ("slots", ctypes.POINTER(_i32)), ("pos", ctypes.POINTER(_i32)),
                ("d_tokens", _vp), ("d_logits", _vp), ("d_next", _vp), ("d_hidden_out", _vp),
                ("n_taps", _i32), ("tap_exec", ctypes.POINTER(_i32)), ("d_taps", _vp), ("loop_passes", _i32)]


class loop_mixer_args(ctypes.Structure):
    _fields_ = [("exec", _i32), ("batch", _i32), ("seq_len", _i32), ("slots", ctypes.POINTER(_i32)),
                ("start_pos", ctypes.POINTER(_i32)), ("decode", _i32), ("d_proj", _vp), ("ld_proj", _i64),
                ("d_out", _vp), ("ld_out", _i64)]


LOOP_VERIFY_MAX = 16


class loop_q8_layer(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_in", "s_in", "w_o", "s_o", "w_gateup", "s_gateup", "w_down", "s_down")]


class loop_q4_layer(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_in", "s_in", "w_o", "s_o", "w_gateup", "s_gateup", "w_down", "s_down")]


def _load():
    # The library links the HIP runtime that PyTorch-ROCm loads; importing
    # torch first makes that runtime the process's only one.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "loop_kv_bytes": (_i64, [P(loop_config), _i32, _i64]),
        "loop_state_bytes": (_i64, [P(loop_config), _i32]),
        "loop_arena_bytes": (_i64, [P(loop_config)]),
        "loop_workspace_bytes": (_i64, [P(loop_config), _i32]),
        "loop_cache_offset": (_i64, [P(loop_config), _i32, _i32, _i32]),
        "loop_schedule": (_i32, [P(loop_config), P(_i32), _i32]),
        "loop_model_create": (ctypes.c_int, [P(loop_config), P(loop_weights), _vp, _sz, _vp, _sz,
                                             P(_vp)]),
        "loop_model_destroy": (None, [_vp]),
        "loop_prefill": (ctypes.c_int, [_vp, P(loop_prefill_args), _vp]),
        "loop_decode_step": (ctypes.c_int, [_vp, P(loop_decode_args), _vp]),
        "loop_decode_graph_create": (ctypes.c_int, [_vp, P(loop_decode_args), _i32, P(_vp)]),
        "loop_decode_graph_launch": (ctypes.c_int, [_vp, _vp]),
        "loop_decode_graph_positions": (ctypes.c_int, [_vp, P(_i32)]),
        "loop_decode_graph_destroy": (None, [_vp]),
        "loop_verify_step": (ctypes.c_int, [_vp, P(loop_verify_args), _vp]),
        "loop_exec_mixer": (ctypes.c_int, [_vp, P(loop_mixer_args), _vp]),
        "loop_model_set_int8": (ctypes.c_int, [_vp, _vp]),
        "loop_quantize_int8": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp]),
        "loop_model_set_int4": (ctypes.c_int, [_vp, _vp]),
        "loop_quantize_int4": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp]),
        "loop_debug_mhc": (ctypes.c_int, [_vp, _vp, _vp]),
        "loop_last_error": (ctypes.c_char_p, []),
        "loop_profile": (ctypes.c_int, [_vp, _i32]),
        "loop_profile_read": (ctypes.c_int, [_vp, P(_f64), P(_i64)]),
        "loop_op_gemm": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i32, _i32, _i32,
                                        _i32, _vp, _sz, _vp]),
        "loop_op_gemm_static": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i32, _i32, _i32,
                                               _i32, _vp]),
        "loop_op_gemm_quant": (ctypes.c_int, [_i32, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i32, _i32,
                                              _i32, _i32, _vp, _sz, _vp]),
        "loop_synth_normal": (ctypes.c_int, [_vp, _i64, _i32, _u32, _u32, _i64, _f64, _f64, _vp]),
        "loop_synth_token_ids": (ctypes.c_int, [_vp, _i64, _u32, _u32, _u32, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("loop_kv_bytes", "loop_state_bytes", "loop_arena_bytes", "loop_workspace_bytes",
            "loop_cache_offset", "loop_schedule", "loop_model_create", "loop_model_destroy",
            "loop_prefill", "loop_decode_step", "loop_decode_graph_create", "loop_decode_graph_launch",
            "loop_decode_graph_positions", "loop_decode_graph_destroy", "loop_verify_step", "loop_debug_mhc", "loop_last_error",
            "loop_model_set_int8", "loop_quantize_int8", "loop_model_set_int4", "loop_quantize_int4",
            "loop_profile", "loop_profile_read", "loop_op_gemm", "loop_synth_normal",
            "loop_synth_token_ids")
LOOP_K = dict(gemm_gateup=0, gemm_down=1, gemm_in=2, gemm_o=3, attn_prep=4, flash=5, gdn=6,
              decode_attn=7, rows=8, head=9)


def _check(code: int) -> None:
    if code != 0:
        raise LoopError(code, _lib.loop_last_error().decode())


def make_config(dims: dict, max_batch: int = 1, max_seq: int = 1, max_tokens: int = 1,
                gdn_chunk: int = 64) -> loop_config:
    c = loop_config()
    for name, _ in loop_config._fields_:
        if name in dims:
            setattr(c, name, dims[name])
    c.max_batch, c.max_seq, c.max_tokens, c.gdn_chunk = max_batch, max_seq, max_tokens, gdn_chunk
    return c


def loop_last_error() -> str:
    return _lib.loop_last_error().decode()


def loop_kv_bytes(cfg: loop_config, batch: int, seq_len: int) -> int:
    return _lib.loop_kv_bytes(ctypes.byref(cfg), batch, seq_len)


def loop_state_bytes(cfg: loop_config, batch: int) -> int:
    return _lib.loop_state_bytes(ctypes.byref(cfg), batch)


def loop_arena_bytes(cfg: loop_config) -> int:
    return _lib.loop_arena_bytes(ctypes.byref(cfg))


def loop_workspace_bytes(cfg: loop_config, max_tokens: int) -> int:
    return _lib.loop_workspace_bytes(ctypes.byref(cfg), max_tokens)


def loop_cache_offset(cfg: loop_config, which: int, slot: int, seq_slot: int) -> int:
    return _lib.loop_cache_offset(ctypes.byref(cfg), which, slot, seq_slot)


def loop_schedule(cfg: loop_config) -> list:
    n = _lib.loop_schedule(ctypes.byref(cfg), None, 0)
    if n < 0:
        _check(n)
    buf = (_i32 * (6 * n))()
    _check(0 if _lib.loop_schedule(ctypes.byref(cfg), buf, n) == n else -1)
    return [tuple(buf[6 * i:6 * i + 6]) for i in range(n)]


def loop_op_gemm(A: int, lda: int, B: int, ldb: int, C: int, ldc: int, R: int, M: int, N: int,
                 K: int, epi: int, stream: int = 0, ws: int = 0, ws_bytes: int = 0) -> None:
    _check(_lib.loop_op_gemm(A, lda, B, ldb, C, ldc, R or None, M, N, K, epi, ws or None, ws_bytes,
                             stream or None))


def loop_op_gemm_quant(bits: int, A: int, lda: int, Bq: int, ldq: int, scale: int, C: int, ldc: int, R: int,
                       M: int, N: int, K: int, epi: int, stream: int = 0, ws: int = 0, ws_bytes: int = 0) -> None:
    _check(_lib.loop_op_gemm_quant(bits, A, lda, Bq, ldq, scale, C, ldc, R or None, M, N, K, epi, ws or None,
                                   ws_bytes, stream or None))


LOOP_GEMM_STATIC_SCRATCH_BYTES = 32 << 20
LOOP_GEMM_STATIC_MAX_ROWS = 64


def loop_op_gemm_static(A: int, lda: int, B: int, ldb: int, C: int, ldc: int, R: int, M: int, N: int,
                        K: int, epi: int, stream: int = 0) -> None:
    _check(_lib.loop_op_gemm_static(A, lda, B, ldb, C, ldc, R or None, M, N, K, epi, stream or None))


def loop_synth_normal(dst: int, n: int, dtype: int, seed: int, key: int, start: int, std: float,
                      mean: float = 0.0, stream: int = 0) -> None:
    _check(_lib.loop_synth_normal(dst, n, dtype, seed, key, start, std, mean, stream or None))


def loop_synth_token_ids(dst: int, n: int, vocab: int, seed: int, key: int, stream: int = 0) -> None:
    _check(_lib.loop_synth_token_ids(dst, n, vocab, seed, key, stream or None))


# ------------------------------------------------------------ model calls

LAYER_FIELDS = ("attn_norm", "ffn_norm", "w_in", "w_o", "q_norm", "k_norm", "o_norm", "w_gateup",
                "w_down")
MHC_FIELDS = {"mhc.read_w": "mhc_read_w", "mhc.read_b": "mhc_read_b", "mhc.write_w": "mhc_write_w",
              "mhc.write_b": "mhc_write_b", "mhc.mix": "mhc_mix"}


def make_weights_struct(n_layers: int, ptr: dict):
    """loop_weights from a {tensor name: device pointer} dict with the names
    "embed", "head", "final_norm", "L{l}.<field>" (see include/loop.h)."""
    arr = (loop_layer_weights * n_layers)()
    for l in range(n_layers):
        for f in LAYER_FIELDS:
            setattr(arr[l], f, ptr.get(f"L{l}.{f}") or None)
        for k, f in MHC_FIELDS.items():
            setattr(arr[l], f, ptr.get(f"L{l}.{k}") or None)
    w = loop_weights()
    w.embed = ptr.get("embed") or None
    w.head = ptr.get("head") or None
    w.final_norm = ptr.get("final_norm") or None
    w.n_layers = n_layers
    w.layers = arr
    w._keep = arr
    return w


def loop_model_create(cfg: loop_config, weights: loop_weights, arena: int, arena_bytes: int,
                      workspace: int, ws_bytes: int) -> int:
    h = _vp()
    _check(_lib.loop_model_create(ctypes.byref(cfg), ctypes.byref(weights), arena, arena_bytes,
                                  workspace, ws_bytes, ctypes.byref(h)))
    return h.value


def loop_model_destroy(model: int) -> None:
    _lib.loop_model_destroy(model)


def _i32arr(xs):
    xs = [int(x) for x in xs]
    return (_i32 * max(len(xs), 1))(*xs)


def loop_prefill(model: int, batch: int, seq_len: int, slots, start_pos, d_tokens: int = 0,
                 d_hidden_in: int = 0, d_logits: int = 0, d_hidden_out: int = 0, tap_exec=(),
                 d_taps: int = 0, stream: int = 0, loop_passes: int = 0, taps_all_positions: bool = False,
                 d_final_out: int = 0) -> None:
    a = loop_prefill_args()
    a.d_final_out = d_final_out or None
    a.loop_passes = loop_passes
    a.taps_all_positions = 1 if taps_all_positions else 0
    a.batch, a.seq_len = batch, seq_len
    sl, sp, te = _i32arr(slots), _i32arr(start_pos), _i32arr(tap_exec)
    a.slots, a.start_pos = sl, sp
    a.d_tokens, a.d_hidden_in = d_tokens or None, d_hidden_in or None
    a.d_logits, a.d_hidden_out = d_logits or None, d_hidden_out or None
    a.n_taps = len(tap_exec)
    a.tap_exec = te if len(tap_exec) else None
    a.d_taps = d_taps or None
    _check(_lib.loop_prefill(model, ctypes.byref(a), stream or None))


def loop_exec_mixer(model: int, exec_index: int, batch: int, seq_len: int, slots, start_pos, d_proj: int,
                    ld_proj: int, d_out: int, ld_out: int, decode: bool = False, stream: int = 0) -> None:
    a = loop_mixer_args()
    a.exec, a.batch, a.seq_len, a.decode = exec_index, batch, seq_len, 1 if decode else 0
    sl, sp = _i32arr(slots), _i32arr(start_pos)
    a.slots, a.start_pos = sl, sp
    a.d_proj, a.ld_proj, a.d_out, a.ld_out = d_proj, ld_proj, d_out, ld_out
    _check(_lib.loop_exec_mixer(model, ctypes.byref(a), stream or None))


def loop_decode_step(model: int, batch: int, slots, pos, d_tokens: int, d_logits: int = 0,
                     d_next: int = 0, d_hidden_out: int = 0, stream: int = 0, loop_passes: int = 0) -> None:
    a = loop_decode_args()
    a.loop_passes = loop_passes
    a.batch = batch
    sl, ps = _i32arr(slots), _i32arr(pos)
    a.slots, a.pos = sl, ps
    a.d_tokens = d_tokens
    a.d_logits, a.d_next, a.d_hidden_out = d_logits or None, d_next or None, d_hidden_out or None
    _check(_lib.loop_decode_step(model, ctypes.byref(a), stream or None))


def loop_decode_graph_create(model: int, batch: int, slots, pos, d_tokens: int, max_steps: int,
                             d_logits: int = 0, d_next: int = 0, d_hidden_out: int = 0,
                             loop_passes: int = 0) -> int:
    """Capture the decode step of this batch into a graph; returns its handle."""
    a = loop_decode_args()
    a.loop_passes = loop_passes
    a.batch = batch
    sl, ps = _i32arr(slots), _i32arr(pos)
    a.slots, a.pos = sl, ps
    a.d_tokens = d_tokens
    a.d_logits, a.d_next, a.d_hidden_out = d_logits or None, d_next or None, d_hidden_out or None
    g = _vp()
    _check(_lib.loop_decode_graph_create(model, ctypes.byref(a), max_steps, ctypes.byref(g)))
    return g.value


def loop_decode_graph_launch(graph: int, stream: int = 0) -> None:
    _check(_lib.loop_decode_graph_launch(graph, stream or None))


def loop_decode_graph_positions(graph: int, batch: int) -> list:
    out = (_i32 * batch)()
    _check(_lib.loop_decode_graph_positions(graph, out))
    return list(out)


def loop_decode_graph_destroy(graph: int) -> None:
    _lib.loop_decode_graph_destroy(graph)


def loop_verify_step(model: int, batch: int, k: int, slots, pos, d_tokens: int, d_logits: int = 0,
                     d_next: int = 0, d_hidden_out: int = 0, tap_exec=(), d_taps: int = 0, stream: int = 0,
                     loop_passes: int = 0) -> None:
    a = loop_verify_args()
    a.batch, a.k, a.loop_passes = batch, k, loop_passes
    sl, ps, te = _i32arr(slots), _i32arr(pos), _i32arr(tap_exec)
    a.slots, a.pos = sl, ps
    a.d_tokens = d_tokens
    a.d_logits, a.d_next, a.d_hidden_out = d_logits or None, d_next or None, d_hidden_out or None
    a.n_taps = len(tap_exec)
    a.tap_exec = te if len(tap_exec) else None
    a.d_taps = d_taps or None
    _check(_lib.loop_verify_step(model, ctypes.byref(a), stream or None))


def loop_quantize_int8(d_w: int, N: int, K: int, ldw: int, d_q: int, d_scale: int, stream: int = 0) -> None:
    _check(_lib.loop_quantize_int8(d_w, N, K, ldw, d_q, d_scale, stream or None))


def loop_model_set_int8(model: int, layers) -> None:
    """layers: list (one per weight layer) of dicts of device pointers with the
    keys of loop_q8_layer, or None to turn int8 decode off."""
    if layers is None:
        _check(_lib.loop_model_set_int8(model, None))
        return
    arr = (loop_q8_layer * len(layers))()
    for i, d in enumerate(layers):
        for name, _ in loop_q8_layer._fields_:
            setattr(arr[i], name, d[name])
    _check(_lib.loop_model_set_int8(model, arr))


def loop_quantize_int4(d_w: int, N: int, K: int, ldw: int, d_q: int, d_scale: int, stream: int = 0) -> None:
    _check(_lib.loop_quantize_int4(d_w, N, K, ldw, d_q, d_scale, stream or None))


def loop_model_set_int4(model: int, layers) -> None:
    """layers: list (one per weight layer) of dicts of device pointers with the
    keys of loop_q4_layer, or None to turn int4 decode off."""
    if layers is None:
        _check(_lib.loop_model_set_int4(model, None))
        return
    arr = (loop_q4_layer * len(layers))()
    for i, d in enumerate(layers):
        for name, _ in loop_q4_layer._fields_:
            setattr(arr[i], name, d[name])
    _check(_lib.loop_model_set_int4(model, arr))


def loop_debug_mhc(model: int, d_out: int, stream: int = 0) -> None:
    _check(_lib.loop_debug_mhc(model, d_out, stream or None))


def loop_profile(model: int, kernel_class: int) -> None:
    _check(_lib.loop_profile(model, kernel_class))


def loop_profile_read(model: int):
    """(summed milliseconds, number of launches) of the selected class."""
    t, n = _f64(), _i64()
    _check(_lib.loop_profile_read(model, ctypes.byref(t), ctypes.byref(n)))
    return t.value, n.value
