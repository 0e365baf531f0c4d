#!/usr/bin/env python3
"""Throughput of the looped hybrid decoder's forward pass on one MI355X.

Headline: prefill tokens/s through the full 56-execution looped stack
(32 weight layers run 4 + 24x2 + 4; d 4096, FFN 12288, vocab 248,320;
bf16 weights N(0, 0.02) drawn on the device by the seeded generator), batch
1 x 8192 uniform token ids, logits at the last position.  One step = one
prefill call over the 8192 tokens (every kernel of the path).  Beside it:
decode tokens/s at batch 64 with 32,768-token contexts (caches pre-filled with
seeded N(0, 1) bf16 KV and N(0, 0.1) fp32 GDN states), one token per sequence
per step.

Prints one JSON line (see the repository's benchmark contract).  --gpus N
with N > 1 exits: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

LONG_T = 131072
VERIFY_K, VERIFY_STEPS = 4, 8
INT8_STEPS, INT8_WARMUP = 32, 2
GROUP_T = 4096
PREFILL_T = 8192
DECODE_B, DECODE_CTX = 64, 32768

# HBM bytes per launch of the roofline kernels, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes scaled by the same counters on a plain 1 GiB copy
# (--copy-calibration).  Each record carries the SHA-256 of the sources the
# kernel was built from; once they change the figure no longer applies and
# ``traffic`` is reported as null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "looped_hybrid_attention_amd", "csrc")
TRAFFIC_SOURCES = {
    "gemm_gateup": ["gemm.hip", "common.h"],
    "decode_attn": ["attention.hip", "common.h"],
}


def sources_sha256(key: str) -> str:
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[key]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key: str):
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)[key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256(key):
        return None
    return rec["hbm_bytes_per_launch"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5, help="timed prefill steps")
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--decode-steps", type=int, default=128)
    p.add_argument("--decode-warmup", type=int, default=3)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-prefill", action="store_true", help="decode only (for kernel profiles)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run one plain 1 GiB device-to-device copy (scale for HBM byte counters)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-long", action="store_true", help="skip the 131,072-token chunked prefill")
    p.add_argument("--long-tokens", type=int, default=LONG_T,
                   help="length of the chunked long prefill (a multiple of 8192; 262144 = the trained length)")
    p.add_argument("--no-verify", action="store_true", help="skip the multi-token verify step")
    p.add_argument("--no-int8", action="store_true", help="skip the weight-only int8 decode")
    p.add_argument("--no-int4", action="store_true", help="skip the weight-only int4 decode")
    p.add_argument("--no-b1", action="store_true", help="skip the batch-1 decode (bf16 / int8 / int4)")
    p.add_argument("--no-group", action="store_true",
                   help="skip the one-group real-width prefill (4 layers, 4096 hidden-state rows)")
    p.add_argument("--cpu-sample-tokens", type=int, default=8192)
    return p.parse_args()


# ------------------------------------------------------- algorithmic work

def layer_matrix_params(d, F, kind, Hq=16, Hkv=4, D=256, H=16, Dk=128, Dv=128):
    ffn = 3 * d * F
    if kind == "full":
        return ffn + (2 * Hq * D + 2 * Hkv * D) * d + d * Hq * D
    return ffn + (2 * H * Dk + 2 * H * Dv + 2 * H) * d + d * H * Dv


def layer_matrix_rows(d, F, kind, Hq=16, Hkv=4, D=256, H=16, Dk=128, Dv=128):
    """Output rows of a layer's four projection matrices (one scale each in int8)."""
    n_in = 2 * Hq * D + 2 * Hkv * D if kind == "full" else 2 * H * Dk + 2 * H * Dv + 2 * H
    return n_in + d + 2 * F + d


def prefill_flops(dims, kinds_exec, T):
    """GEMM 2*M*N*K + causal attention 4*Hq*D*sum(keys <= pos) + GDN
    6*H*Dk*Dv per token + head at the last position."""
    d, F = dims["d_model"], dims["d_ff"]
    gemm = sum(2 * T * layer_matrix_params(d, F, k) for k in kinds_exec)
    n_full = sum(k == "full" for k in kinds_exec)
    attn = n_full * 4 * dims["n_q_heads"] * dims["head_dim"] * (T * (T + 1) // 2)
    gdn = (len(kinds_exec) - n_full) * 6 * dims["gdn_heads"] * dims["gdn_dk"] * dims["gdn_dv"] * T
    head = 2 * d * dims["vocab"]
    return dict(gemm=gemm, attn=attn, gdn=gdn, head=head, total=gemm + attn + gdn + head)


def decode_bytes(dims, kinds_exec, B, L, int8=False, int4=False):
    """Per step: each executed layer's weights once (bf16; with int8, one
    byte per element plus a 4-byte scale per matrix row; with int4, half a
    byte per element plus a 4-byte scale per 128 elements), the LM head
    (bf16), all K/V read (L keys) + the appended K/V, GDN state read +
    write."""
    d, F = dims["d_model"], dims["d_ff"]
    if int4:
        weights = sum(layer_matrix_params(d, F, k) // 2 + 4 * (layer_matrix_params(d, F, k) // 128)
                      for k in kinds_exec)
    elif int8:
        weights = sum(layer_matrix_params(d, F, k) + 4 * layer_matrix_rows(d, F, k) for k in kinds_exec)
    else:
        weights = sum(2 * layer_matrix_params(d, F, k) for k in kinds_exec)
    weights += 2 * d * dims["vocab"]
    n_full = sum(k == "full" for k in kinds_exec)
    kv_tok = dims["n_kv_heads"] * dims["head_dim"] * 2 * 2
    kv = n_full * B * kv_tok * (L + 1)
    st = (len(kinds_exec) - n_full) * B * dims["gdn_heads"] * dims["gdn_dk"] * dims["gdn_dv"] * 4 * 2
    return dict(weights=weights, kv=kv, state=st, total=weights + kv + st)


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by sequence or by heads across GPUs; that is not implemented)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import looped_hybrid_attention_amd as L
    import synth
    from synth.presets import weight_specs

    dims = synth.preset("full")
    max_seq = ((DECODE_CTX + args.decode_warmup + args.decode_steps + 1 + VERIFY_K * (VERIFY_STEPS + 1)
                + 8 * (INT8_STEPS + INT8_WARMUP) + 63) // 64) * 64
    cfg = L.make_config(dims, max_batch=DECODE_B, max_seq=max_seq, max_tokens=PREFILL_T)
    sched = L.loop_schedule(cfg)
    kinds_layer = {}
    for layer, full, *_ in sched:
        kinds_layer[layer] = "full" if full else "gdn"
    kinds = [kinds_layer[l] for l in range(dims["n_layers"])]
    kinds_exec = ["full" if r[1] else "gdn" for r in sched]
    stream = torch.cuda.current_stream().cuda_stream

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # weights drawn on the device by the seeded generator (same stream names
    # and recipe as the host generator)
    t0 = time.time()
    tensors, ptrs = {}, {}
    for name, shape, dt, std, mean in weight_specs(dims, kinds):
        t = torch.empty(shape, dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda")
        L.loop_synth_normal(t.data_ptr(), t.numel(), 1 if dt == "bf16" else 0, synth.SEED_W,
                            synth.fnv1a32(name), 0, std, mean, stream)
        tensors[name] = t
        ptrs[name] = t.data_ptr()
    wstruct = L.make_weights_struct(dims["n_layers"], ptrs)
    arena_bytes = L.loop_arena_bytes(cfg)
    ws_bytes = L.loop_workspace_bytes(cfg, PREFILL_T)
    arena = torch.empty(arena_bytes, dtype=torch.uint8, device="cuda")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    model = L.loop_model_create(cfg, wstruct, arena.data_ptr(), arena_bytes, ws.data_ptr(), ws_bytes)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    # ------------------------------------------------------------ prefill
    ids = torch.empty(PREFILL_T, dtype=torch.int32, device="cuda")
    L.loop_synth_token_ids(ids.data_ptr(), PREFILL_T, dims["vocab"], synth.SEED_X,
                           synth.fnv1a32("bench.prefill.ids"), stream)
    logits = torch.empty((1, dims["vocab"]), dtype=torch.float32, device="cuda")

    def prefill_step():
        L.loop_prefill(model, 1, PREFILL_T, [0], [0], d_tokens=ids.data_ptr(), d_logits=logits.data_ptr(),
                       stream=stream)

    tok_s = ms_step = step_frac = roofline = fl = None
    if not args.no_prefill:
        for _ in range(args.warmup):
            prefill_step()
        torch.cuda.synchronize()
        L.loop_profile(model, L.LOOP_K["gemm_gateup"])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            prefill_step()
        e1.record()
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / args.steps
        k_ms, k_n = L.loop_profile_read(model)
        L.loop_profile(model, -1)
        assert torch.isfinite(logits).all().item(), "non-finite logits"
        fl = prefill_flops(dims, kinds_exec, PREFILL_T)
        tok_s = PREFILL_T / (ms_step / 1e3)
        k_avg_ms = k_ms / max(k_n, 1)
        k_flop = 2 * PREFILL_T * (2 * dims["d_ff"]) * dims["d_model"]
        k_tflops = k_flop / (k_avg_ms / 1e3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(k_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic("gemm_gateup"),
                    "kernel": "gemm_db_kernel<SWIGLU> (256x256 tiles, LDS-copy fed; gate/up projection + SwiGLU epilogue)",
                    "launch_ms": round(k_avg_ms, 4), "launches": k_n,
                    "algorithmic_flop_per_launch": k_flop}
        step_frac = fl["total"] / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS

    # ------------------------------------------- one group at real width
    # One shared 4-layer group (GDN, GDN, GDN, full attention) run once as a
    # loop block (fork, mHC, merge), prefill of 4096 N(0, 1) hidden-state
    # rows (no embedding or head); its weights are layers 4..7 of the full
    # model's (the first loop group, which carries the mHC parameters).
    group = None
    if not args.no_group:
        dims_g = synth.preset("group")
        cfg_g = L.make_config(dims_g, max_batch=1, max_seq=GROUP_T, max_tokens=GROUP_T)
        kinds_g = ["full" if r[1] else "gdn" for r in L.loop_schedule(cfg_g)]
        gptrs = {"final_norm": ptrs["final_norm"]}
        for l in range(dims_g["n_layers"]):
            for name, ptr in ptrs.items():
                if name.startswith(f"L{cfg.loop_start + l}."):
                    gptrs[f"L{l}." + name.split(".", 1)[1]] = ptr
        ws_g_struct = L.make_weights_struct(dims_g["n_layers"], gptrs)
        ab_g, wb_g = L.loop_arena_bytes(cfg_g), L.loop_workspace_bytes(cfg_g, GROUP_T)
        arena_g = torch.empty(ab_g, dtype=torch.uint8, device="cuda")
        wsp_g = torch.empty(wb_g, dtype=torch.uint8, device="cuda")
        model_g = L.loop_model_create(cfg_g, ws_g_struct, arena_g.data_ptr(), ab_g, wsp_g.data_ptr(), wb_g)
        xg = torch.empty((GROUP_T, dims_g["d_model"]), dtype=torch.float32, device="cuda")
        L.loop_synth_normal(xg.data_ptr(), xg.numel(), 0, synth.SEED_X, synth.fnv1a32("bench.group.x"), 0,
                            1.0, 0.0, stream)
        hg = torch.empty_like(xg)

        def group_step():
            L.loop_prefill(model_g, 1, GROUP_T, [0], [0], d_hidden_in=xg.data_ptr(), d_hidden_out=hg.data_ptr(),
                           stream=stream)

        for _ in range(args.warmup):
            group_step()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            group_step()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        assert torch.isfinite(hg).all().item(), "non-finite group output"
        flg = prefill_flops(dims_g, kinds_g, GROUP_T)
        group = {"metric": "prefill tok/s, one shared 4-layer group at real width", "unit": "tok/s",
                 "value": round(GROUP_T / (gms / 1e3), 1), "ms_per_step": round(gms, 3), "tokens": GROUP_T,
                 "steps": args.steps, "warmup": args.warmup,
                 "mfma_frac_step": round(flg["total"] / (gms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "algorithmic_flop_per_step": flg["total"]}
        L.loop_model_destroy(model_g)
        del arena_g, wsp_g, xg, hg

    # ------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        nf = sum(k == "full" for k in kinds_exec)
        ng = len(kinds_exec) - nf
        for s in range(nf):
            for which in (0, 1):
                off = L.loop_cache_offset(cfg, which, s, 0)
                n = DECODE_B * dims["n_kv_heads"] * max_seq * dims["head_dim"]
                L.loop_synth_normal(arena.data_ptr() + off, n, 1, synth.SEED_C,
                                    synth.fnv1a32(f"bench.kv{which}.{s}"), 0, 1.0, 0.0, stream)
        for s in range(ng):
            off = L.loop_cache_offset(cfg, 2, s, 0)
            n = DECODE_B * dims["gdn_heads"] * dims["gdn_dv"] * dims["gdn_dk"]
            L.loop_synth_normal(arena.data_ptr() + off, n, 0, synth.SEED_C,
                                synth.fnv1a32(f"bench.state.{s}"), 0, 0.1, 0.0, stream)
        tok = torch.empty(DECODE_B, dtype=torch.int32, device="cuda")
        L.loop_synth_token_ids(tok.data_ptr(), DECODE_B, dims["vocab"], synth.SEED_X,
                               synth.fnv1a32("bench.decode.ids"), stream)
        nxt = torch.empty(DECODE_B, dtype=torch.int32, device="cuda")
        slots = list(range(DECODE_B))
        pos = DECODE_CTX

        def decode_step(p):
            L.loop_decode_step(model, DECODE_B, slots, [p] * DECODE_B, tok.data_ptr(), d_next=nxt.data_ptr(),
                               stream=stream)
            tok.copy_(nxt)

        for _ in range(args.decode_warmup):
            decode_step(pos)
            pos += 1
        torch.cuda.synchronize()
        L.loop_profile(model, L.LOOP_K["decode_attn"])
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        p_start = pos
        for _ in range(args.decode_steps):
            decode_step(pos)
            pos += 1
        d1.record()
        torch.cuda.synchronize()
        dms = d0.elapsed_time(d1) / args.decode_steps
        a_ms, a_n = L.loop_profile_read(model)
        L.loop_profile(model, -1)
        L_mid = (p_start + pos) // 2
        by = decode_bytes(dims, kinds_exec, DECODE_B, L_mid)
        kv_launch = DECODE_B * dims["n_kv_heads"] * (L_mid + 1) * dims["head_dim"] * 2 * 2
        a_avg = a_ms / max(a_n, 1)
        a_gbs = kv_launch / (a_avg / 1e3) / 1e9
        decode = {"metric": "decode tok/s", "value": round(DECODE_B / (dms / 1e3), 1), "unit": "tok/s",
                  "ms_per_step": round(dms, 3), "steps": args.decode_steps, "warmup": args.decode_warmup,
                  "batch": DECODE_B, "context": DECODE_CTX,
                  "hbm_frac_step": round(by["total"] / (dms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                  "algorithmic_bytes_per_step": by["total"],
                  "roofline": {"bound": "hbm", "achieved": round(a_gbs, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(a_gbs / PEAK_HBM_GBS, 4),
                               "traffic": measured_traffic("decode_attn"),
                               "kernel": "decode_attn_kernel<256,4> + combine (split-L attention)",
                               "launch_ms": round(a_avg, 4), "launches": a_n,
                               "algorithmic_bytes_per_launch": kv_launch}}

        # weight-only int8 and int4 decode: codes of every layer's four
        # projections, quantized on the device, then the same decode batch
        # continues (INT8_STEPS timed steps each)
        def quant_layers(bits):
            """Codes and scales of every layer's four projections, quantized
            on the device: (pointer dicts, keep-alive list)."""
            q_keep, q_layers = [], []
            short = {"w_in": "in", "w_o": "o", "w_gateup": "gateup", "w_down": "down"}
            for l in range(dims["n_layers"]):
                dq = {}
                for nm in ("w_in", "w_o", "w_gateup", "w_down"):
                    w = tensors[f"L{l}.{nm}"]
                    N, K = w.shape
                    if bits == 8:
                        q = torch.empty((N, K), dtype=torch.int8, device="cuda")
                        sc = torch.empty(N, dtype=torch.float32, device="cuda")
                        L.loop_quantize_int8(w.data_ptr(), N, K, K, q.data_ptr(), sc.data_ptr(), stream)
                    else:
                        q = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
                        sc = torch.empty((N, K // 128), dtype=torch.float32, device="cuda")
                        L.loop_quantize_int4(w.data_ptr(), N, K, K, q.data_ptr(), sc.data_ptr(), stream)
                    q_keep += [q, sc]
                    dq["w_" + short[nm]], dq["s_" + short[nm]] = q.data_ptr(), sc.data_ptr()
                q_layers.append(dq)
            return q_layers, q_keep

        for bits in (8, 4):
            if (bits == 8 and args.no_int8) or (bits == 4 and args.no_int4):
                continue
            q_layers, q_keep = quant_layers(bits)
            set_q = L.loop_model_set_int8 if bits == 8 else L.loop_model_set_int4
            set_q(model, q_layers)
            for _ in range(INT8_WARMUP):
                decode_step(pos)
                pos += 1
            torch.cuda.synchronize()
            i0, i1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            i_start = pos
            i0.record()
            for _ in range(INT8_STEPS):
                decode_step(pos)
                pos += 1
            i1.record()
            torch.cuda.synchronize()
            set_q(model, None)
            del q_keep
            ims = i0.elapsed_time(i1) / INT8_STEPS
            byq = decode_bytes(dims, kinds_exec, DECODE_B, (i_start + pos) // 2, int8=bits == 8, int4=bits == 4)
            decode[f"int{bits}"] = {"metric": f"decode tok/s (weight-only int{bits} projections)",
                                    "value": round(DECODE_B / (ims / 1e3), 1), "unit": "tok/s",
                                    "ms_per_step": round(ims, 3), "steps": INT8_STEPS, "warmup": INT8_WARMUP,
                                    "hbm_frac_step": round(byq["total"] / (ims / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                                    "algorithmic_bytes_per_step": byq["total"],
                                    "weight_bytes_per_step": byq["weights"]}

        # multi-token verify: VERIFY_K drafted tokens per sequence checked in
        # one call (logits and greedy token at every position), continuing
        # the decode batch's caches
        if not args.no_verify:
            vt = torch.empty(DECODE_B * VERIFY_K, dtype=torch.int32, device="cuda")
            L.loop_synth_token_ids(vt.data_ptr(), vt.numel(), dims["vocab"], synth.SEED_X,
                                   synth.fnv1a32("bench.verify.ids"), stream)
            vlog = torch.empty((DECODE_B * VERIFY_K, dims["vocab"]), dtype=torch.float32, device="cuda")
            vnx = torch.empty(DECODE_B * VERIFY_K, dtype=torch.int32, device="cuda")

            def verify_step(p):
                L.loop_verify_step(model, DECODE_B, VERIFY_K, slots, [p] * DECODE_B, vt.data_ptr(),
                                   d_logits=vlog.data_ptr(), d_next=vnx.data_ptr(), stream=stream)

            verify_step(pos)  # warm-up
            pos += VERIFY_K
            v_ctx = pos
            torch.cuda.synchronize()
            v0, v1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            v0.record()
            for _ in range(VERIFY_STEPS):
                verify_step(pos)
                pos += VERIFY_K
            v1.record()
            torch.cuda.synchronize()
            vms = v0.elapsed_time(v1) / VERIFY_STEPS
            assert torch.isfinite(vlog).all().item(), "non-finite verify logits"
            decode["verify"] = {"metric": "verified tok/s", "value": round(DECODE_B * VERIFY_K / (vms / 1e3), 1),
                                "unit": "tok/s", "k": VERIFY_K, "batch": DECODE_B, "ms_per_step": round(vms, 3),
                                "steps": VERIFY_STEPS, "context": v_ctx}

        # batch-1 decode: sequence slot 0 alone, after the batch legs (its
        # caches continue from their last position), with the bf16 matrices,
        # then int8, then int4 codes (weights dominate the step); each timed
        # as eager calls and as launches of the captured decode graph (one
        # host call per token; the graph feeds its greedy token back itself)
        if not args.no_b1:
            tok1 = tok[:1].clone()
            nxt1 = torch.zeros(1, dtype=torch.int32, device="cuda")
            p1 = pos
            b1 = {"metric": "decode tok/s at batch 1 (decode graph; eager calls beside)", "unit": "tok/s",
                  "context": p1, "steps": INT8_STEPS, "warmup": INT8_WARMUP}
            for bits in (16, 8, 4):
                keep = None
                if bits == 8:
                    layers, keep = quant_layers(8)
                    L.loop_model_set_int8(model, layers)
                elif bits == 4:
                    layers, keep = quant_layers(4)
                    L.loop_model_set_int4(model, layers)
                for _ in range(INT8_WARMUP):
                    L.loop_decode_step(model, 1, [0], [p1], tok1.data_ptr(), d_next=nxt1.data_ptr(), stream=stream)
                    tok1.copy_(nxt1)
                    p1 += 1
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(INT8_STEPS):
                    L.loop_decode_step(model, 1, [0], [p1], tok1.data_ptr(), d_next=nxt1.data_ptr(), stream=stream)
                    tok1.copy_(nxt1)
                    p1 += 1
                e1.record()
                torch.cuda.synchronize()
                ms_e = e0.elapsed_time(e1) / INT8_STEPS
                graph = L.loop_decode_graph_create(model, 1, [0], [p1], tok1.data_ptr(), INT8_WARMUP + INT8_STEPS,
                                                   d_next=tok1.data_ptr())
                for _ in range(INT8_WARMUP):
                    L.loop_decode_graph_launch(graph, stream)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(INT8_STEPS):
                    L.loop_decode_graph_launch(graph, stream)
                e1.record()
                torch.cuda.synchronize()
                L.loop_decode_graph_destroy(graph)
                p1 += INT8_WARMUP + INT8_STEPS
                L.loop_model_set_int8(model, None)
                L.loop_model_set_int4(model, None)
                del keep
                ms1 = e0.elapsed_time(e1) / INT8_STEPS
                by1 = decode_bytes(dims, kinds_exec, 1, p1 - INT8_STEPS // 2, int8=bits == 8, int4=bits == 4)
                b1["bf16" if bits == 16 else f"int{bits}"] = {
                    "value": round(1e3 / ms1, 1), "ms_per_step": round(ms1, 3),
                    "hbm_frac_step": round(by1["total"] / (ms1 / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                    "algorithmic_bytes_per_step": by1["total"],
                    "eager": {"value": round(1e3 / ms_e, 1), "ms_per_step": round(ms_e, 3),
                              "hbm_frac_step": round(by1["total"] / (ms_e / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}}
            decode["b1"] = b1

    L.loop_model_destroy(model)

    # ------------------------------------------------------ long prefill
    # One sequence of 131,072 tokens in 16 calls of 8192 (call c at position
    # 8192 c): a model over the same weights with one 131,136-position slot.
    long = None
    if not args.no_long:
        del arena, ws
        torch.cuda.empty_cache()
        n_long = args.long_tokens
        assert n_long % PREFILL_T == 0 and n_long > 0, "--long-tokens must be a multiple of 8192"
        cfg_l = L.make_config(dims, max_batch=1, max_seq=n_long + 64, max_tokens=PREFILL_T)
        ab_l, wb_l = L.loop_arena_bytes(cfg_l), L.loop_workspace_bytes(cfg_l, PREFILL_T)
        arena_l = torch.empty(ab_l, dtype=torch.uint8, device="cuda")
        ws_l = torch.empty(wb_l, dtype=torch.uint8, device="cuda")
        model_l = L.loop_model_create(cfg_l, wstruct, arena_l.data_ptr(), ab_l, ws_l.data_ptr(), wb_l)
        ids_l = torch.empty(n_long, dtype=torch.int32, device="cuda")
        L.loop_synth_token_ids(ids_l.data_ptr(), n_long, dims["vocab"], synth.SEED_X,
                               synth.fnv1a32("bench.long.ids"), stream)

        def long_pass(n_calls):
            for c in range(n_calls):
                last = c == n_long // PREFILL_T - 1
                L.loop_prefill(model_l, 1, PREFILL_T, [0], [c * PREFILL_T], d_tokens=ids_l[c * PREFILL_T:].data_ptr(),
                               d_logits=logits.data_ptr() if last else 0, stream=stream)

        long_pass(2)  # warm-up: the first two calls
        torch.cuda.synchronize()
        l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        l0.record()
        long_pass(n_long // PREFILL_T)
        l1.record()
        torch.cuda.synchronize()
        lms = l0.elapsed_time(l1)
        assert torch.isfinite(logits).all().item(), "non-finite logits (long prefill)"
        fl_l = prefill_flops(dims, kinds_exec, n_long)
        long = {"metric": "long prefill tok/s", "value": round(n_long / (lms / 1e3), 1), "unit": "tok/s",
                "tokens": n_long, "calls": n_long // PREFILL_T, "tokens_per_call": PREFILL_T,
                "ms_total": round(lms, 1),
                "mfma_frac": round(fl_l["total"] / (lms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "algorithmic_flop": fl_l["total"],
                "kv_bytes": L.loop_kv_bytes(cfg_l, 1, n_long), "gdn_state_bytes": L.loop_state_bytes(cfg_l, 1)}
        L.loop_model_destroy(model_l)

    # --------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_sample_tokens)

    out = {
        "metric": "prefill tok/s through 56-exec looped stack + decode tok/s; % MFMA/HBM peak",
        "value": round(tok_s, 1) if tok_s else None,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3) if ms_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, uniform token ids)",
        "config": {"workload": "full_prefill_8192", "model": "looped hybrid decoder, 32 layers x 56 executions",
                   "global_batch": 1, "seq_len": PREFILL_T, "parallelism": "none (1 GPU)"},
        "mfma_frac_step": round(step_frac, 4) if step_frac else None,
        "algorithmic_flop_per_step": fl["total"] if fl else None,
        "roofline": roofline,
        "decode": decode,
        "group_prefill": group,
        "long_prefill": long,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(T: int):
    """The oracle (NumPy, fp32, as it stands) on the host cores: one 4-layer
    group at real width (3 GDN + 1 full-attention layers) over T tokens,
    scaled to the 56-execution stack (x 56/4 of the layer time)."""
    import numpy as np
    import oracle
    from oracle import model as om
    import synth
    from synth.presets import make_weights
    dims = synth.preset("group")
    cfg = oracle.Config.from_dims(dims)
    kinds = [oracle.layer_kind(cfg, l) for l in range(cfg.n_layers)]
    W = om.to_dtype(make_weights(dims, kinds), np.float32)
    x = synth.normal(synth.SEED_X, "bench.cpu.hidden", (1, T, dims["d_model"]), 1.0)
    t0 = time.time()
    om.prefill(cfg, W, [om.SeqState(cfg)], hidden=x, chunked_gdn=True)
    dt = time.time() - t0
    per_stack = dt * 56 / 4
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    return {"value": round(T / per_stack, 2), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle fp32 forward of one real-width 4-layer group (3 GDN + 1 full attention, "
                      f"mHC fork/merge) over {T} tokens took {dt:.2f} s; scaled by 56/4 executions",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
