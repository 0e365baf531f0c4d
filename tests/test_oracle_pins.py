"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print (tests/golden/pages_numbers.json, cited there), closed forms,
invariants, brute force on tiny inputs, or a textbook routine written
differently.  Several tests also plant a plausible mistake in a copy of an
oracle routine and check that the pin catches it.
"""
import math

import numpy as np
import pytest

import synth
from synth.presets import make_weights
import oracle
from oracle import accounting, attention, gdn, mhc, model, ops
from oracle.config import Config, schedule, layer_kind, exec_layers

F64 = np.float64


def cfg_of(name, **kw):
    return Config.from_dims(synth.preset(name), **kw)


def weights(cfg, dtype=np.float32, gain_std=0.1, bias_std=0.1, seed=0):
    dims = cfg.as_dict()
    kinds = [layer_kind(cfg, l) for l in range(cfg.n_layers)]
    return model.to_dtype(make_weights(dims, kinds, seed=seed, gain_std=gain_std,
                                       bias_std=bias_std), dtype)


# ----------------------------------------------------------------- schedule

def test_schedule_counts_full(golden):
    cfg = cfg_of("full")
    c = accounting.exec_counts(cfg)
    assert c["n_exec"] == golden["schedule"]["n_exec"] == 56
    assert c["n_full"] == golden["hybrid"]["n_full_exec"] == 14
    assert c["n_gdn"] == golden["hybrid"]["n_gdn_exec"] == 42
    lay = exec_layers(cfg)
    assert lay[:4] == [0, 1, 2, 3]
    assert lay[4:28] == list(range(4, 28)) and lay[28:52] == list(range(4, 28))
    assert lay[52:] == [28, 29, 30, 31]
    assert [layer_kind(cfg, l) for l in range(4)] == golden["hybrid"]["group"]


def test_schedule_toy_cfg(golden):
    t = golden["toy_cfg"]
    cfg = Config(n_layers=t["n_layers"], loop_start=t["loop_start"], loop_end=t["loop_end"],
                 loop_passes=t["loop_passes"], d_model=t["d_model"], d_ff=t["d_ff"],
                 vocab=t["vocab"], n_q_heads=t["n_heads"], n_kv_heads=t["n_heads"],
                 head_dim=64, rotary_dim=16, gdn_heads=4, gdn_dk=64, gdn_dv=64)
    assert len(schedule(cfg)) == t["exec_count"]


def test_schedule_three_passes(golden):
    cfg = cfg_of("full", loop_passes=3)
    assert len(schedule(cfg)) == golden["three_passes"]["arithmetic"] == 80


def test_schedule_tiny_and_slots():
    cfg = cfg_of("tiny")
    rows = schedule(cfg)
    assert len(rows) == 16
    assert sum(r.kind == "full" for r in rows) == 4
    full_slots = [r.slot for r in rows if r.kind == "full"]
    gdn_slots = [r.slot for r in rows if r.kind == "gdn"]
    assert full_slots == list(range(4)) and gdn_slots == list(range(12))
    assert [r.e for r in rows if r.fork] == [4] and [r.e for r in rows if r.merge] == [11]
    assert all(r.loop == (4 <= r.e <= 11) for r in rows)


def test_schedule_taps_meaning(golden):
    """Tap indices: 3 = last head execution, 27 = last execution of pass 1,
    51 = last execution of pass 2 (merge), 53/54 inside the tail."""
    cfg = cfg_of("full")
    rows = schedule(cfg)
    t = golden["taps"]["exec"]
    assert not rows[t[0]].loop and rows[t[0] + 1].fork
    assert rows[t[1]].layer == cfg.loop_end - 1 and rows[t[1] + 1].layer == cfg.loop_start
    assert rows[t[2]].merge
    assert not rows[t[3]].loop and not rows[t[4]].loop and rows[t[3]].layer >= cfg.loop_end


# --------------------------------------------------------------- accounting

def _sig(x, n):
    return float(f"{x:.{n}g}")


def test_param_accounting_recipe(golden):
    g = golden["params"]
    cfg = cfg_of("full")
    per = accounting.layer_params_recipe(cfg)
    assert _sig(per, g["per_layer_sig"]) == g["per_layer"]
    ex = accounting.executed_params(cfg, per)
    assert _sig(ex["stored"], 2) == g["stored_32_layers"]
    assert _sig(ex["head_tail"], 2) == g["head_tail_8_layers"]
    assert _sig(ex["loop"], 3) == g["loop_48_execs"]
    assert _sig(ex["embedding"], 3) == g["embedding"]
    # the pages multiply the rounded per-layer figure
    assert _sig(accounting.flops_per_token_estimate(56, g["per_layer"]), 3) == g["flops_per_token_56"]
    assert _sig(accounting.flops_per_token_estimate(32, g["per_layer"]), 3) == g["flops_per_token_32"]
    assert _sig(2 * 27e9, 2) == g["flops_per_token_27b"]


def test_param_accounting_exact():
    cfg = cfg_of("full")
    assert accounting.layer_params_exact(cfg, "full") - 2 * 4096 - 512 == 150994944 + 58720256
    assert accounting.layer_params_exact(cfg, "gdn") - 2 * 4096 - 128 == 150994944 + 42074112
    # 56 executions: 14 full + 42 GDN layers' matrices, 2 FLOP per weight
    assert accounting.gemm_flops_per_token_exact(cfg) == 2 * (14 * 209715200 + 42 * 193069056)


def test_kv_accounting(golden):
    k = golden["kv"]
    cfg = cfg_of("full")
    per = accounting.kv_bytes_per_token_per_exec(cfg)
    assert per == k["per_layer_per_token_KB"] * 1024
    assert accounting.kv_bytes(cfg, 1, 1) == k["per_token_KB"] * 1024 == 57344
    # the page converts with 1 KB = 1000 B, 128K = 128,000 tokens
    assert round(k["per_token_KB"] * 1000 * 128000 / 1e9, 1) == k["ctx_128k_GB"]
    assert abs(k["per_token_KB"] * 1000 * 256000 / 1e9 - k["ctx_256k_GB"]) / k["ctx_256k_GB"] < 0.01
    assert accounting.kv_bytes(cfg, 1, 131072) == 7516192768
    d = k["dense27b"]
    assert d["kv_heads"] * d["head_dim"] * 2 * 2 == d["per_layer_per_token_KB"] * 1024
    assert d["layers"] * d["per_layer_per_token_KB"] == d["per_token_KB"]
    assert round(d["per_token_KB"] * 1000 * 128000 / 1e9, 1) == d["ctx_128k_GB"]
    assert accounting.state_bytes(cfg, 1) == 42 * 2 ** 20
    assert accounting.kv_bytes(cfg_of("tiny"), 1, 1) == 4 * 1 * 64 * 2 * 2


# ----------------------------------------------------------------- row ops

def test_rmsnorm_textbook():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 33))
    g = rng.standard_normal(33)
    y = ops.rmsnorm(x, g, 1e-6)
    for i in range(5):
        rms = math.sqrt(sum(v * v for v in x[i]) / 33 + 1e-6)
        assert np.allclose(y[i], [x[i, j] / rms * g[j] for j in range(33)], rtol=1e-13)


def test_activations_textbook():
    x = np.linspace(-30, 30, 101)
    assert np.allclose(ops.softplus(x), [math.log1p(math.exp(v)) for v in x], rtol=1e-12)
    assert np.allclose(ops.silu(x), [v / (1 + math.exp(-v)) for v in x], rtol=1e-12)
    assert np.allclose(np.exp(-ops.softplus(x)), 1 / (1 + np.exp(x)), rtol=1e-12)


def test_swiglu_textbook():
    rng = np.random.default_rng(1)
    hn = rng.standard_normal((3, 8))
    wgu = rng.standard_normal((10, 8))
    wd = rng.standard_normal((8, 5))
    out = ops.swiglu_ffn(hn, wgu, wd)
    for t in range(3):
        act = []
        for j in range(5):
            gt = sum(hn[t, i] * wgu[j, i] for i in range(8))
            up = sum(hn[t, i] * wgu[5 + j, i] for i in range(8))
            act.append(gt / (1 + math.exp(-gt)) * up)
        ref = [sum(act[j] * wd[o, j] for j in range(5)) for o in range(8)]
        assert np.allclose(out[t], ref, rtol=1e-12)


# ------------------------------------------------------------------ rotary

def test_rope_adjacent_pairs_closed_form():
    """A unit vector on dim 2i rotates within the plane (2i, 2i+1) by
    pos * theta^(-2i/R); dims >= R are untouched."""
    D, R, theta = 16, 8, 10000.0
    for i in range(R // 2):
        x = np.zeros((1, 1, D))
        x[0, 0, 2 * i] = 1.0
        x[0, 0, R + 1] = 3.0
        pos = 7
        y = ops.apply_rope(x, np.array([pos]), R, theta)
        ang = pos * theta ** (-2.0 * i / R)
        exp = np.zeros(D)
        exp[2 * i], exp[2 * i + 1], exp[R + 1] = math.cos(ang), math.sin(ang), 3.0
        assert np.allclose(y[0, 0], exp, atol=1e-15)


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    def score(m, n):
        return float(ops.apply_rope(q, np.array([m]), 16, 1e4)[0, 0]
                     @ ops.apply_rope(k, np.array([n]), 16, 1e4)[0, 0])
    assert abs(score(10, 3) - score(1010, 1003)) < 1e-10
    assert abs(score(10, 3) - score(11, 3)) > 1e-6
    assert np.array_equal(ops.apply_rope(q, np.array([5]), 0, 1e4), q)


# --------------------------------------------------------------- attention

def _attention_bruteforce(q, K, V, qpos):
    T, Hq, D = q.shape
    Hkv, L, _ = K.shape
    out = np.zeros_like(q)
    for t in range(T):
        for j in range(Hq):
            kv = j * Hkv // Hq
            sc = [sum(q[t, j, d] * K[kv, n, d] for d in range(D)) / math.sqrt(D)
                  for n in range(L) if n <= qpos[t]]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            z = sum(e)
            for d in range(D):
                out[t, j, d] = sum(e[n] * V[kv, n, d] for n in range(len(e))) / z
    return out


def test_attention_bruteforce_gqa_causal():
    rng = np.random.default_rng(3)
    T, Hq, Hkv, D, L0 = 3, 4, 2, 5, 2
    q = rng.standard_normal((T, Hq, D))
    K = rng.standard_normal((Hkv, L0 + T, D))
    V = rng.standard_normal((Hkv, L0 + T, D))
    qpos = np.arange(L0, L0 + T)
    assert np.allclose(attention.attention_core(q, K, V, qpos),
                       _attention_bruteforce(q, K, V, qpos), rtol=1e-12)


def test_attention_single_key_and_gqa_repeat():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 4, 8))
    K = rng.standard_normal((1, 1, 8))
    V = rng.standard_normal((1, 1, 8))
    o = attention.attention_core(q, K, V, np.array([0]))
    assert np.allclose(o[0], np.repeat(V[:, 0], 4, axis=0))
    q = rng.standard_normal((5, 4, 8))
    K = rng.standard_normal((2, 5, 8))
    V = rng.standard_normal((2, 5, 8))
    a = attention.attention_core(q, K, V, np.arange(5))
    b = attention.attention_core(q, np.repeat(K, 2, axis=0), np.repeat(V, 2, axis=0), np.arange(5))
    assert np.allclose(a, b, rtol=1e-14)


# --------------------------------------------------------------------- GDN

def _gdn_inputs(T, H, Dk, Dv, seed=5, beta_zero=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, Dk))
    k = rng.standard_normal((T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, Dv))
    la = -np.log1p(np.exp(rng.standard_normal((T, H))))
    beta = 0 * la if beta_zero else 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((H, Dv, Dk)) * 0.3
    return q, k, v, la, beta, S0


def test_gdn_recurrent_bruteforce_literal():
    """The literal form alpha * S (I - beta k k^T) + beta v k^T with explicit
    matrices, token by token."""
    q, k, v, la, beta, S0 = _gdn_inputs(7, 2, 4, 3)
    o, S = gdn.gdn_recurrent(q, k, v, np.exp(la), beta, S0)
    for h in range(2):
        Sh = S0[h].copy()
        for t in range(7):
            I = np.eye(4)
            Sh = np.exp(la[t, h]) * Sh @ (I - beta[t, h] * np.outer(k[t, h], k[t, h])) \
                + beta[t, h] * np.outer(v[t, h], k[t, h])
            assert np.allclose(o[t, h], Sh @ q[t, h], rtol=1e-12, atol=1e-14)
        assert np.allclose(S[h], Sh, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("chunk,T", [(16, 64), (32, 70), (64, 130), (64, 5), (16, 1)])
def test_gdn_chunked_equals_recurrent_f64(chunk, T):
    q, k, v, la, beta, S0 = _gdn_inputs(T, 3, 8, 6)
    o1, S1 = gdn.gdn_recurrent(q, k, v, np.exp(la), beta, S0)
    o2, S2 = gdn.gdn_chunked(q, k, v, la, beta, S0, chunk)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 * max(1, np.abs(o1).max())
    assert np.max(np.abs(S1 - S2)) <= 1e-12 * max(1, np.abs(S1).max())


def test_gdn_chunked_equals_recurrent_f32():
    q, k, v, la, beta, S0 = (x.astype(np.float32) for x in _gdn_inputs(200, 2, 32, 32))
    o1, S1 = gdn.gdn_recurrent(q, k, v, np.exp(la), beta, S0)
    o2, S2 = gdn.gdn_chunked(q, k, v, la, beta, S0, 64)
    assert np.max(np.abs(o1 - o2)) / np.abs(o1).max() < 1e-5


def test_gdn_pure_decay():
    q, k, v, la, beta, S0 = _gdn_inputs(9, 2, 4, 3, beta_zero=True)
    o, S = gdn.gdn_recurrent(q, k, v, np.exp(la), beta, S0)
    cum = np.exp(np.cumsum(la, axis=0))
    for t in range(9):
        for h in range(2):
            assert np.allclose(o[t, h], cum[t, h] * S0[h] @ q[t, h], rtol=1e-12)
    assert np.allclose(S, cum[-1][:, None, None] * S0, rtol=1e-12)


def test_gdn_exact_retrieval():
    """alpha = 1, beta = 1, orthonormal keys: every written value is read back."""
    rng = np.random.default_rng(6)
    Dk, Dv, T = 8, 5, 6
    Q, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Q[:, :T].T[:, None, :]
    v = rng.standard_normal((T, 1, Dv))
    o, S = gdn.gdn_recurrent(k, k, v, np.ones((T, 1)), np.ones((T, 1)), np.zeros((1, Dv, Dk)))
    for i in range(T):
        assert np.allclose(S[0] @ k[i, 0], v[i, 0], atol=1e-12)
    assert np.allclose(o[:, 0], v[:, 0], atol=1e-12)


def test_gdn_layer_normalisation():
    cfg = cfg_of("tiny")
    W = weights(cfg, F64)
    lw = model.layer_weights(W, 0)
    rng = np.random.default_rng(7)
    xn = rng.standard_normal((5, cfg.d_model))
    a1, S1 = gdn.gdn_layer(xn, lw, np.zeros((4, 64, 64)), cfg)
    a2, S2 = gdn.gdn_layer(xn, lw, np.zeros((4, 64, 64)), cfg, chunked=True, chunk=2)
    assert np.allclose(a1, a2, rtol=1e-10, atol=1e-14) and np.allclose(S1, S2, atol=1e-14)
    # scaling the input scales q, k, v, z, a, b; with the L2 norms, o only via v, z
    assert a1.shape == (5, cfg.d_model)


# ---------------------------------------------------------------- Sinkhorn

def _sinkhorn_linear(L, iters, rows_first=True):
    """Sinkhorn-Knopp in the linear domain: alternate row and column
    normalisation of exp(L), then normalise rows."""
    A = np.exp(np.asarray(L, F64))
    for _ in range(iters):
        if rows_first:
            A = A / A.sum(1, keepdims=True)
            A = A / A.sum(0, keepdims=True)
        else:
            A = A / A.sum(0, keepdims=True)
            A = A / A.sum(1, keepdims=True)
    return A / A.sum(1, keepdims=True)


def test_sinkhorn_matches_linear_domain():
    rng = np.random.default_rng(8)
    for _ in range(50):
        L = rng.standard_normal((2, 2)) * 2
        assert np.allclose(mhc.sinkhorn(L, 20), _sinkhorn_linear(L, 20), rtol=1e-12)
    L3 = rng.standard_normal((3, 3)) * 2
    assert np.allclose(mhc.sinkhorn(L3, 7), _sinkhorn_linear(L3, 7), rtol=1e-12)
    # the order matters before convergence: columns-first differs
    L = np.array([[3.0, -2.0], [1.0, 2.5]])
    assert np.abs(_sinkhorn_linear(L, 1) - _sinkhorn_linear(L, 1, rows_first=False)).max() > 1e-3


def test_sinkhorn_closed_form_limit():
    """For 2x2 the limit is [[p, 1-p], [1-p, p]], p = sigmoid((L00+L11-L01-L10)/2)."""
    rng = np.random.default_rng(9)
    for _ in range(20):
        L = rng.standard_normal((2, 2))
        p = 1 / (1 + math.exp(-(L[0, 0] + L[1, 1] - L[0, 1] - L[1, 0]) / 2))
        assert np.allclose(mhc.sinkhorn(L, 400), [[p, 1 - p], [1 - p, p]], atol=1e-12)


def test_sinkhorn_doubly_stochastic_at_init_scale(golden):
    m = golden["mhc"]
    worst_r = worst_c = 0.0
    for i in range(500):
        L = synth.normal(0, f"mix{i}", (2, 2), m["mix_logit_std"])
        P = mhc.sinkhorn(L, m["iters"])
        worst_r = max(worst_r, np.abs(P.sum(1) - 1).max())
        worst_c = max(worst_c, np.abs(P.sum(0) - 1).max())
        assert np.isclose(np.linalg.norm(P.astype(F64), 2), 1.0, atol=1e-5)
    assert worst_r < 1e-6 and worst_c < 1e-5
    assert worst_c < m["sum_atol_printed"]


# --------------------------------------------------------------------- mHC

def test_mhc_write_orientation_rows_are_destinations():
    """Equal streams and a zero layer output stay equal to the fork value for any
    mix logits and any iteration count: the new stream s is sum_t P[s, t] s_t and
    the rows of P sum to one exactly (final row softmax); columns need not."""
    rng = np.random.default_rng(10)
    h = rng.standard_normal((3, 6))
    L = np.array([[2.0, -1.0], [0.5, 1.5]])
    P = mhc.sinkhorn(L, 0)
    assert np.abs(P.sum(0) - 1).max() > 0.1
    new = mhc.write([h, h.copy()], np.zeros_like(h), rng.standard_normal((2, 6)),
                    np.zeros(2), P)
    assert np.allclose(new[0], h, rtol=1e-14) and np.allclose(new[1], h, rtol=1e-14)


def test_mhc_total_conserved(golden):
    """Doubly stochastic mixing keeps the total of the streams; only the written
    output is added ([P1 section 5])."""
    rng = np.random.default_rng(11)
    s = [rng.standard_normal((4, 8)), rng.standard_normal((4, 8))]
    out = rng.standard_normal((4, 8))
    P = mhc.sinkhorn(np.array([[0.3, -0.7], [0.2, 0.9]]), golden["mhc"]["iters"])
    new = mhc.write(s, out, rng.standard_normal((2, 8)), rng.standard_normal(2), P)
    assert np.abs((new[0] + new[1]) - (s[0] + s[1]) - out).max() < 1e-5 * 10


def test_mhc_read_weights():
    rng = np.random.default_rng(12)
    s = [rng.standard_normal((3, 5)), rng.standard_normal((3, 5))]
    wr = rng.standard_normal((2, 10))
    br = rng.standard_normal(2)
    x, r = mhc.read(s, wr, br)
    for t in range(3):
        z = [sum(wr[j, i] * (s[0][t, i] if i < 5 else s[1][t, i - 5]) for i in range(10)) + br[j]
             for j in range(2)]
        e = [math.exp(v - max(z)) for v in z]
        rr = [v / sum(e) for v in e]
        assert np.allclose(r[t], rr, rtol=1e-13)
        assert np.allclose(x[t], rr[0] * s[0][t] + rr[1] * s[1][t], rtol=1e-13)


# ------------------------------------------------------------- whole model

@pytest.fixture(scope="module")
def tiny64():
    cfg = cfg_of("tiny")
    return cfg, weights(cfg, F64)


def _ids(n, vocab, name="ids"):
    return synth.token_ids(synth.SEED_X, name, n, vocab)


def test_looped_equals_unrolled_bitwise():
    cfg = cfg_of("tiny")
    W = weights(cfg, np.float32)
    ids = _ids(40, cfg.vocab).reshape(1, -1)
    h1, l1, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids)
    ucfg, UW = model.unrolled(cfg, W)
    assert len(schedule(ucfg)) == len(schedule(cfg)) and ucfg.loop_passes == 1
    h2, l2, _ = model.prefill(ucfg, UW, [model.SeqState(ucfg)], ids=ids)
    assert np.array_equal(h1, h2) and np.array_equal(l1, l2)


def test_weights_shared_between_passes(tiny64):
    """Perturbing a looped layer's weights changes both of its executions:
    the unrolled copy of only the second pass gives a different result."""
    cfg, W = tiny64
    ids = _ids(12, cfg.vocab).reshape(1, -1)
    ucfg, UW = model.unrolled(cfg, W)
    UW2 = dict(UW)
    UW2["L9.w_down"] = UW["L9.w_down"] * 1.5   # second-pass copy of layer 5
    ha, _, _ = model.prefill(ucfg, UW, [model.SeqState(ucfg)], ids=ids)
    hb, _, _ = model.prefill(ucfg, UW2, [model.SeqState(ucfg)], ids=ids)
    W2 = dict(W)
    W2["L5.w_down"] = W["L5.w_down"] * 1.5
    hc, _, _ = model.prefill(cfg, W2, [model.SeqState(cfg)], ids=ids)
    assert np.abs(hb - ha).max() > 1e-6 and np.abs(hc - hb).max() > 1e-6


def test_chunked_prefill_equals_whole(tiny64):
    cfg, W = tiny64
    ids = _ids(37, cfg.vocab).reshape(1, -1)
    h, lg, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids)
    st = [model.SeqState(cfg)]
    ha, _, _ = model.prefill(cfg, W, st, ids=ids[:, :20])
    hb, lb, _ = model.prefill(cfg, W, st, ids=ids[:, 20:])
    assert np.allclose(np.concatenate([ha, hb], 1), h, rtol=1e-10, atol=1e-12)
    assert np.allclose(lb, lg, rtol=1e-10, atol=1e-12)


def test_prefill_then_decode_equals_longer_prefill(tiny64):
    cfg, W = tiny64
    ids = _ids(9, cfg.vocab).reshape(1, -1)
    h, lg, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids)
    st = [model.SeqState(cfg)]
    model.prefill(cfg, W, st, ids=ids[:, :8])
    lg2, nxt, hd = model.decode_step(cfg, W, st, ids[:, 8])
    assert np.allclose(lg2, lg, rtol=1e-10, atol=1e-12)
    assert np.allclose(hd, h[:, -1], rtol=1e-10, atol=1e-12)
    assert nxt[0] == int(np.argmax(lg[0]))


def test_causal(tiny64):
    cfg, W = tiny64
    ids = _ids(10, cfg.vocab).reshape(1, -1)
    ids2 = ids.copy()
    ids2[0, 7] = (ids2[0, 7] + 1) % cfg.vocab
    h1, _, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids)
    h2, _, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids2)
    assert np.array_equal(h1[0, :7], h2[0, :7]) and np.abs(h1[0, 7:] - h2[0, 7:]).max() > 0


def test_single_stream_reduces_to_plain():
    """With one stream the mHC layer is a plain residual layer (reading R8)."""
    cfg = cfg_of("tiny", n_streams=1)
    W = weights(cfg, F64)
    ids = _ids(11, cfg.vocab).reshape(1, -1)
    h1, l1, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids)
    ucfg, UW = model.unrolled(cfg, W)
    pcfg = Config.from_dims(ucfg.as_dict(), loop_end=ucfg.loop_start)   # no loop: all plain
    assert not any(r.loop for r in schedule(pcfg))
    h2, l2, _ = model.prefill(pcfg, UW, [model.SeqState(pcfg)], ids=ids)
    assert np.allclose(h1, h2, rtol=1e-12, atol=1e-13) and np.allclose(l1, l2, rtol=1e-12)


def test_one_hot_routing_gives_independent_plain_stream():
    """Read only stream 0, write only stream 0, identity mixing: stream 0 runs
    the plain residual stack, stream 1 keeps the fork value; merge averages."""
    cfg = cfg_of("tiny")
    W = weights(cfg, F64)
    big = 60.0
    for l in range(cfg.loop_start, cfg.loop_end):
        p = f"L{l}."
        W[p + "mhc.read_w"] = np.zeros_like(W[p + "mhc.read_w"])
        W[p + "mhc.read_b"] = np.array([big, -big])
        W[p + "mhc.write_w"] = np.zeros_like(W[p + "mhc.write_w"])
        W[p + "mhc.write_b"] = np.array([big, -big])
        W[p + "mhc.mix"] = np.array([[big, -big], [-big, big]])
    ids = _ids(6, cfg.vocab).reshape(1, -1)
    _, _, taps = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids, taps=(3, 11))
    ucfg, UW = model.unrolled(cfg, W)
    pcfg = Config.from_dims(ucfg.as_dict(), loop_end=ucfg.loop_start)
    _, _, ptaps = model.prefill(pcfg, UW, [model.SeqState(pcfg)], ids=ids, taps=(3, 11))
    # merge = (plain result + fork value) / 2
    assert np.allclose(taps[11], (ptaps[11] + ptaps[3]) / 2, rtol=1e-10, atol=1e-12)


def test_toy_literal_write_grows_streams():
    """The reproduction writes the whole block output x + a + f back into the
    streams; summed over streams it then grows by about the layer input each
    layer, which is what the residual-branch reading avoids."""
    cfg = cfg_of("tiny")
    W = weights(cfg, F64, bias_std=0.0, gain_std=0.0)
    ids = _ids(6, cfg.vocab).reshape(1, -1)
    h1, _, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids)
    h2, _, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids, write_full=True)
    assert np.linalg.norm(h2) > 5 * np.linalg.norm(h1)


def test_gdn_chunked_model_equals_recurrent(tiny64):
    cfg, W = tiny64
    ids = _ids(70, cfg.vocab).reshape(1, -1)
    h1, l1, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids)
    h2, l2, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids, chunked_gdn=True)
    assert np.allclose(h1, h2, rtol=1e-10, atol=1e-12) and np.allclose(l1, l2, rtol=1e-10)


def test_batch_independent(tiny64):
    cfg, W = tiny64
    ids = _ids(16, cfg.vocab).reshape(2, 8)
    h, lg, _ = model.prefill(cfg, W, [model.SeqState(cfg), model.SeqState(cfg)], ids=ids)
    h1, l1, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids[1:])
    assert np.array_equal(h[1], h1[0]) and np.array_equal(lg[1], l1[0])


# ----------------------------------------------- planted mistakes are caught

def test_planted_mistake_sinkhorn_axis_caught(monkeypatch):
    def wrong(logits, iters):
        m = np.array(logits, copy=True)
        for _ in range(iters):
            m = m - ops.logsumexp(m, axis=0)
            m = m - ops.logsumexp(m, axis=1)
        return ops.softmax(m, axis=1)
    L = np.array([[3.0, -2.0], [1.0, 2.5]])
    assert np.abs(wrong(L, 1) - _sinkhorn_linear(L, 1)).max() > 1e-3


def test_planted_mistake_gdn_missing_gate_caught():
    q, k, v, la, beta, S0 = _gdn_inputs(40, 2, 8, 6)
    o1, _ = gdn.gdn_recurrent(q, k, v, np.exp(la), beta, S0)
    o2, _ = gdn.gdn_chunked(q, k, v, 0 * la, beta, S0, 16)   # gate dropped in one form
    assert np.abs(o1 - o2).max() > 1e-3


# ------------------------------------------------------ precision policy

def test_round_bf16_matches_library_cast():
    """round_bf16 against torch's float32 -> bfloat16 conversion (round to
    nearest even), including exact ties."""
    import torch
    from oracle.precision import round_bf16
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 10000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16(x), ref)
    assert round_bf16(np.float32(1.0 + 2 ** -8)) == 1.0            # tie -> even
    assert round_bf16(np.float32(1.0 + 3 * 2 ** -8)) == 1.0 + 2 ** -6  # tie -> even (up)


def test_bf16_policy_is_a_perturbation_of_the_definition():
    """The bf16 policy rounds stored tensors only: at one token through the
    first execution it moves the result by about the bf16 unit roundoff
    (2^-9 relative), and with rounding disabled it is the fp32 definition."""
    cfg = cfg_of("tiny")
    W = weights(cfg, np.float32)
    ids = _ids(1, cfg.vocab).reshape(1, -1)
    _, _, t32 = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids, taps=(0,))
    _, _, t16 = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids, taps=(0,), bf16=True)
    r = np.abs(t16[0] - t32[0]).max() / np.abs(t32[0]).max()
    assert 2 ** -12 < r < 2 ** -6
    h1, l1, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids)
    h2, l2, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids, bf16=False)
    assert np.array_equal(h1, h2) and np.array_equal(l1, l2)


def test_bf16_policy_keeps_structural_invariants():
    """Looped = unrolled bit for bit, and chunked prefill = whole prefill,
    hold in the bf16 policy too (rounding acts on the same tensors)."""
    cfg = cfg_of("tiny")
    W = weights(cfg, np.float32)
    ids = _ids(24, cfg.vocab).reshape(1, -1)
    h1, l1, _ = model.prefill(cfg, W, [model.SeqState(cfg)], ids=ids, bf16=True)
    ucfg, UW = model.unrolled(cfg, W)
    h2, l2, _ = model.prefill(ucfg, UW, [model.SeqState(ucfg)], ids=ids, bf16=True)
    assert np.array_equal(h1, h2) and np.array_equal(l1, l2)


# ----------------------------------------------------------- int8 decode weights

def test_int8_codes_definition():
    """Per-row symmetric int8: the largest magnitude of every row maps to
    +-127 exactly, every code is the nearest integer to w / s (ties to even),
    dequantization is within s / 2 of w, a zero row stays zero."""
    from oracle.quant import quantize_rows_int8, dequantize_rows
    rng = np.random.default_rng(7)
    w = rng.normal(0, 0.02, (37, 300)).astype(np.float32)
    w[5] = 0.0
    w[6, 17] = -0.5          # a row whose extreme is negative
    q, s = quantize_rows_int8(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert s[5] == 0 and not q[5].any()
    assert q[6, 17] == -127
    for n in range(w.shape[0]):
        if s[n] == 0:
            continue
        assert np.abs(q[n]).max() == 127
        assert s[n] == np.float32(np.abs(w[n]).max()) / np.float32(127)
    err = np.abs(dequantize_rows(q, s) - w)
    assert np.all(err <= s[:, None] * 0.5 * (1 + 1e-6))
    # values on the grid come back exactly; a half-way value rounds to even
    g = np.array([[127.0, 3.0, -2.5, 2.5, 1.5]], dtype=np.float32) * np.float32(0.25)
    qg, sg = quantize_rows_int8(g)
    assert sg[0] == np.float32(0.25) and list(qg[0]) == [127, 3, -2, 2, 2]


def test_int8_decode_weights_only_projections(tiny64):
    from oracle.quant import int8_decode_weights, PROJECTIONS
    cfg, W = tiny64[0], tiny64[1]
    Wq = int8_decode_weights(W, cfg.n_layers)
    for k, v in W.items():
        name = k.split(".", 1)[-1]
        if k.startswith("L") and name in PROJECTIONS:
            assert not np.array_equal(Wq[k], v) and np.abs(Wq[k] - v).max() <= np.abs(v).max() / 254 * 1.0001
        else:
            assert Wq[k] is v


# ----------------------------------------------------------- int4 decode weights

def test_int4_codes_definition():
    """Group-wise symmetric int4 (groups of 128 k): the largest magnitude of
    every group maps to +-7 exactly, codes are the nearest integers to
    w / s (ties to even), the bf16 dequantization is within s / 2 plus one
    bf16 rounding of w, and a zero group stays zero."""
    from oracle.quant import quantize_groups_int4, dequantize_groups_int4
    rng = np.random.default_rng(11)
    w = rng.normal(0, 0.02, (9, 384)).astype(np.float32)
    w[2, 128:256] = 0.0         # one zero group
    w[4, 300] = -0.5            # a group whose extreme is negative
    q, s = quantize_groups_int4(w)
    assert q.dtype == np.int8 and s.dtype == np.float32 and s.shape == (9, 3)
    assert s[2, 1] == 0 and not q[2, 128:256].any()
    assert q[4, 300] == -7
    for n in range(9):
        for g in range(3):
            blk = w[n, 128 * g:128 * (g + 1)]
            if s[n, g] == 0:
                continue
            assert np.abs(q[n, 128 * g:128 * (g + 1)]).max() == 7
            assert s[n, g] == np.float32(np.abs(blk).max()) / np.float32(7)
    d = dequantize_groups_int4(q, s)
    srep = np.repeat(s, 128, axis=1)
    assert np.all(np.abs(d - w) <= srep * 0.5 * (1 + 1e-6) + np.abs(w) * 2.0 ** -8 + 1e-30)
    # values on the grid come back exactly; half-way values round to even
    g = np.zeros((1, 128), dtype=np.float32)
    g[0, :6] = np.array([7.0, 3.0, -2.5, 2.5, 1.5, -7.0], dtype=np.float32) * np.float32(0.25)
    qg, sg = quantize_groups_int4(g)
    assert sg[0, 0] == np.float32(0.25) and list(qg[0, :6]) == [7, 3, -2, 2, 2, -7]
    assert np.array_equal(dequantize_groups_int4(qg, sg)[0, :6], np.array([1.75, 0.75, -0.5, 0.5, 0.5, -1.75],
                                                                          dtype=np.float32))


def test_int4_dequant_rounds_product_to_bf16():
    """A code times a scale that is not a bf16 value: the dequantized
    weight is the bf16 value nearest the float32 product (here 3 * s with
    s = 1 + 2^-9 + 2^-20: the float32 product 3.0059 lies between the bf16
    values 3 and 3 + 2^-6 and rounds to 3)."""
    from oracle.quant import dequantize_groups_int4
    s = np.array([[np.float32(1 + 2.0 ** -9 + 2.0 ** -20)]], dtype=np.float32)
    q = np.zeros((1, 128), dtype=np.int8)
    q[0, 0] = 3
    d = dequantize_groups_int4(q, s)
    assert d[0, 0] == np.float32(3.0)  # 3.0059 is nearer 3 than 3.015625
    q[0, 0] = 5  # 5 * s = 5.00977: bf16 neighbours 5.0 and 5.03125
    assert dequantize_groups_int4(q, s)[0, 0] == np.float32(5.0)
    q[0, 0] = -7  # -7.01367: neighbours -7.0 and -7.03125, nearer -7.0
    assert dequantize_groups_int4(q, s)[0, 0] == np.float32(-7.0)
    s2 = np.array([[np.float32(1 + 2.0 ** -7)]], dtype=np.float32)
    q[0, 0] = 3  # 3.0234375 exactly: halfway between 3.015625 and 3.03125, ties to even (3.03125)
    assert dequantize_groups_int4(q, s2)[0, 0] == np.float32(3.03125)


def test_int4_packing_layout():
    """Per 8 consecutive k, byte i holds k = i (low nibble) and k = i + 4
    (high nibble), codes offset by 8; worked bytes and a round trip."""
    from oracle.quant import pack_int4, unpack_int4
    q = np.array([[1, 2, 3, 4, 5, 6, 7, -7, 0, 0, 0, 0, -1, -2, -3, -4]], dtype=np.int8)
    p = pack_int4(q)
    assert list(p[0]) == [0xD9, 0xEA, 0xFB, 0x1C, 0x78, 0x68, 0x58, 0x48]
    rng = np.random.default_rng(3)
    r = rng.integers(-7, 8, (5, 256)).astype(np.int8)
    assert np.array_equal(unpack_int4(pack_int4(r)), r)


def test_int4_decode_weights_only_projections(tiny64):
    from oracle.quant import int4_decode_weights, PROJECTIONS
    cfg, W = tiny64[0], tiny64[1]
    Wq = int4_decode_weights(W, cfg.n_layers)
    for k, v in W.items():
        name = k.split(".", 1)[-1]
        if k.startswith("L") and name in PROJECTIONS:
            assert not np.array_equal(Wq[k], v)
            assert np.abs(Wq[k] - v).max() <= np.abs(v).max() * (1 / 14 + 2.0 ** -8) * 1.0001
        else:
            assert Wq[k] is v
