"""Pins of the oracle's two mixer layers as composed wholes.

The full-attention layer and the Gated-DeltaNet layer of the oracle
(``oracle.attention.full_attention``, ``oracle.gdn.gdn_layer``) are composed
from parts that are pinned one by one elsewhere.  Here each composition is
written out a second time as a scalar, loop-by-loop evaluation in float64 on
tiny shapes -- plain Python over lists, no array library, straight from the
layer's definition:

* full attention ([P1] hncyxsy.com/news/268323 section 3: GQA, QK-norm, output
  gate, rotary on a quarter of the head dims; [P1] section 4: the cache holds
  post-norm, post-rotary K and raw V): fused projection rows [q; g; k; v],
  RMSNorm over each head's D dims with one gain for q and one for k, rotary of
  the adjacent pairs (2i, 2i+1) for i < R/2 at angle pos * base^(-2i/R), causal
  softmax(q.k / sqrt(D)) V with query head j reading KV head j // (Hq/Hkv),
  elementwise sigmoid gate of g on the attention output, then W_o;
* Gated-DeltaNet ([P1] section 3: gate + delta rule, constant-size state; the
  gated delta rule of Yang et al., ICLR 2025): fused rows [q; k; v; z; a; b],
  q and k divided by their L2 norms (eps), q by sqrt(Dk), alpha =
  exp(-softplus(a)), beta = sigmoid(b), S <- alpha S (I - beta k k^T) +
  beta v k^T with the matrix I - beta k k^T formed explicitly, o = S q, then
  RMSNorm over Dv of o with its gain, times SiLU(z), then W_o.

Each pin runs two calls (the second continues the first's cache / state) and
must agree with the oracle to 1e-12.  Planted mistakes -- each a copy of the
oracle's composition with one plausible error -- must disagree with the scalar
evaluation, so the pin is shown to see them.
"""
import math

import numpy as np
import pytest

from oracle import attention, gdn
from oracle.config import Config
from oracle.ops import rmsnorm, apply_rope, sigmoid, silu, softplus
from oracle.precision import round_bf16

F64 = np.float64

# tiny shapes; d == Hq * D so that a gate misplaced after W_o is expressible
CFG = Config(n_layers=4, loop_start=0, loop_end=0, loop_passes=1, d_model=16, d_ff=32, vocab=0,
             n_q_heads=2, n_kv_heads=1, head_dim=8, rotary_dim=4,
             gdn_heads=2, gdn_dk=4, gdn_dv=6, eps=1e-6, rope_theta=10000.0)


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def _attn_weights(rng, cfg=CFG):
    Hq, Hkv, D, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_model
    return {"w_in": _rand(rng, 2 * Hq * D + 2 * Hkv * D, d, s=0.4),
            "w_o": _rand(rng, d, Hq * D, s=0.3),
            # gains far from 1 so that their order against rotary matters
            "q_norm": 1.0 + _rand(rng, D, s=0.5), "k_norm": 1.0 + _rand(rng, D, s=0.5)}


def _gdn_weights(rng, cfg=CFG):
    H, Dk, Dv, d = cfg.gdn_heads, cfg.gdn_dk, cfg.gdn_dv, cfg.d_model
    return {"w_in": _rand(rng, 2 * H * Dk + 2 * H * Dv + 2 * H, d, s=0.4),
            "w_o": _rand(rng, d, H * Dv, s=0.3), "o_norm": 1.0 + _rand(rng, Dv, s=0.5)}


# ------------------------------------------------------------- scalar helpers

def _matvec(W, x):
    return [sum(W[r][c] * x[c] for c in range(len(x))) for r in range(len(W))]


def _rms_scaled(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    inv = 1.0 / math.sqrt(ms + eps)
    return [x[i] * inv * g[i] for i in range(len(x))]


def _sig(x):
    return 1.0 / (1.0 + math.exp(-x))


# ------------------------------------------------------- scalar full attention

class ScalarAttention:
    """One full-attention layer for one sequence, token by token."""

    def __init__(self, w, cfg=CFG):
        self.w = {k: np.asarray(v).tolist() for k, v in w.items()}
        self.cfg = cfg
        self.K = []   # per position: [Hkv][D] post-norm, post-rotary
        self.V = []   # per position: [Hkv][D]

    def rotate(self, x, pos):
        c = self.cfg
        y = list(x)
        for i in range(c.rotary_dim // 2):
            ang = pos * c.rope_theta ** (-2.0 * i / c.rotary_dim)
            co, si = math.cos(ang), math.sin(ang)
            a, b = x[2 * i], x[2 * i + 1]
            y[2 * i] = a * co - b * si
            y[2 * i + 1] = a * si + b * co
        return y

    def step(self, xn_row, pos):
        c, w = self.cfg, self.w
        Hq, Hkv, D = c.n_q_heads, c.n_kv_heads, c.head_dim
        p = _matvec(w["w_in"], xn_row)
        q = [p[j * D:(j + 1) * D] for j in range(Hq)]
        g = p[Hq * D:2 * Hq * D]
        k = [p[2 * Hq * D + h * D:2 * Hq * D + (h + 1) * D] for h in range(Hkv)]
        v = [p[2 * Hq * D + Hkv * D + h * D:2 * Hq * D + Hkv * D + (h + 1) * D] for h in range(Hkv)]
        q = [self.rotate(_rms_scaled(qj, w["q_norm"], c.eps), pos) for qj in q]
        k = [self.rotate(_rms_scaled(kh, w["k_norm"], c.eps), pos) for kh in k]
        assert len(self.K) == pos
        self.K.append(k)
        self.V.append(v)
        out = []
        for j in range(Hq):
            kv = j // (Hq // Hkv)
            s = [sum(q[j][e] * self.K[u][kv][e] for e in range(D)) / math.sqrt(D) for u in range(pos + 1)]
            m = max(s)
            ex = [math.exp(x - m) for x in s]
            z = sum(ex)
            for e in range(D):
                out.append(sum(ex[u] * self.V[u][kv][e] for u in range(pos + 1)) / z)
        gated = [out[i] * _sig(g[i]) for i in range(Hq * D)]
        return _matvec(w["w_o"], gated)


# -------------------------------------------------------------- scalar GDN

class ScalarGDN:
    """One Gated-DeltaNet layer for one sequence, token by token."""

    def __init__(self, w, cfg=CFG):
        self.w = {k: np.asarray(v).tolist() for k, v in w.items()}
        self.cfg = cfg
        H, Dk, Dv = cfg.gdn_heads, cfg.gdn_dk, cfg.gdn_dv
        self.S = [[[0.0] * Dk for _ in range(Dv)] for _ in range(H)]

    def step(self, xn_row):
        c, w = self.cfg, self.w
        H, Dk, Dv = c.gdn_heads, c.gdn_dk, c.gdn_dv
        p = _matvec(w["w_in"], xn_row)
        off = 0
        q = [p[off + h * Dk:off + (h + 1) * Dk] for h in range(H)]; off += H * Dk
        k = [p[off + h * Dk:off + (h + 1) * Dk] for h in range(H)]; off += H * Dk
        v = [p[off + h * Dv:off + (h + 1) * Dv] for h in range(H)]; off += H * Dv
        z = [p[off + h * Dv:off + (h + 1) * Dv] for h in range(H)]; off += H * Dv
        a = p[off:off + H]; off += H
        b = p[off:off + H]
        out = []
        for h in range(H):
            nq = math.sqrt(sum(x * x for x in q[h]) + c.eps)
            nk = math.sqrt(sum(x * x for x in k[h]) + c.eps)
            qh = [x / nq / math.sqrt(Dk) for x in q[h]]
            kh = [x / nk for x in k[h]]
            alpha = math.exp(-math.log1p(math.exp(a[h])))
            beta = _sig(b[h])
            # M = I - beta k k^T, then S <- alpha S M + beta v k^T
            M = [[(1.0 if i == j else 0.0) - beta * kh[i] * kh[j] for j in range(Dk)] for i in range(Dk)]
            S = self.S[h]
            SM = [[sum(S[r][l] * M[l][j] for l in range(Dk)) for j in range(Dk)] for r in range(Dv)]
            S = [[alpha * SM[r][j] + beta * v[h][r] * kh[j] for j in range(Dk)] for r in range(Dv)]
            self.S[h] = S
            o = [sum(S[r][j] * qh[j] for j in range(Dk)) for r in range(Dv)]
            y = _rms_scaled(o, w["o_norm"], c.eps)
            out += [y[r] * z[h][r] * _sig(z[h][r]) for r in range(Dv)]
        return _matvec(w["w_o"], out)


def _rel(a, b):
    a, b = np.asarray(a, F64), np.asarray(b, F64)
    return float(np.abs(a - b).max() / np.abs(b).max())


# ----------------------------------------------------------- full attention

def _attn_oracle(xn_parts, w, layer=attention.full_attention):
    cache = attention.KVCache(CFG.n_kv_heads, CFG.head_dim, F64)
    out, pos = [], 0
    for xn in xn_parts:
        out.append(layer(xn, w, cache, pos, CFG))
        pos += xn.shape[0]
    return np.concatenate(out), cache


def _attn_scalar(xn_parts, w):
    sa = ScalarAttention(w)
    rows, pos = [], 0
    for xn in xn_parts:
        for t in range(xn.shape[0]):
            rows.append(sa.step(xn[t].tolist(), pos))
            pos += 1
    return np.array(rows), sa


def _parts(rng, lens, d=CFG.d_model):
    return [rng.standard_normal((n, d)) for n in lens]


def test_full_attention_layer_scalar():
    rng = np.random.default_rng(101)
    w = _attn_weights(rng)
    xs = _parts(rng, [5, 3])
    got, cache = _attn_oracle(xs, w)
    ref, sa = _attn_scalar(xs, w)
    assert _rel(got, ref) < 1e-12
    # the cache holds post-norm, post-rotary K and raw V
    assert np.abs(cache.k.transpose(1, 0, 2) - np.array(sa.K)).max() < 1e-12
    assert np.abs(cache.v.transpose(1, 0, 2) - np.array(sa.V)).max() < 1e-12


def _mutant_attention(kind):
    """A copy of the oracle's full-attention composition with one mistake."""
    def layer(xn, w, cache, pos0, cfg):
        T = xn.shape[0]
        Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        proj = xn @ w["w_in"].T
        if kind == "slice_order":   # rows read as [q; k; v; g]
            q = proj[:, :Hq * D]
            k = proj[:, Hq * D:Hq * D + Hkv * D]
            v = proj[:, Hq * D + Hkv * D:Hq * D + 2 * Hkv * D]
            g = proj[:, Hq * D + 2 * Hkv * D:]
        else:
            q = proj[:, :Hq * D]
            g = proj[:, Hq * D:2 * Hq * D]
            k = proj[:, 2 * Hq * D:2 * Hq * D + Hkv * D]
            v = proj[:, 2 * Hq * D + Hkv * D:]
        q, k, v = q.reshape(T, Hq, D), k.reshape(T, Hkv, D), v.reshape(T, Hkv, D)
        pos = np.arange(pos0, pos0 + T)
        if kind == "rope_before_norm":
            q = rmsnorm(apply_rope(q, pos, cfg.rotary_dim, cfg.rope_theta), w["q_norm"], cfg.eps)
            k = rmsnorm(apply_rope(k, pos, cfg.rotary_dim, cfg.rope_theta), w["k_norm"], cfg.eps)
        else:
            q = apply_rope(rmsnorm(q, w["q_norm"], cfg.eps), pos, cfg.rotary_dim, cfg.rope_theta)
            k = apply_rope(rmsnorm(k, w["k_norm"], cfg.eps), pos, cfg.rotary_dim, cfg.rope_theta)
        cache.append(k, v)
        o = attention.attention_core(q, cache.k, cache.v, pos).reshape(T, Hq * D)
        if kind == "gate_after_wo":
            return (o @ w["w_o"].T) * sigmoid(g)
        if kind == "no_sigmoid":
            return (o * g) @ w["w_o"].T
        return (o * sigmoid(g)) @ w["w_o"].T
    return layer


@pytest.mark.parametrize("kind", ["gate_after_wo", "no_sigmoid", "rope_before_norm", "slice_order"])
def test_full_attention_planted_mistakes_caught(kind):
    rng = np.random.default_rng(102)
    w = _attn_weights(rng)
    xs = _parts(rng, [5, 3])
    ref, _ = _attn_scalar(xs, w)
    good, _ = _attn_oracle(xs, w, _mutant_attention("none"))
    assert _rel(good, ref) < 1e-12          # the unmutated copy is the layer
    bad, _ = _attn_oracle(xs, w, _mutant_attention(kind))
    assert _rel(bad, ref) > 1e-3, kind


# ----------------------------------------------------------------------- GDN

def _gdn_oracle(xn_parts, w, layer=gdn.gdn_layer, **kw):
    S = np.zeros((CFG.gdn_heads, CFG.gdn_dv, CFG.gdn_dk))
    out = []
    for xn in xn_parts:
        a, S = layer(xn, w, S, CFG, **kw)
        out.append(a)
    return np.concatenate(out), S


def _gdn_scalar(xn_parts, w):
    sg = ScalarGDN(w)
    rows = [sg.step(xn[t].tolist()) for xn in xn_parts for t in range(xn.shape[0])]
    return np.array(rows), np.array(sg.S)


@pytest.mark.parametrize("chunked", [False, True])
def test_gdn_layer_scalar(chunked):
    rng = np.random.default_rng(103)
    w = _gdn_weights(rng)
    xs = _parts(rng, [7, 4])
    got, S = _gdn_oracle(xs, w, chunked=chunked, chunk=4)
    ref, Sref = _gdn_scalar(xs, w)
    assert _rel(got, ref) < 1e-12
    assert np.abs(S - Sref).max() < 1e-12


def _mutant_gdn(kind):
    """A copy of the oracle's Gated-DeltaNet composition with one mistake."""
    def layer(xn, w, S0, cfg):
        T = xn.shape[0]
        H, Dk, Dv = cfg.gdn_heads, cfg.gdn_dk, cfg.gdn_dv
        proj = xn @ w["w_in"].T
        o0 = 0
        q = proj[:, o0:o0 + H * Dk].reshape(T, H, Dk); o0 += H * Dk
        k = proj[:, o0:o0 + H * Dk].reshape(T, H, Dk); o0 += H * Dk
        v = proj[:, o0:o0 + H * Dv].reshape(T, H, Dv); o0 += H * Dv
        z = proj[:, o0:o0 + H * Dv].reshape(T, H, Dv); o0 += H * Dv
        a = proj[:, o0:o0 + H]; o0 += H
        b = proj[:, o0:o0 + H]
        qh = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + cfg.eps)
        if kind != "no_q_scale":
            qh = qh / np.sqrt(Dk)
        kh = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + cfg.eps)
        log_alpha = -softplus(-a) if kind == "softplus_sign" else -softplus(a)
        o, S = gdn.gdn_recurrent(qh, kh, v, np.exp(log_alpha), sigmoid(b), S0)
        if kind == "norm_after_gate":
            y = rmsnorm(o * silu(z), w["o_norm"], cfg.eps)
        else:
            y = rmsnorm(o, w["o_norm"], cfg.eps) * silu(z)
        return y.reshape(T, H * Dv) @ w["w_o"].T, S
    return layer


@pytest.mark.parametrize("kind", ["no_q_scale", "softplus_sign", "norm_after_gate"])
def test_gdn_planted_mistakes_caught(kind):
    rng = np.random.default_rng(104)
    w = _gdn_weights(rng)
    xs = _parts(rng, [7, 4])
    ref, _ = _gdn_scalar(xs, w)
    good, _ = _gdn_oracle(xs, w, _mutant_gdn("none"))
    assert _rel(good, ref) < 1e-12
    bad, _ = _gdn_oracle(xs, w, _mutant_gdn(kind))
    # The output RMSNorm over Dv makes the layer nearly invariant to a
    # constant scale of q (o = S q scales with it): a dropped 1/sqrt(Dk)
    # shows only through the norm's eps, ~1e-4 here -- still 1e8 times the
    # pin's 1e-12 agreement.
    assert _rel(bad, ref) > (1e-6 if kind == "no_q_scale" else 1e-3), kind


# ---------------------------------------- the mixers on a given projection

def test_mixers_on_projection_equal_layers():
    """attention_mixer / gdn_mixer (the part between the two projections) are
    the layers with the projections taken off: layer = mixer(xn W_in^T) W_o^T."""
    rng = np.random.default_rng(105)
    wa, wg = _attn_weights(rng), _gdn_weights(rng)
    xn = rng.standard_normal((6, CFG.d_model))
    c1 = attention.KVCache(CFG.n_kv_heads, CFG.head_dim, F64)
    c2 = attention.KVCache(CFG.n_kv_heads, CFG.head_dim, F64)
    a1 = attention.full_attention(xn, wa, c1, 0, CFG)
    m2 = attention.attention_mixer(xn @ wa["w_in"].T, wa, c2, 0, CFG)
    assert np.array_equal(a1, m2 @ wa["w_o"].T)
    S0 = np.zeros((CFG.gdn_heads, CFG.gdn_dv, CFG.gdn_dk))
    g1, S1 = gdn.gdn_layer(xn, wg, S0, CFG)
    m3, S3 = gdn.gdn_mixer(xn @ wg["w_in"].T, wg, S0, CFG)
    assert np.array_equal(g1, m3 @ wg["w_o"].T) and np.array_equal(S1, S3)


# ------------------------------------------- bf16 branch of attention_core

def test_attention_core_bf16_branch_scalar():
    """The precision policy's attention: the unnormalised probabilities
    exp(s - max) that multiply V are bf16 values, the normaliser is their
    full-precision sum.  Scalar evaluation, causal with a cache offset."""
    rng = np.random.default_rng(106)
    T, Hq, Hkv, D, L = 3, 4, 2, 8, 7
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    K = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    V = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    qpos = np.array([4, 5, 6])
    got = attention.attention_core(q, K, V, qpos, bf16=True)
    for t in range(T):
        for j in range(Hq):
            kv = j // (Hq // Hkv)
            s = [float(np.dot(q[t, j].astype(F64), K[kv, u].astype(F64))) / math.sqrt(D)
                 for u in range(qpos[t] + 1)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            pb = [float(round_bf16(np.array([x], np.float32))[0]) for x in e]
            for dd in range(D):
                ref = sum(pb[u] * float(V[kv, u, dd]) for u in range(len(e))) / sum(e)
                assert abs(float(got[t, j, dd]) - ref) <= 1e-5 * (1 + abs(ref))
    # against the unrounded definition: within the bf16 unit roundoff of the
    # largest term (each probability moves by at most 2^-9 relative)
    plain = attention.attention_core(q.astype(F64), K.astype(F64), V.astype(F64), qpos)
    assert np.abs(got - plain).max() <= 2 ** -8 * np.abs(V).max()
    # and it is not the plain definition (the rounding is really applied)
    assert np.abs(got - plain).max() > 1e-6
