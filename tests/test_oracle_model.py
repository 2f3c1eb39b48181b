"""Pins for the oracle's model forward.  The pages give no model equations,
so the forward is held to invariants and to special cases that reduce to
library routines (numpy matmul, scipy softmax/expit); the whole-pass special
cases and the planted mistakes are in test_oracle_forward_pins.py:
  - RoPE: identity at position 0, a rotation (norm-preserving, composes
    additively in position), scores depend only on relative position;
  - RMSNorm: closed form on constant vectors, scale invariance;
  - attention: one key returns its value, equal keys average the values;
  - causality, row invariance (batch == one row at a time, bit-exact),
    GQA head mapping == explicit MHA with duplicated K/V heads (bit-exact);
  - the residual paths with other blocks zeroed, against numpy / scipy."""
import numpy as np
import pytest
from scipy import special

import oracle
import synth


# ------------------------------------------------------------------ RoPE --
def test_rope_identity_at_zero():
    v = np.random.default_rng(0).standard_normal(16)
    assert np.array_equal(oracle.rope(v, 0, 10000.0), v)


def test_rope_is_rotation_and_composes():
    rng = np.random.default_rng(1)
    hd = 32
    v = rng.standard_normal(hd)
    for a, b in ((3, 5), (100, 27), (1000, 1)):
        ra = oracle.rope(v, a, 500000.0)
        # norm of every (j, j+hd/2) pair is preserved
        h = hd // 2
        np.testing.assert_allclose(ra[:h] ** 2 + ra[h:] ** 2, v[:h] ** 2 + v[h:] ** 2, rtol=1e-12)
        # rotating by a then b equals rotating by a+b
        np.testing.assert_allclose(oracle.rope(ra, b, 500000.0), oracle.rope(v, a + b, 500000.0),
                                   atol=1e-9)


def test_rope_angle_schedule_closed_form():
    """The frequencies themselves.  hd = 4, theta = 1e4: pair j = 0 holds dims
    (0, 2) and turns by pos * 1e4^0 = pos rad, pair j = 1 holds dims (1, 3)
    and turns by pos * 1e4^(-2/4) = pos / 100 rad.  A basis vector e_j goes
    to cos(a) e_j + sin(a) e_{j+2} (rotate-half: x_j' = x_j cos - x_{j+2} sin,
    x_{j+2}' = x_{j+2} cos + x_j sin).  A wrong exponent (theta^(-j/hd),
    theta^(-2j/(hd-2))) or a wrong pairing (j with j+1) moves these values."""
    for pos in (1, 7):
        for j, ang in ((0, float(pos)), (1, pos / 100.0)):
            e = np.zeros(4)
            e[j] = 1.0
            want = np.zeros(4)
            want[j], want[j + 2] = np.cos(ang), np.sin(ang)
            np.testing.assert_allclose(oracle.rope(e, pos, 1e4), want, atol=1e-15)
            e2 = np.zeros(4)
            e2[j + 2] = 1.0
            want2 = np.zeros(4)
            want2[j], want2[j + 2] = -np.sin(ang), np.cos(ang)
            np.testing.assert_allclose(oracle.rope(e2, pos, 1e4), want2, atol=1e-15)


def test_rope_angle_schedule_8b_head():
    """One 8B-shaped head (hd = 128, theta = 5e5) at position 1000 on a random
    vector, against math.cos / math.sin of pos * theta^(-2j/hd) written out
    per pair (j, j + 64)."""
    import math
    hd, theta, pos = 128, 5e5, 1000
    v = np.random.default_rng(4).standard_normal(hd)
    got = oracle.rope(v, pos, theta)
    h = hd // 2
    for j in range(h):
        a = pos * theta ** (-2.0 * j / hd)
        c, s = math.cos(a), math.sin(a)
        assert abs(got[j] - (v[j] * c - v[j + h] * s)) < 1e-12
        assert abs(got[j + h] - (v[j + h] * c + v[j] * s)) < 1e-12


def test_rope_scores_depend_on_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    s = [oracle.rope(q, a + t, 10000.0) @ oracle.rope(k, b + t, 10000.0)
         for a, b in ((7, 3),) for t in (0, 11, 250)]
    np.testing.assert_allclose(s, s[0], rtol=1e-9)


# --------------------------------------------------------------- RMSNorm --
def test_rmsnorm_constant_vector_closed_form():
    d, c, eps = 64, 0.37, 1e-5
    g = np.full(d, synth.ONE_BF16, np.uint16)
    h = oracle.rmsnorm(np.full(d, c), g, eps)
    np.testing.assert_allclose(h, c / np.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm_scale_invariant_and_unit_rms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(128)
    g = np.full(128, synth.ONE_BF16, np.uint16)
    h1 = oracle.rmsnorm(x, g, 0.0)
    h2 = oracle.rmsnorm(x * 123.0, g, 0.0)
    np.testing.assert_allclose(h1, h2, rtol=1e-13)
    assert abs(np.sqrt(np.mean(h1 ** 2)) - 1.0) < 1e-13
    # gains multiply elementwise
    gb = synth.f32_to_bf16_bits(np.linspace(0.5, 2.0, 128).astype(np.float32))
    np.testing.assert_allclose(oracle.rmsnorm(x, gb, 0.0), h1 * synth.bf16_bits_to_f32(gb), rtol=1e-13)


# ------------------------------------------------------------- attention --
def test_attention_single_key_returns_value():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal(16), rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    assert np.array_equal(oracle.attend(q, k, v), v[0])


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(5)
    q = rng.standard_normal(8)
    k = np.tile(rng.standard_normal(8), (5, 1))
    v = rng.standard_normal((5, 8))
    np.testing.assert_allclose(oracle.attend(q, k, v), v.mean(0), rtol=1e-13)


def test_attention_matches_scipy_softmax_weights():
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal(16), rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    p = special.softmax(k @ q / 4.0)
    np.testing.assert_allclose(oracle.attend(q, k, v), p @ v, rtol=1e-12)


def test_softmax_f32_matches_scipy():
    rng = np.random.default_rng(7)
    z = rng.standard_normal(1000) * 3
    np.testing.assert_allclose(oracle.softmax_f32(z), special.softmax(z).astype(np.float32),
                               rtol=2e-7, atol=1e-12)


# ------------------------------------------------------------ model level --
CFG = synth.ModelConfig("pin-2L", 2, 64, 4, 2, 16, 96, 40)


def make(cfg=CFG, **zero):
    w = synth.weights_np(cfg, seed=77)
    for k in zero:
        w[k] = np.zeros_like(w[k])
    return oracle.Model(cfg, w), w


def test_row_invariance_batch_equals_one_at_a_time():
    m, _ = make()
    toks = synth.prompt(CFG.vocab, 12, seed=3)
    kv = oracle.KV(m, 32)
    full = oracle.forward(m, kv, toks, 0)
    kv2 = oracle.KV(m, 32)
    rows = [oracle.forward(m, kv2, toks[i:i + 1], i)[0] for i in range(12)]
    assert np.array_equal(full, np.stack(rows))
    # prefill + chunked continuation also agrees bit for bit
    kv3 = oracle.KV(m, 32)
    a = oracle.forward(m, kv3, toks[:5], 0)
    b = oracle.forward(m, kv3, toks[5:], 5)
    assert np.array_equal(full, np.concatenate([a, b]))


def test_causality():
    m, _ = make()
    toks = synth.prompt(CFG.vocab, 10, seed=4)
    alt = toks.copy()
    alt[7:] = (alt[7:] + 1) % CFG.vocab
    a = oracle.forward(m, oracle.KV(m, 16), toks, 0)
    b = oracle.forward(m, oracle.KV(m, 16), alt, 0)
    assert np.array_equal(a[:7], b[:7])
    assert not np.array_equal(a[7:], b[7:])


def test_gqa_equals_mha_with_duplicated_kv_heads():
    cfg = CFG
    m, w = make(cfg)
    g = cfg.n_heads // cfg.n_kv_heads
    hd = cfg.head_dim
    mha = cfg.replace(name="pin-2L-mha", n_kv_heads=cfg.n_heads)
    w2 = dict(w)
    for k in ("wk", "wv"):
        t = w[k].reshape(cfg.n_layers, cfg.n_kv_heads, hd, cfg.d_model)
        w2[k] = np.repeat(t, g, axis=1).reshape(cfg.n_layers, cfg.n_heads * hd, cfg.d_model)
    m2 = oracle.Model(mha, w2)
    toks = synth.prompt(cfg.vocab, 9, seed=5)
    a = oracle.forward(m, oracle.KV(m, 16), toks, 0)
    b = oracle.forward(m2, oracle.KV(m2, 16), toks, 0)
    assert np.array_equal(a, b)


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _norm(x, g, eps):
    return x / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps) * _f(g)


def test_zero_blocks_reduce_to_norm_and_head():
    """Wo = Wd = 0: the residual stream stays the embedding; logits are the
    final-normed embedding times the LM head (numpy matmul)."""
    m, w = make(wo=True, wd=True)
    toks = synth.prompt(CFG.vocab, 6, seed=6)
    got = oracle.forward(m, oracle.KV(m, 8), toks, 0)
    x = _f(w["embed"])[toks]
    want = _norm(x, w["final_norm"], CFG.rms_eps) @ _f(w["lm_head"]).T
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)


def test_single_token_attention_path():
    """One token at position 0 sees only itself: attention returns its value
    vector, so the block adds (RMSNorm(x) Wv^T, expanded per GQA group) Wo^T.
    FFN zeroed (Wd = 0); one layer."""
    cfg = CFG.replace(name="pin-1L", n_layers=1)
    w = synth.weights_np(cfg, seed=78)
    w["wd"] = np.zeros_like(w["wd"])
    m = oracle.Model(cfg, w)
    tok = np.array([11], np.int32)
    got = oracle.forward(m, oracle.KV(m, 4), tok, 0)
    x = _f(w["embed"])[tok]
    h = _norm(x, w["attn_norm"][0], cfg.rms_eps)
    v = (h @ _f(w["wv"][0]).T).reshape(1, cfg.n_kv_heads, cfg.head_dim)
    o = np.repeat(v, cfg.n_heads // cfg.n_kv_heads, axis=1).reshape(1, -1)
    x1 = x + o @ _f(w["wo"][0]).T
    want = _norm(x1, w["final_norm"], cfg.rms_eps) @ _f(w["lm_head"]).T
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_ffn_path_swiglu():
    """Wo = 0: each layer adds (silu(h Wg^T) * (h Wu^T)) Wd^T with
    silu(x) = x * expit(x) (scipy)."""
    m, w = make(wo=True)
    toks = synth.prompt(CFG.vocab, 5, seed=8)
    got = oracle.forward(m, oracle.KV(m, 8), toks, 0)
    x = _f(w["embed"])[toks]
    for l in range(CFG.n_layers):
        h = _norm(x, w["ffn_norm"][l], CFG.rms_eps)
        g = h @ _f(w["wg"][l]).T
        u = h @ _f(w["wu"][l]).T
        x = x + (g * special.expit(g) * u) @ _f(w["wd"][l]).T
    want = _norm(x, w["final_norm"], CFG.rms_eps) @ _f(w["lm_head"]).T
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
