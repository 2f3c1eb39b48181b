"""Model-level pins of the oracle's forward pass.

The pages name a forward pass that gives a next-token distribution at every
position ([en] Floor 3) but print no model equations, so the oracle's
Llama-style decoder is held to the mathematics instead: special cases of the
whole pass that reduce to textbook routines computed another way here --
rotate-half RoPE as multiplication by the complex numbers e^(i pos w_j),
scaled dot-product attention with scipy's softmax, SiLU through scipy's
expit -- with norm gains and query/key scales drawn at random so that a
gain on the wrong vector or a flat softmax cannot hide a mistake.

test_oracle_planted_mistakes.py plants plausible mistakes in copies of the
oracle and checks that each fails one of these pins or those of
test_oracle_model.py."""
import numpy as np
import pytest
from scipy import special

import oracle
import synth

CFG1 = synth.ModelConfig("fwd-pin-1L", 1, 64, 4, 2, 16, 96, 40, rope_theta=10000.0)
CFG2 = synth.ModelConfig("fwd-pin-2L", 2, 64, 4, 2, 16, 96, 40, rope_theta=500.0)


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _weights(cfg, seed, zero=()):
    """Seeded weights with random norm gains in [0.5, 1.5) and query/key
    projections scaled up (bf16 rounded again) so attention is far from
    uniform."""
    w = synth.weights_np(cfg, seed=seed)
    rng = np.random.default_rng(seed + 1)
    for k in ("attn_norm", "ffn_norm", "final_norm"):
        w[k] = synth.f32_to_bf16_bits((0.5 + rng.random(w[k].shape)).astype(np.float32))
    for k in ("wq", "wk"):
        w[k] = synth.f32_to_bf16_bits((synth.bf16_bits_to_f32(w[k]) * np.float32(12.0)))
    for k in zero:
        w[k] = np.zeros_like(w[k])
    return w


def _norm(x, g, eps):
    return x / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps) * _f(g)


def _rope_complex(x, pos, theta):
    """Rotate-half RoPE written as complex multiplication: dims j and
    j + hd/2 are the real and imaginary parts of z_j, turned by
    e^(i pos theta^(-2j/hd))."""
    hd = x.shape[-1]
    half = hd // 2
    z = x[..., :half] + 1j * x[..., half:]
    z = z * np.exp(1j * pos * theta ** (-2.0 * np.arange(half) / hd))
    return np.concatenate([z.real, z.imag], -1)


def _forward_numpy(cfg, w, toks, attn=True, ffn=True):
    """Logits of a context that starts at position 0."""
    n, H, Hkv, hd = len(toks), cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    G = H // Hkv
    pos = np.arange(n, dtype=np.float64)[:, None, None]
    causal = np.tril(np.ones((n, n), bool))
    x = _f(w["embed"])[toks]
    for l in range(cfg.n_layers):
        if attn:
            h = _norm(x, w["attn_norm"][l], cfg.rms_eps)
            q = _rope_complex((h @ _f(w["wq"][l]).T).reshape(n, H, hd), pos, cfg.rope_theta)
            k = _rope_complex((h @ _f(w["wk"][l]).T).reshape(n, Hkv, hd), pos, cfg.rope_theta)
            v = (h @ _f(w["wv"][l]).T).reshape(n, Hkv, hd)
            o = np.empty((n, H, hd))
            for hh in range(H):
                s = q[:, hh] @ k[:, hh // G].T / np.sqrt(hd)
                p = special.softmax(np.where(causal, s, -np.inf), axis=-1)
                o[:, hh] = p @ v[:, hh // G]
            x = x + o.reshape(n, H * hd) @ _f(w["wo"][l]).T
        if ffn:
            h = _norm(x, w["ffn_norm"][l], cfg.rms_eps)
            g = h @ _f(w["wg"][l]).T
            u = h @ _f(w["wu"][l]).T
            x = x + (g * special.expit(g) * u) @ _f(w["wd"][l]).T
    return _norm(x, w["final_norm"], cfg.rms_eps) @ _f(w["lm_head"]).T


def test_attention_block_rope_gqa():
    """One layer with the feed-forward output zeroed: causal GQA attention of
    five tokens with RoPE, against the complex-rotation reference."""
    w = _weights(CFG1, 90, zero=("wd",))
    m = oracle.Model(CFG1, w)
    toks = synth.prompt(CFG1.vocab, 5, seed=31)
    got = oracle.forward(m, oracle.KV(m, 8), toks, 0)
    want = _forward_numpy(CFG1, w, toks, ffn=False)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-11)


def test_two_full_layers():
    """Two layers with both blocks live (each block's input includes the
    previous block's residual update), seven tokens."""
    w = _weights(CFG2, 91)
    m = oracle.Model(CFG2, w)
    toks = synth.prompt(CFG2.vocab, 7, seed=32)
    got = oracle.forward(m, oracle.KV(m, 8), toks, 0)
    want = _forward_numpy(CFG2, w, toks)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-11)


def test_attention_is_not_flat():
    """The scaled-up query/key projections make the attention weights of the
    pins above far from uniform, so the scale and RoPE matter to them."""
    w = _weights(CFG1, 90, zero=("wd",))
    toks = synth.prompt(CFG1.vocab, 5, seed=31)
    flat = _forward_numpy(CFG1, dict(w, wq=np.zeros_like(w["wq"])), toks, ffn=False)
    assert np.abs(_forward_numpy(CFG1, w, toks, ffn=False) - flat).max() > 1e-3
