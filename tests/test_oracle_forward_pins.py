"""Model-level pins of the oracle's forward pass, and planted mistakes.

The pages name a forward pass that gives a next-token distribution at every
position ([en] Floor 3) but print no model equations, so the oracle's
Llama-style decoder is held to the mathematics instead: special cases of the
whole pass that reduce to textbook routines computed another way here --
rotate-half RoPE as multiplication by the complex numbers e^(i pos w_j),
scaled dot-product attention with scipy's softmax, SiLU through scipy's
expit -- with norm gains and query/key scales drawn at random so that a
gain on the wrong vector or a flat softmax cannot hide a mistake.

The last test plants plausible mistakes in copies of oracle/oracle.c (the
attention scale, RoPE on the wrong vector or position, the causal window,
the GQA head mapping, each residual, the SiLU operand, the RMSNorm epsilon
and gains, the LM head's input, ...) and checks that each mutant fails at
least one of the model pins (this file and test_oracle_model.py)."""
import concurrent.futures
import os
import subprocess
import sys

import numpy as np
import pytest
from scipy import special

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
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


# (pattern, replacement, occurrence) -- applied to a copy of oracle.c
_ROPE_Q = ("for (int32_t hh = 0; hh < H; hh++) rope_head(q + (size_t)r * qd + (size_t)hh * hd, hd, "
           "pos, m->rope_theta);")
_ROPE_K = ("for (int32_t hh = 0; hh < Hkv; hh++) rope_head(k + (size_t)r * kvd + (size_t)hh * hd, "
           "hd, pos, m->rope_theta);")
_RESID = "for (size_t i = 0; i < (size_t)n * d; i++) x[i] += y[i];"
MUTANTS = {
    "attention scale 1/hd": ("const double scale = 1.0 / sqrt((double)hd);",
                             "const double scale = 1.0 / (double)hd;", 0),
    "attention weights unnormalised": ("const double p = sc[t] / den;", "const double p = sc[t];", 0),
    "values read from the keys": ("const double* vt = vbase", "const double* vt = kbase", 0),
    "no RoPE on keys": (_ROPE_K, "", 0),
    "RoPE on values too": (_ROPE_K, _ROPE_K + _ROPE_K.replace("rope_head(k", "rope_head(v"), 0),
    "queries rotated one position late": (_ROPE_Q, _ROPE_Q.replace("hd, pos,", "hd, pos + 1,"), 0),
    "RoPE exponent -j/hd": ("pow(theta, -2.0 * (double)j / (double)hd)",
                            "pow(theta, -(double)j / (double)hd)", 0),
    "non-causal window": ("(size_t)Hkv * hd, pos + 1, hd,", "(size_t)Hkv * hd, pos0 + n, hd,", 0),
    "GQA head mapping hh % Hkv": ("const int32_t kh = (int32_t)(((int64_t)hh * Hkv) / H);",
                                  "const int32_t kh = hh % Hkv;", 0),
    "attention residual dropped": (_RESID, _RESID.replace("x[i] += y[i]", "x[i] = y[i]"), 0),
    "feed-forward residual dropped": (_RESID, _RESID.replace("x[i] += y[i]", "x[i] = y[i]"), 1),
    "SiLU on the up projection": ("g[i] = silu(g[i]) * u[i];", "g[i] = g[i] * silu(u[i]);", 0),
    "RMSNorm epsilon outside the root": ("double inv = 1.0 / sqrt(ss / (double)d + eps);",
                                         "double inv = 1.0 / (sqrt(ss / (double)d) + eps);", 0),
    "RMSNorm gain dropped": ("h[k] = x[k] * inv * bf16_to_f64(g[k]);", "h[k] = x[k] * inv;", 0),
    "final norm with the attention gains": ("rmsnorm_row(x + (size_t)r * d, d, m->final_norm,",
                                            "rmsnorm_row(x + (size_t)r * d, d, m->attn_norm,", 0),
    "LM head on the un-normed state": ("if (logits) matmul_rows(h, n, d, m->lm_head, V, logits);",
                                       "if (logits) matmul_rows(x, n, d, m->lm_head, V, logits);", 0),
}


def _mutate(src, pattern, repl, occurrence):
    parts = src.split(pattern)
    assert len(parts) > occurrence + 1, f"pattern not found (occurrence {occurrence}): {pattern}"
    return pattern.join(parts[:occurrence + 1]) + repl + pattern.join(parts[occurrence + 1:])


def _build_and_run(name, src, tmp):
    path = os.path.join(tmp, name.replace(" ", "_").replace("/", "_"))
    os.makedirs(path, exist_ok=True)
    c_file, so = os.path.join(path, "oracle.c"), os.path.join(path, "liboracle.so")
    with open(c_file, "w") as fh:
        fh.write(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-I", os.path.join(ROOT, "oracle"), c_file, "-o", so, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, SPEC_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", "not planted",
                        os.path.join(ROOT, "tests", "test_oracle_model.py"),
                        os.path.join(ROOT, "tests", "test_oracle_forward_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_planted_mistakes_fail_a_pin(tmp_path):
    with open(os.path.join(ROOT, "oracle", "oracle.c")) as fh:
        src = fh.read()
    mutants = {name: _mutate(src, *spec) for name, spec in MUTANTS.items()}
    assert all(m != src for m in mutants.values())
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_build_and_run, name, m, str(tmp_path)) for name, m in mutants.items()}
        rcs = {name: f.result() for name, f in futs.items()}
    survivors = [name for name, rc in rcs.items() if rc == 0]
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
    assert all(rc == 1 for rc in rcs.values()), rcs  # failed tests, not a crash or usage error
